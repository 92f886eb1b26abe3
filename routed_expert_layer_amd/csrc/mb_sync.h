// Cross-workgroup communication inside one persistent launch on gfx950.
//
// Each XCD of an MI355X has its own L2, and the L2s are not coherent with one
// another.  A device-scope release/acquire fence makes them so by writing back
// and invalidating the whole L2, which costs microseconds per wave.  Instead,
// data that one workgroup hands to another within a launch is written and
// read with the sc1 cache-policy bit (device-scope coherent: written through
// to memory, read past the local L2) by 16-, 8- and 4-byte buffer accesses,
// and the only ordering needed is that a workgroup's coherent stores have
// completed (s_waitcnt vmcnt(0) in every wave) before it signals arrival.
//
// Dependency counters are incremented once per producing task after its
// coherent stores completed, and polled (bounded) by consumers; block.hip
// describes the counter sets and their per-launch epochs.
#pragma once

#include "mb_device.h"

typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kCoherent = 16;  // sc1

__device__ __forceinline__ rsrc_t make_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7FFFFFFF, 0x00020000);
}

__device__ __forceinline__ u32x4_t ld_co16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}
__device__ __forceinline__ u32x2_t ld_co8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent));
}
__device__ __forceinline__ uint32_t ld_co4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent);
}
__device__ __forceinline__ void st_co16(rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(
      __attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ void st_co8(rsrc_t r, uint32_t off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(
      __attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ void st_co4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kCoherent);
}

// Streaming (non-temporal) buffer loads of weights.  An offset at or above
// kOob lies outside every resource made by make_rsrc: the load reads no
// memory and returns zeros (buffer range checking), which lets loops issue
// padding loads without branches.
constexpr int kNonTemporal = 2;  // nt
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ u32x4_t ld_nt16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}
// Plain (cached) buffer loads of data no other workgroup writes in the launch.
__device__ __forceinline__ u32x4_t ld_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2_t ld_b64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t ld_b8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

constexpr unsigned kSpinLimit = 1u << 21;  // polls before a wait gives up
