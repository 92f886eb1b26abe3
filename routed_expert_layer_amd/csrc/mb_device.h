// Device helpers shared by the gfx950 kernels of libmb.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

#define MB_WAVE 64

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even (the __bf16 conversion is RNE).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// E8M0 scale byte -> the fp32 whose exponent field is that byte (2^(s-127)
// for 1 <= s <= 254), the form the scaled fp4 converts take.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s << 23);
}

// 16 packed E2M1 bytes (32 codes, element 2m in the low nibble of byte m)
// times one block scale -> four groups of 8 bf16 (group d = elements
// 8d..8d+7).  The bf16 results are exact: an E2M1 value times a power of two
// within bf16's range.
__device__ __forceinline__ void dequant_fp4x32(u32x4_t v, float scale, bf16x8_t out[4]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[d], scale, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[d], scale, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[d], scale, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v[d], scale, 3);
    out[d] = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
}

// Group d of dequant_fp4x32: 4 packed E2M1 bytes (8 codes) times the block
// scale -> 8 bf16.
__device__ __forceinline__ bf16x8_t dequant_fp4x8(uint32_t v, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// D[16x16] += A[16 x 32] * B[32 x 16] in fp32.  Lane l holds row (l % 16) of
// A and column (l % 16) of B, contraction elements 8*(l/16) .. +8; it gets
// back D rows 4*(l/16) .. +4 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ u32x4_t ld16(const void *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

__device__ __forceinline__ u32x4_t ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MB_WAVE);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, MB_WAVE));
  return v;
}

// Block-wide sum in a fixed order (wave sums, then the wave totals in wave
// order), so the result does not depend on scheduling.  `red` holds
// blockDim/64 entries.  Every thread gets the total.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T *red) {
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int nw = blockDim.x / MB_WAVE;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  T t = red[0];
  for (int w = 1; w < nw; ++w) t += red[w];
  return t;
}
