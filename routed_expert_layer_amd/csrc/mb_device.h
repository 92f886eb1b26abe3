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

// D[16x16] += A[16 x 4] * B[4 x 16] in fp64.  Lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16]; element v of the result is D[4 v + l / 16][l % 16].
typedef double f64x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f64x4_t mfma_f64(double a, double b, f64x4_t c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// D += (A with its lanes' E8M0 scales) x (B with theirs), A and B MXFP4: the
// 16x16x128 scaled MFMA with E2M1 operands.  A lane holds 32 codes (16 bytes,
// element k at nibble k % 8 of word k / 8, low nibble first) of row / column
// lane % 16, K block lane / 16; byte OP of sa / sb is its block's scale.  D is
// laid out as for the 16x16x32 bf16 MFMA.
template <int OP>
__device__ __forceinline__ f32x4_t mfma_fp4(u32x4_t a, u32x4_t b, f32x4_t c, uint32_t sa, uint32_t sb) {
  typedef __attribute__((ext_vector_type(8))) int i32x8_t;
  const i32x8_t A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8_t B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, OP, (int)sa, OP, (int)sb);
}

// E2M1 code of x (already divided by its block scale): the nearest of 0, 0.5,
// 1, 1.5, 2, 3, 4, 6, ties to the even mantissa, saturating at 6; sign in
// bit 3 (OCP Microscaling Formats v1.0: E2M1, and section 6.3's rounding).
__device__ __forceinline__ uint32_t e2m1_code(float x) {
  const float a = fabsf(x);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return m | (x < 0.f ? 8u : 0u);
}

// E8M0 byte of a block's shared exponent: floor(log2(amax)) - 2, within
// [-127, 127] (amax 0: the smallest, 2^-127).  amax is a normal fp32 value or 0.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 : -127;
  const int se = min(127, max(-127, e - 2));
  return (uint32_t)(se + 127);
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
