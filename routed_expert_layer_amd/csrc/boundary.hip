// The FFN boundary after the unpooler ([providers] BoundaryProvider:
// post_ffn_norm, the gated add into the fp32 stream in place, and the next
// pre-norm into a bf16 output):
//   v      = u / sqrt(mean_H(u^2) + eps) * ffn_norm_w
//   stream = fp32(stream + gate * v)          (one rounding: fma)
//   x_next = bf16(stream / sqrt(mean_H(stream^2) + eps) * next_norm_w)
// One workgroup per row: rows of up to 8192 with all of the row's loads issued
// at once, wider rows in three passes; both sums of squares are fixed-order
// block sums.

#include "mb_device.h"
#include "mb_internal.h"

namespace mb {
namespace {

__device__ __forceinline__ void unpack4(u32x2_t v, float o[4]) {
  o[0] = bf16_bits_to_f32(v[0] & 0xFFFFu);
  o[1] = bf16_bits_to_f32(v[0] >> 16);
  o[2] = bf16_bits_to_f32(v[1] & 0xFFFFu);
  o[3] = bf16_bits_to_f32(v[1] >> 16);
}

// Rows wider than 8192: three passes over the row.
__global__ __launch_bounds__(256) void boundary_kernel_wide(
    const uint16_t *__restrict__ u, float *__restrict__ stream, const uint16_t *__restrict__ gate,
    const uint16_t *__restrict__ wpff, const uint16_t *__restrict__ win,
    uint16_t *__restrict__ x_next, int H, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const uint16_t *urow = u + (size_t)t * H;
  float *srow = stream + (size_t)t * H;
  float ss = 0.f;
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    float v[4];
    unpack4(*reinterpret_cast<const u32x2_t *>(urow + h), v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float ru = 1.0f / sqrtf(ss / (float)H + eps);
  float s2 = 0.f;
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    float v[4], gg[4], wf[4] = {1.f, 1.f, 1.f, 1.f};
    unpack4(*reinterpret_cast<const u32x2_t *>(urow + h), v);
    unpack4(*reinterpret_cast<const u32x2_t *>(gate + h), gg);
    if (wpff) unpack4(*reinterpret_cast<const u32x2_t *>(wpff + h), wf);
    f32x4_t s = *reinterpret_cast<const f32x4_t *>(srow + h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float vn = v[i] * ru * wf[i];
      s[i] = fmaf(gg[i], vn, s[i]);
      s2 += s[i] * s[i];
    }
    *reinterpret_cast<f32x4_t *>(srow + h) = s;
  }
  s2 = block_sum(s2, red);
  const float rsn = 1.0f / sqrtf(s2 / (float)H + eps);
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    float wi[4] = {1.f, 1.f, 1.f, 1.f};
    if (win) unpack4(*reinterpret_cast<const u32x2_t *>(win + h), wi);
    const f32x4_t s = *reinterpret_cast<const f32x4_t *>(srow + h);
    u32x2_t pk = {pack_bf16x2(s[0] * rsn * wi[0], s[1] * rsn * wi[1]),
                  pack_bf16x2(s[2] * rsn * wi[2], s[3] * rsn * wi[3])};
    *reinterpret_cast<u32x2_t *>(x_next + (size_t)t * H + h) = pk;
  }
}

// Thread t holds elements 4 (t + 256 g) .. + 3 of the row for g < kRowGroups
// (H <= 4096 * kRowGroups / 4): every load of the row is issued at once, so
// the row costs one memory round trip rather than one per pass and group.
constexpr int kRowGroups = 8;

__global__ __launch_bounds__(256) void boundary_kernel(
    const uint16_t *__restrict__ u, float *__restrict__ stream, const uint16_t *__restrict__ gate,
    const uint16_t *__restrict__ wpff, const uint16_t *__restrict__ win,
    uint16_t *__restrict__ x_next, int H, float eps) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const uint16_t *urow = u + (size_t)t * H;
  float *srow = stream + (size_t)t * H;
  u32x2_t uv[kRowGroups], gv[kRowGroups], fv[kRowGroups], iv[kRowGroups];
  f32x4_t sv[kRowGroups];
#pragma unroll
  for (int g = 0; g < kRowGroups; ++g) {
    const int h = (threadIdx.x + 256 * g) * 4;
    const bool ok = h < H;
    const u32x2_t one = {0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
    uv[g] = ok ? *reinterpret_cast<const u32x2_t *>(urow + h) : u32x2_t{0u, 0u};
    gv[g] = ok ? *reinterpret_cast<const u32x2_t *>(gate + h) : u32x2_t{0u, 0u};
    fv[g] = (ok && wpff) ? *reinterpret_cast<const u32x2_t *>(wpff + h) : one;
    iv[g] = (ok && win) ? *reinterpret_cast<const u32x2_t *>(win + h) : one;
    sv[g] = ok ? *reinterpret_cast<const f32x4_t *>(srow + h) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int g = 0; g < kRowGroups; ++g) {
    float v[4];
    unpack4(uv[g], v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float ru = 1.0f / sqrtf(ss / (float)H + eps);
  float s2 = 0.f;
#pragma unroll
  for (int g = 0; g < kRowGroups; ++g) {
    float v[4], gg[4], wf[4];
    unpack4(uv[g], v);
    unpack4(gv[g], gg);
    unpack4(fv[g], wf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float vn = v[i] * ru * wf[i];
      sv[g][i] = fmaf(gg[i], vn, sv[g][i]);
      s2 += sv[g][i] * sv[g][i];
    }
    const int h = (threadIdx.x + 256 * g) * 4;
    if (h < H) *reinterpret_cast<f32x4_t *>(srow + h) = sv[g];
  }
  s2 = block_sum(s2, red);
  const float rsn = 1.0f / sqrtf(s2 / (float)H + eps);
#pragma unroll
  for (int g = 0; g < kRowGroups; ++g) {
    float wi[4];
    unpack4(iv[g], wi);
    const f32x4_t s = sv[g];
    const int h = (threadIdx.x + 256 * g) * 4;
    if (h < H)
      *reinterpret_cast<u32x2_t *>(x_next + (size_t)t * H + h) =
          u32x2_t{pack_bf16x2(s[0] * rsn * wi[0], s[1] * rsn * wi[1]),
                  pack_bf16x2(s[2] * rsn * wi[2], s[3] * rsn * wi[3])};
  }
}

// out[i] = bf16(fp32(weight[i] + add)), round to nearest even.
__global__ __launch_bounds__(256) void norm_weight_kernel(const float *__restrict__ weight, int n, float add,
                                                          uint16_t *__restrict__ out) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256)
    out[i] = f32_to_bf16_bits(weight[i] + add);
}

}  // namespace

hipError_t launch_norm_weight(const float *weight, int n, float add, uint16_t *out, hipStream_t s) {
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  hipLaunchKernelGGL(norm_weight_kernel, dim3(blocks), dim3(256), 0, s, weight, n, add, out);
  return hipGetLastError();
}

hipError_t launch_boundary(const mb_dims &d, const uint16_t *u, float *stream,
                           const uint16_t *gate, const uint16_t *ffn_norm_w,
                           const uint16_t *next_norm_w, uint16_t *x_next, hipStream_t s) {
  if (d.hidden > 1024 * kRowGroups) {
    hipLaunchKernelGGL(boundary_kernel_wide, dim3(d.rows), dim3(256), 0, s, u, stream, gate, ffn_norm_w,
                       next_norm_w, x_next, d.hidden, d.norm_eps);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(boundary_kernel, dim3(d.rows), dim3(256), 0, s, u, stream, gate, ffn_norm_w,
                     next_norm_w, x_next, d.hidden, d.norm_eps);
  return hipGetLastError();
}

}  // namespace mb
