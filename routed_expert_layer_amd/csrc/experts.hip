// Routed MXFP4 experts and the tail (per-route norm, weighting, sum).
//
// Semantics ([muse_moe_runner] MuseSparkAiterExperts.apply returns one
// unweighted output per route; MuseSparkTopKWeightAndReduce.apply applies the
// per-route norm, then the route weight, then sums over routes and casts):
//   gu  = dec(w13[e]) @ h[t]            act = bf16(silu(gu[:I]) * gu[I:])
//   y   = dec(w2[e]) @ act              yn  = RMSNorm_P(y) * w_post
//   moe_out[t] = bf16(sum_j w[t, j] * yn(t, j))
// Weights are MXFP4 in the layout of [mono.decoder] MonoDims.expert_shapes:
// w13 u8 [E, 2I, P/2] + E8M0 [E, 2I, P/32], w2 u8 [E, P, I/2] + [E, P, I/32].
//
// Kernel layout.  The expert weights are the bulk of the block's HBM traffic
// and are read once.  Work items are (active expert, tile of weight rows);
// the four waves of a workgroup split the contraction into interleaved
// 128-element chunks.  Per chunk a lane loads 16 bytes (one 32-element MXFP4
// block, one scale byte) of weight row (l % 16), 128-bit and coalesced as
// 16 rows x 64 contiguous bytes per wave load, converts them to bf16 in
// registers with the hardware's scaled fp4 converts (exact), and feeds four
// 16x16x32 bf16 MFMAs whose B operand is 16 routes of the expert's bf16
// activations.  The four waves' partial sums meet in LDS and the epilogue is
// fused: the gated activation after w13, and after w2 the route-order store
// of y with per-tile sums of squares for the per-route norm.  The routes of
// an expert are processed 16 at a time, so any number of rows per expert is
// served by the same kernel.

#include "mb_device.h"
#include "mb_internal.h"

namespace mb {
namespace {

template <int UNR>
__global__ __launch_bounds__(256) void experts_up_kernel(
    const uint16_t *__restrict__ h, const int32_t *__restrict__ offset,
    const int32_t *__restrict__ route_list, const int32_t *__restrict__ active,
    const int32_t *__restrict__ n_active, const uint8_t *__restrict__ w13,
    const uint8_t *__restrict__ w13s, uint16_t *__restrict__ act, int P, int I, int k) {
  const int tiles = I / 16;
  const int a = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (a >= *n_active) return;
  const int e = active[a];
  const int row0 = offset[e], nrows = offset[e + 1] - row0;
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int g = lane >> 4, r16 = lane & 15;
  const int i0 = tile * 16;
  const size_t rb = (size_t)P / 2, sb = (size_t)P / 32;
  const size_t rg = (size_t)e * 2 * I + i0 + r16, ru = rg + I;
  const uint8_t *wg = w13 + rg * rb + 16 * g;
  const uint8_t *wu = w13 + ru * rb + 16 * g;
  const uint8_t *sg = w13s + rg * sb + g;
  const uint8_t *su = w13s + ru * sb + g;
  const int nch = P / 128;
  __shared__ f32x4_t red[4][2][MB_WAVE];

  for (int m0 = 0; m0 < nrows; m0 += 16) {
    const int m = m0 + r16;
    const bool valid = m < nrows;
    const int t = valid ? route_list[row0 + m] / k : 0;
    const uint16_t *hrow = h + (size_t)t * P + 32 * g;
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nch; c += 4 * UNR) {
      u32x4_t vg[UNR], vu[UNR], hv[UNR][4];
      uint32_t bg[UNR], bu[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int cc = c + 4 * u;
        const bool ok = cc < nch;
        vg[u] = ok ? ld16_nt(wg + 64 * cc) : u32x4_t{0, 0, 0, 0};
        vu[u] = ok ? ld16_nt(wu + 64 * cc) : u32x4_t{0, 0, 0, 0};
        bg[u] = ok ? sg[4 * cc] : 0u;
        bu[u] = ok ? su[4 * cc] : 0u;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int cc = c + 4 * u;
        const bool ok = cc < nch && valid;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hv[u][i] = ok ? ld16(hrow + 128 * cc + 8 * i) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (c + 4 * u < nch) {
          bf16x8_t G[4], U[4];
          dequant_fp4x32(vg[u], e8m0_to_f32(bg[u]), G);
          dequant_fp4x32(vu[u], e8m0_to_f32(bu[u]), U);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ag = mfma_bf16(G[i], as_bf16x8(hv[u][i]), ag);
            au = mfma_bf16(U[i], as_bf16x8(hv[u][i]), au);
          }
        }
      }
    }
    red[wave][0][lane] = ag;
    red[wave][1][lane] = au;
    __syncthreads();
    if (wave == 0 && valid) {
      const f32x4_t gs = ((red[0][0][lane] + red[1][0][lane]) + red[2][0][lane]) + red[3][0][lane];
      const f32x4_t us = ((red[0][1][lane] + red[1][1][lane]) + red[2][1][lane]) + red[3][1][lane];
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = gs[i];
        const float sz = z / (1.0f + expf(-z));
        o[i] = sz * us[i];
      }
      u32x2_t pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2_t *>(act + (size_t)(row0 + m) * I + i0 + 4 * g) = pk;
    }
    __syncthreads();
  }
}

template <int UNR>
__global__ __launch_bounds__(256) void experts_down_kernel(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ offset,
    const int32_t *__restrict__ route_list, const int32_t *__restrict__ active,
    const int32_t *__restrict__ n_active, const uint8_t *__restrict__ w2,
    const uint8_t *__restrict__ w2s, float *__restrict__ y, float *__restrict__ ssq, int P, int I) {
  const int tiles = P / 32;
  const int a = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (a >= *n_active) return;
  const int e = active[a];
  const int row0 = offset[e], nrows = offset[e + 1] - row0;
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int g = lane >> 4, r16 = lane & 15;
  const int p0 = tile * 32;
  const size_t rb = (size_t)I / 2, sb = (size_t)I / 32;
  const size_t r0 = (size_t)e * P + p0 + r16, r1 = r0 + 16;
  const uint8_t *w0 = w2 + r0 * rb + 16 * g;
  const uint8_t *w1 = w2 + r1 * rb + 16 * g;
  const uint8_t *s0 = w2s + r0 * sb + g;
  const uint8_t *s1 = w2s + r1 * sb + g;
  const int nch = I / 128;
  __shared__ f32x4_t red[4][2][MB_WAVE];

  for (int m0 = 0; m0 < nrows; m0 += 16) {
    const int m = m0 + r16;
    const bool valid = m < nrows;
    const uint16_t *arow = act + (size_t)(row0 + (valid ? m : 0)) * I + 32 * g;
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int c = wave; c < nch; c += 4 * UNR) {
      u32x4_t v0[UNR], v1[UNR], av[UNR][4];
      uint32_t b0[UNR], b1[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int cc = c + 4 * u;
        const bool ok = cc < nch;
        v0[u] = ok ? ld16_nt(w0 + 64 * cc) : u32x4_t{0, 0, 0, 0};
        v1[u] = ok ? ld16_nt(w1 + 64 * cc) : u32x4_t{0, 0, 0, 0};
        b0[u] = ok ? s0[4 * cc] : 0u;
        b1[u] = ok ? s1[4 * cc] : 0u;
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int cc = c + 4 * u;
        const bool ok = cc < nch && valid;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[u][i] = ok ? ld16(arow + 128 * cc + 8 * i) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (c + 4 * u < nch) {
          bf16x8_t A0[4], A1[4];
          dequant_fp4x32(v0[u], e8m0_to_f32(b0[u]), A0);
          dequant_fp4x32(v1[u], e8m0_to_f32(b1[u]), A1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a0 = mfma_bf16(A0[i], as_bf16x8(av[u][i]), a0);
            a1 = mfma_bf16(A1[i], as_bf16x8(av[u][i]), a1);
          }
        }
      }
    }
    red[wave][0][lane] = a0;
    red[wave][1][lane] = a1;
    __syncthreads();
    if (wave == 0) {
      const f32x4_t y0 = ((red[0][0][lane] + red[1][0][lane]) + red[2][0][lane]) + red[3][0][lane];
      const f32x4_t y1 = ((red[0][1][lane] + red[1][1][lane]) + red[2][1][lane]) + red[3][1][lane];
      float ss = 0.f;
      if (valid) {
        ss = y0[0] * y0[0] + y0[1] * y0[1] + y0[2] * y0[2] + y0[3] * y0[3];
        ss += y1[0] * y1[0] + y1[1] * y1[1] + y1[2] * y1[2] + y1[3] * y1[3];
      }
      ss += __shfl_xor(ss, 16, MB_WAVE);
      ss += __shfl_xor(ss, 32, MB_WAVE);
      if (valid) {
        const int r = route_list[row0 + m];
        *reinterpret_cast<f32x4_t *>(y + (size_t)r * P + p0 + 4 * g) = y0;
        *reinterpret_cast<f32x4_t *>(y + (size_t)r * P + p0 + 16 + 4 * g) = y1;
        if (g == 0) ssq[(size_t)r * tiles + tile] = ss;
      }
    }
    __syncthreads();
  }
}

// moe_out[t] = bf16(sum_j w[t, j] * y(t, j) / sqrt(ss(t, j) / P + eps) * w_post),
// ss(t, j) = the sum of the route's per-tile sums of squares in tile order.
__global__ __launch_bounds__(256) void experts_finalize_kernel(
    const float *__restrict__ y, const float *__restrict__ ssq, const float *__restrict__ wts,
    const uint16_t *__restrict__ post, uint16_t *__restrict__ moe_out, int P, int k, float eps) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int tiles = P / 32;
  __shared__ float coef[kMaxTopK];
  for (int j = wave; j < k; j += 4) {
    const float *row = ssq + (size_t)(t * k + j) * tiles;
    float s = 0.f;
    for (int q = lane; q < tiles; q += MB_WAVE) s += row[q];
    s = wave_sum(s);
    if (lane == 0) {
      const float rs = 1.0f / sqrtf(s / (float)P + eps);
      coef[j] = wts[(size_t)t * k + j] * rs;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x * 4; p < P; p += blockDim.x * 4) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j)
      acc += coef[j] * *reinterpret_cast<const f32x4_t *>(y + (size_t)(t * k + j) * P + p);
    const u32x2_t pw = *reinterpret_cast<const u32x2_t *>(post + p);
    const float o0 = acc[0] * bf16_bits_to_f32(pw[0] & 0xFFFFu);
    const float o1 = acc[1] * bf16_bits_to_f32(pw[0] >> 16);
    const float o2 = acc[2] * bf16_bits_to_f32(pw[1] & 0xFFFFu);
    const float o3 = acc[3] * bf16_bits_to_f32(pw[1] >> 16);
    u32x2_t pk = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
    *reinterpret_cast<u32x2_t *>(moe_out + (size_t)t * P + p) = pk;
  }
}

}  // namespace

hipError_t launch_experts_up(const mb_dims &d, const uint16_t *h, const int32_t *offset,
                             const int32_t *route_list, const int32_t *active,
                             const int32_t *n_active, const uint8_t *w13,
                             const uint8_t *w13_scale, uint16_t *act, hipStream_t s) {
  dim3 grid(d.experts * (d.inter / 16));
  hipLaunchKernelGGL((experts_up_kernel<4>), grid, dim3(256), 0, s, h, offset, route_list, active,
                     n_active, w13, w13_scale, act, d.pooled, d.inter, d.top_k);
  return hipGetLastError();
}

hipError_t launch_experts_down(const mb_dims &d, const uint16_t *act, const int32_t *offset,
                               const int32_t *route_list, const int32_t *active,
                               const int32_t *n_active, const uint8_t *w2,
                               const uint8_t *w2_scale, float *y, float *ssq, hipStream_t s) {
  dim3 grid(d.experts * (d.pooled / 32));
  hipLaunchKernelGGL((experts_down_kernel<4>), grid, dim3(256), 0, s, act, offset, route_list,
                     active, n_active, w2, w2_scale, y, ssq, d.pooled, d.inter);
  return hipGetLastError();
}

hipError_t launch_experts_finalize(const mb_dims &d, const float *y, const float *ssq,
                                   const float *wts, const uint16_t *post_norm_w,
                                   uint16_t *moe_out, hipStream_t s) {
  hipLaunchKernelGGL(experts_finalize_kernel, dim3(d.rows), dim3(256), 0, s, y, ssq, wts,
                     post_norm_w, moe_out, d.pooled, d.top_k, d.norm_eps);
  return hipGetLastError();
}

}  // namespace mb
