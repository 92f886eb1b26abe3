// Skinny bf16 projections: the pooler h = bf16(x @ Wp^T) and the unpooler
// u = bf16(moe_out @ Wu^T) ([providers] MoEProvider: pooler GEMM and
// unpooler GEMM; [mono.decoder] layer_refusals: pooler bf16 (P, H), unpooler
// bf16 (H, P)).
//
// At decode row counts the weight matrix is read once and dominates the
// traffic, so the kernel is laid out for streaming it: a workgroup owns 16
// weight rows (output features) and a contiguous slice of the contraction
// dimension, its four waves take interleaved 32-element chunks of that slice,
// and every chunk is one 16x16x32 bf16 MFMA per 16 activation rows (weights
// in the A operand, activations in the B operand).  Lane l loads 16 bytes of
// weight row (l % 16) at element 8*(l/16) of the chunk, so a wave load covers
// 16 rows x 64 contiguous bytes.  When the contraction is split over several
// workgroups, each writes fp32 partial sums and a second small kernel adds
// them in split order and writes bf16, so the result does not depend on
// completion order (and no workgroup pays for a device-wide cache flush).

#include "mb_device.h"
#include "mb_internal.h"

namespace mb {
namespace {

template <int MG, int UNR>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t *__restrict__ a,
                                                        const uint16_t *__restrict__ w,
                                                        uint16_t *__restrict__ out, int rows,
                                                        int n_out, int kdim, int ks_count,
                                                        int chunks_per_wg,
                                                        float *__restrict__ partial) {
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int g = lane >> 4, r16 = lane & 15;
  const int ntile = blockIdx.x, ks = blockIdx.y, rb = blockIdx.z;
  const int row_base = rb * 16 * MG;
  const int nchunks = kdim / 32;
  const int c_begin = ks * chunks_per_wg;
  const int c_end = min(nchunks, c_begin + chunks_per_wg);

  const uint16_t *wrow = w + (size_t)(ntile * 16 + r16) * kdim + 8 * g;
  const uint16_t *arow[MG];
  bool aval[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) {
    const int t = row_base + mg * 16 + r16;
    aval[mg] = t < rows;
    arow[mg] = a + (size_t)(aval[mg] ? t : 0) * kdim + 8 * g;
  }
  f32x4_t acc[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) acc[mg] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = c_begin + wave; c < c_end; c += 4 * UNR) {
    u32x4_t wv[UNR];
    u32x4_t av[UNR][MG];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int cc = c + 4 * u;
      wv[u] = cc < c_end ? ld16_nt(wrow + cc * 32) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int cc = c + 4 * u;
#pragma unroll
      for (int mg = 0; mg < MG; ++mg)
        av[u][mg] = (cc < c_end && aval[mg]) ? ld16(arow[mg] + cc * 32) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (c + 4 * u < c_end) {
#pragma unroll
        for (int mg = 0; mg < MG; ++mg)
          acc[mg] = mfma_bf16(as_bf16x8(wv[u]), as_bf16x8(av[u][mg]), acc[mg]);
      }
    }
  }

  __shared__ f32x4_t red[4][MG][MB_WAVE];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) red[wave][mg][lane] = acc[mg];
  __syncthreads();
  for (int mg = wave; mg < MG; mg += 4) {
    const f32x4_t v = ((red[0][mg][lane] + red[1][mg][lane]) + red[2][mg][lane]) + red[3][mg][lane];
    const int t = row_base + mg * 16 + r16;
    if (t < rows) {
      const int n0 = ntile * 16 + 4 * g;
      if (ks_count == 1) {
        u32x2_t pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2_t *>(out + (size_t)t * n_out + n0) = pk;
      } else {
        *reinterpret_cast<f32x4_t *>(partial + ((size_t)ks * rows + t) * n_out + n0) = v;
      }
    }
  }
}

// out[t, n] = bf16(sum over splits q of partial[q, t, n]), in split order.
__global__ __launch_bounds__(256) void splitk_sum_bf16_kernel(const float *__restrict__ partial,
                                                              uint16_t *__restrict__ out, int rows,
                                                              int n_out, int ks_count) {
  const size_t n4 = (size_t)rows * n_out / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    f32x4_t s = reinterpret_cast<const f32x4_t *>(partial)[i];
    for (int q = 1; q < ks_count; ++q)
      s += reinterpret_cast<const f32x4_t *>(partial + (size_t)q * rows * n_out)[i];
    u32x2_t pk = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    reinterpret_cast<u32x2_t *>(out)[i] = pk;
  }
}

template <int MG, int UNR>
hipError_t launch_mg(dim3 grid, hipStream_t s, const uint16_t *a, const uint16_t *w,
                     uint16_t *out, int rows, int n_out, int kdim, int ks, int cpw, float *partial) {
  hipLaunchKernelGGL((gemm_bf16_kernel<MG, UNR>), grid, dim3(256), 0, s, a, w, out, rows, n_out,
                     kdim, ks, cpw, partial);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (ks > 1) {
    const int n4 = rows * n_out / 4;
    hipLaunchKernelGGL(splitk_sum_bf16_kernel, dim3((n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024),
                       dim3(256), 0, s, partial, out, rows, n_out, ks);
  }
  return hipGetLastError();
}

// In-place RMSNorm of bf16 rows: h = bf16(h / sqrt(mean(h^2) + eps) * w).
__global__ __launch_bounds__(256) void rownorm_bf16_kernel(uint16_t *__restrict__ h,
                                                           const uint16_t *__restrict__ wt,
                                                           int width, float eps) {
  __shared__ float red[4];
  uint16_t *row = h + (size_t)blockIdx.x * width;
  float ss = 0.f;
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    const float v = bf16_bits_to_f32(row[i]);
    ss += v * v;
  }
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)width + eps);
  for (int i = threadIdx.x; i < width; i += blockDim.x) {
    const float v = bf16_bits_to_f32(row[i]) * rs;
    row[i] = f32_to_bf16_bits(v * bf16_bits_to_f32(wt[i]));
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, uint16_t *out, int rows,
                            int n_out, int kdim, float *partial, uint32_t *counters,
                            hipStream_t s, int ks_cap) {
  const int ntiles = n_out / 16;
  const int nchunks = kdim / 32;
  const int per_pass = rows < 128 ? rows : 128;
  int mg = 1;
  while (mg * 16 < per_pass) mg *= 2;
  const int rblocks = (rows + 16 * mg - 1) / (16 * mg);
  // Enough workgroups to keep every CU streaming, but at least 16 chunks
  // (4 per wave) per workgroup.
  int ks = 1;
  while (2 * ks <= ks_cap && ntiles * rblocks * ks < 1024 && nchunks / (2 * ks) >= 16) ks *= 2;
  const int cpw = (nchunks + ks - 1) / ks;
  ks = (nchunks + cpw - 1) / cpw;
  dim3 grid(ntiles, ks, rblocks);
  switch (mg) {
    case 1: return launch_mg<1, 8>(grid, s, a, w, out, rows, n_out, kdim, ks, cpw, partial);
    case 2: return launch_mg<2, 8>(grid, s, a, w, out, rows, n_out, kdim, ks, cpw, partial);
    case 4: return launch_mg<4, 4>(grid, s, a, w, out, rows, n_out, kdim, ks, cpw, partial);
    default: return launch_mg<8, 2>(grid, s, a, w, out, rows, n_out, kdim, ks, cpw, partial);
  }
}

hipError_t launch_rownorm_bf16(uint16_t *h, const uint16_t *w, int rows, int width, float eps,
                               hipStream_t s) {
  hipLaunchKernelGGL(rownorm_bf16_kernel, dim3(rows), dim3(256), 0, s, h, w, width, eps);
  return hipGetLastError();
}

}  // namespace mb
