// Repacking of the MXFP4 expert weights, and of the pooler's and unpooler's
// bf16 weights, into the streaming layouts the block kernel reads (layouts in
// mb_block.h, PackedExperts and PackedProjections).
//
// The values are the caller's: the codes and E8M0 scales of w13 and w2 in the
// layout of [mono.decoder] MonoDims.expert_shapes, moved so that each wave
// load of an expert unit is one contiguous kilobyte instead of sixteen
// 64-byte pieces of sixteen rows; likewise the bf16 pooler and unpooler
// matrices, whose 64-byte row pieces read from sixteen rows at once reach a
// quarter of the rate of contiguous loads.  This is done once per set of weights, when
// they are loaded ([muse_moe_runner] MuseSparkAiterExperts: the ROCm experts
// likewise take their weights in a layout prepared at load time).

#include "mb_block.h"

namespace mb {
namespace {

// One 16-byte piece of one code section per thread: piece q of expert
// blockIdx.y is lane q % 64 of tile (q / 64) % 2 of chunk (q / 128) % nch of
// unit q / (128 nch).  Tile t of unit u is rows unit_rows * u + t * t1_row ..
// + 15 of the expert's [rows, kdim / 2]-byte matrix.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *__restrict__ src, size_t src_stride,
                                                         uint8_t *__restrict__ dst, size_t dst_stride,
                                                         size_t dst_off, int units, int nch, int kdim,
                                                         int unit_rows, int t1_row) {
  const size_t pieces = (size_t)units * nch * 128;
  const uint8_t *s = src + (size_t)blockIdx.y * src_stride;
  uint8_t *o = dst + (size_t)blockIdx.y * dst_stride + dst_off;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < pieces; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q % 64), t = (int)((q / 64) % 2), c = (int)((q / 128) % nch);
    const int u = (int)(q / (128 * (size_t)nch));
    const size_t row = (size_t)unit_rows * u + (size_t)t * t1_row + (lane & 15);
    const size_t from = row * (size_t)(kdim / 2) + 64 * (size_t)c + 16 * (size_t)(lane >> 4);
    *reinterpret_cast<uint4 *>(o + 16 * q) = *reinterpret_cast<const uint4 *>(s + from);
  }
}

// One 4-byte word of one scale section per thread: word q is lane q % 64 of
// tile (q / 64) % 2 of group (q / 128) % ngr of unit q / (128 ngr); byte j
// holds the scale of row q % 16 of the tile, block (q % 64) / 16 of chunk
// 4 ((q / 128) % ngr) + j, with 127 (2^0) past the row's kdim / 32.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t *__restrict__ src, size_t src_stride,
                                                          uint8_t *__restrict__ dst, size_t dst_stride,
                                                          size_t dst_off, int units, int ngr, int kdim,
                                                          int unit_rows, int t1_row) {
  const size_t words = (size_t)units * ngr * 128;
  const int row_bytes = kdim / 32;
  const uint8_t *s = src + (size_t)blockIdx.y * src_stride;
  uint8_t *o = dst + (size_t)blockIdx.y * dst_stride + dst_off;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < words; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q % 64), t = (int)((q / 64) % 2), g = (int)((q / 128) % ngr);
    const int u = (int)(q / (128 * (size_t)ngr));
    const size_t row = (size_t)unit_rows * u + (size_t)t * t1_row + (lane & 15);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 4 * (4 * g + j) + (lane >> 4);
      w |= (uint32_t)(b < row_bytes ? s[row * row_bytes + b] : (uint8_t)127) << (8 * j);
    }
    *reinterpret_cast<uint32_t *>(o + 4 * q) = w;
  }
}

// One 16-byte piece of a packed bf16 matrix per thread (PackedProjections):
// piece q is lane q % 64 of chunk (q / 64) % nch of 16-row tile q / (64 nch),
// i.e. elements 32 c + 8 (lane / 16) .. + 7 of row 16 t + lane % 16 of
// src [n_out][kdim] (zeros past n_out).
__global__ __launch_bounds__(256) void pack_dense_kernel(const uint16_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                         int n_out, int kdim) {
  const int nch = kdim / 32;
  const size_t pieces = (size_t)((n_out + 15) / 16) * nch * 64;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < pieces; q += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(q % 64), c = (int)((q / 64) % nch);
    const size_t t = q / (64 * (size_t)nch);
    const size_t row = 16 * t + (size_t)(lane & 15);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < (size_t)n_out)
      v = *reinterpret_cast<const uint4 *>(src + row * (size_t)kdim + 32 * (size_t)c + 8 * (size_t)(lane >> 4));
    *reinterpret_cast<uint4 *>(dst + 16 * q) = v;
  }
}

dim3 grid_for(size_t pieces, int experts) {
  size_t x = (pieces + 255) / 256;
  if (x > 1024) x = 1024;
  return dim3((unsigned)x, (unsigned)experts);
}

}  // namespace

hipError_t launch_pack_experts(const mb_dims &d, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                               const uint8_t *w2s, uint8_t *packed, hipStream_t s) {
  const int P = d.pooled, I = d.inter, E = d.experts;
  const PackedExperts L = packed_experts(P, I);
  const int up_units = I / 16, down_units = P / 32;
  const int up_nch = P / 128, down_nch = I / 128;
  const int up_ngr = (up_nch + 3) / 4, down_ngr = (down_nch + 3) / 4;
  hipLaunchKernelGGL(pack_codes_kernel, grid_for((size_t)up_units * up_nch * 128, E), dim3(256), 0, s, w13,
                     (size_t)2 * I * (P / 2), packed, L.stride, (size_t)0, up_units, up_nch, P, 16, I);
  hipLaunchKernelGGL(pack_scales_kernel, grid_for((size_t)up_units * up_ngr * 128, E), dim3(256), 0, s, w13s,
                     (size_t)2 * I * (P / 32), packed, L.stride, L.up_s, up_units, up_ngr, P, 16, I);
  hipLaunchKernelGGL(pack_codes_kernel, grid_for((size_t)down_units * down_nch * 128, E), dim3(256), 0, s, w2,
                     (size_t)P * (I / 2), packed, L.stride, L.down, down_units, down_nch, I, 32, 16);
  hipLaunchKernelGGL(pack_scales_kernel, grid_for((size_t)down_units * down_ngr * 128, E), dim3(256), 0, s, w2s,
                     (size_t)P * (I / 32), packed, L.stride, L.down_s, down_units, down_ngr, I, 32, 16);
  return hipGetLastError();
}

hipError_t launch_pack_projections(const mb_dims &d, const uint16_t *pool_w, const uint16_t *unpool_w,
                                   uint8_t *packed, hipStream_t s) {
  const int P = d.pooled, H = d.hidden;
  const PackedProjections L = packed_projections(P, H);
  hipLaunchKernelGGL(pack_dense_kernel, grid_for(packed_matrix_bytes(P, H) / 16, 1), dim3(256), 0, s, pool_w,
                     packed, P, H);
  hipLaunchKernelGGL(pack_dense_kernel, grid_for(packed_matrix_bytes(H, P) / 16, 1), dim3(256), 0, s, unpool_w,
                     packed + L.unpool, H, P);
  return hipGetLastError();
}

}  // namespace mb
