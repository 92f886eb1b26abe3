// A STREAM-like HBM read kernel, built as its own small library
// (libmb_readprobe.so) for bench.py --read-probe: it gives the read
// bandwidth one launch of plain coalesced loads reaches on the device, the
// practical ceiling to set beside the 8 TB/s peak; and an L2-resident read in
// the two shapes a weight tile's wave loads can take.  Not part of libmb.so.
//
// Every thread reads 16-byte words at a grid stride, `U` words in flight per
// step, and folds them into a value it stores only if it equals a constant
// the data never produces (so the loads are kept).

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *__restrict__ p, size_t n, uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// The two shapes of a wave load of an MFMA weight tile, over a buffer small
// enough to stay in the L2 (every step re-reads it): kTile false, each wave
// load 1 KB contiguous (the streaming layouts); kTile true, 16 rows of
// `row_bytes` apart, 64 bytes of each (lane l: row (16 w + l % 16) % rows,
// bytes 16 (l / 16) + 64 c; the caller's row-major layout).  Each step
// requests 8 loads per lane.
template <bool kTile>
__global__ __launch_bounds__(kThreads) void tile_read_kernel(const u32x4 *__restrict__ p, uint32_t words_mask,
                                                             uint32_t rows, uint32_t row_bytes, int steps,
                                                             uint32_t *sink) {
  const uint32_t lane = threadIdx.x % 64, wave = blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int it = 0; it < steps; ++it) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t k = (uint32_t)(it * 8 + u);
      uint32_t w;
      if (kTile) {
        const uint32_t row = (16 * wave + lane % 16) % rows, c = k % (row_bytes / 64);
        w = (row * row_bytes + 64 * c + 16 * (lane / 16)) / 16;
      } else {
        w = (blockIdx.x * kThreads + threadIdx.x + k * stride) & words_mask;
      }
      v[u] = p[w];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// L2-resident read of `buf` in the shape of a weight tile's wave loads
// (tile_read_kernel): tile 0, contiguous over `bytes` (a power of two,
// 16 .. 2^32); tile 1, rows x row_bytes bytes (row_bytes a multiple of 64,
// rows x row_bytes <= bytes < 2^32).  grid workgroups of 256 threads, `steps`
// steps of 8 loads each; reads grid * 256 * 128 * steps bytes.  sink: device
// memory of at least grid words.  0 = ok, 1 = bad argument, 2 = launch failed.
int mbp_tile_read(const void *buf, size_t bytes, int tile, uint32_t rows, uint32_t row_bytes, int steps, int grid,
                  uint32_t *sink, void *stream) {
  if (!buf || !sink || grid < 1 || steps < 1 || bytes < 16 || bytes > (size_t)1 << 32) return 1;
  const u32x4 *p = static_cast<const u32x4 *>(buf);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (tile) {
    if (rows < 1 || row_bytes < 64 || row_bytes % 64 || (size_t)rows * row_bytes > bytes) return 1;
    hipLaunchKernelGGL((tile_read_kernel<true>), dim3(grid), dim3(kThreads), 0, s, p, 0u, rows, row_bytes, steps,
                       sink);
  } else {
    if (bytes & (bytes - 1)) return 1;
    hipLaunchKernelGGL((tile_read_kernel<false>), dim3(grid), dim3(kThreads), 0, s, p, (uint32_t)(bytes / 16 - 1),
                       0u, 0u, steps, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}


// Read `bytes` (a multiple of 16) at `buf` with `grid` workgroups of 256;
// variant 0..3 = {4, 8} words in flight x {plain, nontemporal} loads.  sink:
// device memory of at least grid words (normally never written).  0 = ok,
// 1 = bad argument, 2 = launch failed.
int mbp_read(const void *buf, size_t bytes, int grid, int variant, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes % 16 || grid < 1 || variant < 0 || variant > 3) return 1;
  const u32x4 *p = static_cast<const u32x4 *>(buf);
  const size_t n = bytes / 16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case 0: hipLaunchKernelGGL((read_kernel<4, false>), dim3(grid), dim3(kThreads), 0, s, p, n, sink); break;
    case 1: hipLaunchKernelGGL((read_kernel<8, false>), dim3(grid), dim3(kThreads), 0, s, p, n, sink); break;
    case 2: hipLaunchKernelGGL((read_kernel<4, true>), dim3(grid), dim3(kThreads), 0, s, p, n, sink); break;
    default: hipLaunchKernelGGL((read_kernel<8, true>), dim3(grid), dim3(kThreads), 0, s, p, n, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
