// A STREAM-like HBM read kernel, built as its own small library
// (libmb_readprobe.so) for bench.py --read-probe: it gives the read
// bandwidth one launch of plain coalesced loads reaches on the device, the
// practical ceiling to set beside the 8 TB/s peak.  Not part of libmb.so.
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

}  // namespace

extern "C" {

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
