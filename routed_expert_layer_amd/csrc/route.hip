// Router projection, scoring, top-k, route weights and route grouping.
//
// The routing recipe is the one of [muse_moe_runner] MuseSpark1xRouter
// (_compute_routing_native): optional output multiplier -> sigmoid/softmax ->
// add the expert bias for selection only -> top-k -> gather the unbiased
// scores -> divide by (sum + division eps) -> scale by route_scale.  The ids
// are int32 and the weights fp32 ([providers] RoutedTopk).
//
// Precision.  The router weight is fp32 [E, H] ([mono.decoder]
// layer_refusals) and reads the bf16 activations ([providers]
// RoutedMoE.build).  Each logit is accumulated in fp64 (every bf16 x fp32
// product is exact in fp64) and rounded once to fp32, and each score is the
// fp32 rounding of an fp64 sigmoid / softmax.  The selection keys, the top-k
// decision and the weight arithmetic are fp32, in the recipe's order.  The
// decision therefore depends only on correctly rounded fp32 values, not on
// the summation order of a particular kernel.

#include "mb_device.h"
#include "mb_internal.h"

namespace mb {
namespace {

constexpr int kRouterRows = 16;  // activation rows per router workgroup

// logits[t, e] = fp32(sum_h x[t, h] * w[e, h]); one workgroup per
// (expert, 16-row block), the hidden dimension spread over 256 threads.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *__restrict__ x,
                                                            const float *__restrict__ wr,
                                                            float *__restrict__ logits, int rows,
                                                            int H, int E) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterRows;
  const int nt = min(kRouterRows, rows - t0);
  double acc[kRouterRows];
#pragma unroll
  for (int t = 0; t < kRouterRows; ++t) acc[t] = 0.0;
  const float *wrow = wr + (size_t)e * H;
  for (int h = threadIdx.x * 4; h < H; h += blockDim.x * 4) {
    const float4 w4 = *reinterpret_cast<const float4 *>(wrow + h);
#pragma unroll
    for (int t = 0; t < kRouterRows; ++t) {
      if (t < nt) {
        const u32x2_t xv = *reinterpret_cast<const u32x2_t *>(x + (size_t)(t0 + t) * H + h);
        acc[t] = fma((double)bf16_bits_to_f32(xv[0] & 0xFFFFu), (double)w4.x, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv[0] >> 16), (double)w4.y, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv[1] & 0xFFFFu), (double)w4.z, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv[1] >> 16), (double)w4.w, acc[t]);
      }
    }
  }
  __shared__ double red[4][kRouterRows];
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
#pragma unroll
  for (int t = 0; t < kRouterRows; ++t) {
    const double v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < nt) {
    const int t = threadIdx.x;
    const double s = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    logits[(size_t)(t0 + t) * E + e] = (float)s;
  }
}

// Candidate order of the top-k: a valid number beats a NaN, which beats an
// unavailable slot (class 2 > 1 > 0); among numbers the larger key wins, and
// equal keys (or two NaNs) go to the lower expert id.
__device__ __forceinline__ bool beats(int c1, float k1, int id1, int c2, float k2, int id2) {
  if (c1 != c2) return c1 > c2;
  if (c1 == 2 && k1 != k2) return k1 > k2;
  return id1 < id2;
}

constexpr int kMaxPerLane = kMaxExperts / MB_WAVE;

// One wave per row: scores, selection keys, top-k (k rounds of a wave-wide
// arg-max), then the route weights.  Lane j writes slot j.
__global__ __launch_bounds__(256) void route_select_kernel(const float *__restrict__ logits,
                                                           const float *__restrict__ bias,
                                                           int32_t *__restrict__ ids,
                                                           float *__restrict__ wts, int rows, int E,
                                                           int k, int scoring, float mult,
                                                           float eps, float route_scale) {
  const int lane = threadIdx.x % MB_WAVE;
  const int t = blockIdx.x * (blockDim.x / MB_WAVE) + threadIdx.x / MB_WAVE;
  if (t >= rows) return;
  const int per = (E + MB_WAVE - 1) / MB_WAVE;
  float g[kMaxPerLane], sc[kMaxPerLane], key[kMaxPerLane];
  bool live[kMaxPerLane];
  float gmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + MB_WAVE * i;
    live[i] = (i < per) && (e < E);
    g[i] = live[i] ? logits[(size_t)t * E + e] * mult : 0.0f;
    if (live[i]) gmax = fmaxf(gmax, g[i]);
  }
  if (scoring == MB_SCORING_SIGMOID) {
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      sc[i] = live[i] ? (float)(1.0 / (1.0 + exp(-(double)g[i]))) : 0.0f;
  } else {
    gmax = wave_max(gmax);
    double z[kMaxPerLane];
    double zs = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      z[i] = live[i] ? exp((double)g[i] - (double)gmax) : 0.0;
      zs += z[i];
    }
    zs = wave_sum(zs);
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) sc[i] = live[i] ? (float)(z[i] / zs) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + MB_WAVE * i;
    key[i] = live[i] ? sc[i] + bias[e] : 0.0f;
  }

  int my_id = 0;
  float my_sc = 0.0f;
  float chosen_sc[kMaxTopK];
  for (int j = 0; j < k; ++j) {
    int bc = 0, bid = 0x7FFFFFFF;
    float bk = 0.0f, bs = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (live[i]) {
        const int e = lane + MB_WAVE * i;
        const int c = isnan(key[i]) ? 1 : 2;
        if (beats(c, key[i], e, bc, bk, bid)) {
          bc = c;
          bk = key[i];
          bid = e;
          bs = sc[i];
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const int oc = __shfl_xor(bc, m, MB_WAVE);
      const float ok = __shfl_xor(bk, m, MB_WAVE);
      const int oid = __shfl_xor(bid, m, MB_WAVE);
      const float os = __shfl_xor(bs, m, MB_WAVE);
      if (beats(oc, ok, oid, bc, bk, bid)) {
        bc = oc;
        bk = ok;
        bid = oid;
        bs = os;
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (live[i] && lane + MB_WAVE * i == bid) live[i] = false;
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj)
      if (jj == j) chosen_sc[jj] = bs;
    if (lane == j) {
      my_id = bid;
      my_sc = bs;
    }
  }
  // fp32, in slot order: sum, + eps, divide, then scale.
  float sum = chosen_sc[0];
#pragma unroll
  for (int jj = 1; jj < kMaxTopK; ++jj)
    if (jj < k) sum = sum + chosen_sc[jj];
  const float den = sum + eps;
  if (lane < k) {
    const float q = my_sc / den;
    const float wv = q * route_scale;
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = wv;
  }
}

// Exclusive prefix sum over the block (blockDim = 1024) in a fixed order;
// `total` receives the sum.  `red` holds 16 entries.
__device__ int block_excl_scan(int v, int *red, int &total) {
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  const int nw = blockDim.x / MB_WAVE;
  int x = v;
#pragma unroll
  for (int o = 1; o < MB_WAVE; o <<= 1) {
    const int y = __shfl_up(x, o, MB_WAVE);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == MB_WAVE - 1) red[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) pre += red[w];
    tot += red[w];
  }
  total = tot;
  return pre + x - v;
}

// Route grouping in one workgroup.  Per expert, a bitmap over rows marks the
// rows that chose it (set with LDS atomics, so the result is independent of
// their order); counts are popcounts; offsets and the active list are
// exclusive scans; route (t, j) of expert e lands at offset[e] + the number of
// earlier rows that chose e, which sorts the routes by (expert, t*k + j).
__global__ __launch_bounds__(1024) void route_group_kernel(const int32_t *__restrict__ ids,
                                                           int rows, int k, int E,
                                                           int32_t *__restrict__ count,
                                                           int32_t *__restrict__ offset,
                                                           int32_t *__restrict__ route_list,
                                                           int32_t *__restrict__ active,
                                                           int32_t *__restrict__ n_active) {
  extern __shared__ unsigned long long bits[];
  __shared__ int s_off[kMaxExperts];
  __shared__ int red[16];
  const int W = (rows + 63) / 64;
  const int R = rows * k;
  for (int i = threadIdx.x; i < E * W; i += blockDim.x) bits[i] = 0ull;
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int t = r / k, e = ids[r];
    if ((unsigned)e < (unsigned)E) atomicOr(&bits[e * W + t / 64], 1ull << (t & 63));
  }
  __syncthreads();
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int w = 0; w < W; ++w) c += __popcll(bits[e * W + w]);
  int total_c = 0, total_a = 0;
  const int ex_c = block_excl_scan(c, red, total_c);
  const int ex_a = block_excl_scan(c > 0 ? 1 : 0, red, total_a);
  if (e < E) {
    count[e] = c;
    offset[e] = ex_c;
    s_off[e] = ex_c;
    if (c > 0) active[ex_a] = e;
  }
  if (threadIdx.x == 0) {
    offset[E] = total_c;
    *n_active = total_a;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int t = r / k, ee = ids[r];
    if ((unsigned)ee >= (unsigned)E) continue;
    const unsigned long long *b = bits + ee * W;
    int rank = 0;
    for (int w = 0; w < t / 64; ++w) rank += __popcll(b[w]);
    rank += __popcll(b[t / 64] & ((1ull << (t & 63)) - 1ull));
    route_list[s_off[ee] + rank] = r;
  }
}

}  // namespace

hipError_t launch_router_logits(const mb_dims &d, const uint16_t *x, const float *router_w,
                                float *logits, hipStream_t s) {
  dim3 grid(d.experts, (d.rows + kRouterRows - 1) / kRouterRows);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, x, router_w, logits, d.rows,
                     d.hidden, d.experts);
  return hipGetLastError();
}

hipError_t launch_route_select(const mb_dims &d, const float *logits, const float *bias,
                               int32_t *ids, float *wts, hipStream_t s) {
  dim3 grid((d.rows + 3) / 4);
  hipLaunchKernelGGL(route_select_kernel, grid, dim3(256), 0, s, logits, bias, ids, wts, d.rows,
                     d.experts, d.top_k, d.scoring, d.router_multiplier, d.division_eps,
                     d.route_scale);
  return hipGetLastError();
}

hipError_t launch_route_group(const mb_dims &d, const int32_t *ids, int32_t *count,
                              int32_t *offset, int32_t *route_list, int32_t *active,
                              int32_t *n_active, hipStream_t s) {
  const size_t lds = (size_t)d.experts * ((d.rows + 63) / 64) * sizeof(unsigned long long);
  hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(1024), lds, s, ids, d.rows, d.top_k,
                     d.experts, count, offset, route_list, active, n_active);
  return hipGetLastError();
}

}  // namespace mb
