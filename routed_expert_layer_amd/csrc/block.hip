// The routed-MoE block as one persistent launch driven by a task list.
//
// The block's steps ([providers] MoEProvider: router, routing, pooler, routed
// experts, tail, unpooler; BoundaryProvider: the boundary; [mono.decoder]
// _K3Bucket runs the whole layer as one launch at small row counts) become
// one ordered list of tasks:
//
//   router     (expert, hidden slice)   fp64 partial logits         [Wr]
//   route      (4 rows)                 top-k and weights (many rows)
//   pool       (16 features, K split)   h = bf16(x Wp^T)            [Wp]
//   prenorm    (row)                    optional RMSNorm of h
//   up         (expert, 16 columns)     act = bf16(silu(g) * u)     [w13]
//   down       (expert, 32 features)    y, per-tile sums of squares [w2]
//   finalize   (row, 512 features)      moe_out = bf16(sum_j w_j yn_j)
//   unpool     (16 features, K split)   u = bf16(moe_out Wu^T)      [Wu]
//   boundary   (row)                    stream, x_next
//
// Workgroup w runs tasks w, w + G, w + 2G, ... in order (G workgroups, two
// per CU, all resident: a cooperative launch).  A task waits only for the
// tasks whose output it reads, through per-launch counters: up waits for the
// pooler, down for the up tasks of its own expert, finalize for the down
// tasks of its row's experts, unpool for all finalize tasks, boundary for all
// unpool tiles.  Every dependency points to a lower task index, so the lowest
// unfinished task can always run and the launch always completes; every wait
// is also bounded (mb_sync.h).  Imbalance in one step is absorbed by the next
// step's tasks instead of stalling every workgroup at a barrier.
//
// Routing state (ids, weights, route grouping) is rebuilt in each
// workgroup's LDS from the logits (few rows) or from the route tasks' ids.
//
// Data one workgroup hands to another goes through coherent (sc1) buffer
// accesses; weights are streamed with non-temporal loads.  Arithmetic:
// fp64-accumulated router logits rounded once to fp32, the fp32 routing
// recipe, bf16 MFMA with exact MXFP4 -> bf16 weight conversion and fp32
// accumulation, fixed-order reductions (results do not depend on timing).

#include "mb_block.h"
#include "mb_device.h"
#include "mb_sync.h"

// Each task is its own (non-inlined) function so that the register
// allocation of one step's inner loop is not constrained by the others'.

namespace mb {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MB_WAVE;
constexpr int kPoolMG = 4;      // 16-row groups per projection pass
constexpr int kRouterRows = 8;  // rows per pass of a router task

struct Lane {
  int lane, wave, g, r16;
  __device__ Lane()
      : lane(threadIdx.x % MB_WAVE), wave(threadIdx.x / MB_WAVE), g((threadIdx.x % MB_WAVE) >> 4),
        r16(threadIdx.x & 15) {}
};

// ---------------------------------------------------------------- dependencies

struct Deps {
  unsigned *words;  // [0] epoch, [1] abort
  unsigned *set;    // this launch's counters
  int E;

  __device__ unsigned *ctr(int slot) const { return set + slot * kCtrStride; }
  __device__ unsigned *up(int e) const { return ctr(kCtrUp + e); }
  __device__ unsigned *down(int e) const { return ctr(kCtrUp + E + e); }
};

// This launch uses counter set (epoch & 1); workgroup 0 clears the other set
// for the next launch (the last workgroup to finish bumps the epoch).
__device__ __forceinline__ Deps deps_init(const BlockParams &p) {
  Deps d;
  d.words = p.sync;
  d.E = p.E;
  const unsigned epoch = __hip_atomic_load(&p.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n = kCtrUp + 2 * p.E;
  d.set = p.sync + kSyncHeader + (epoch & 1u) * n * kCtrStride;
  unsigned *other = p.sync + kSyncHeader + ((epoch & 1u) ^ 1u) * n * kCtrStride;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n; i += kThreads)
      __hip_atomic_store(&other[i * kCtrStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return d;
}

// All coherent stores of this workgroup complete, then one increment.
__device__ __forceinline__ void signal(unsigned *c) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0: each lane polls its own counter until every lane's has reached
// `target`.  Bounded: on timeout the abort word is raised, and any wait that
// sees it returns at once, so the launch drains.
__device__ __forceinline__ void poll_ge(const Deps &d, const unsigned *mine, unsigned target) {
  const int lane = threadIdx.x % MB_WAVE;
  unsigned spins = 0;
  while (true) {
    const unsigned have = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all((int)(have >= target))) return;
    if ((++spins & 255u) == 0) {
      if (__hip_atomic_load(&d.words[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
      if (spins > kSpinLimit) {
        if (lane == 0) __hip_atomic_store(&d.words[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ void wait_ge(const Deps &d, const unsigned *c, unsigned target) {
  if (target == 0) return;
  if (threadIdx.x < MB_WAVE) poll_ge(d, c, target);
  __syncthreads();
}

// ---------------------------------------------------------------- router

// Partial logits of expert e over hidden slice s for every row, in fp64
// (bf16 x fp32 products are exact in fp64).  Each thread takes 4 consecutive
// elements per 1024-element pass of the slice for up to 16 rows at a time;
// the row sums are then reduced over the workgroup in a fixed order.
__device__ __noinline__ void router_task(const BlockParams &p, const Deps &d, int task,
                                            unsigned char *lds) {
  const Lane L;
  const int e = task / p.rslices, s = task % p.rslices;
  const int h_begin = s * p.rslice, h_end = min(p.H, h_begin + p.rslice);
  const rsrc_t part = make_rsrc(p.logit_part);
  double *red = reinterpret_cast<double *>(lds);  // [kWaves][kRouterRows]
  for (int t0 = 0; t0 < p.b; t0 += kRouterRows) {
    double acc[kRouterRows];
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r) acc[r] = 0.0;
    for (int h = h_begin + threadIdx.x * 4; h < h_end; h += kThreads * 4) {
      const f32x4_t w = *reinterpret_cast<const f32x4_t *>(p.router_w + (size_t)e * p.H + h);
      u32x2_t xv[kRouterRows];
#pragma unroll
      for (int r = 0; r < kRouterRows; ++r)
        xv[r] = t0 + r < p.b ? *reinterpret_cast<const u32x2_t *>(p.x + (size_t)(t0 + r) * p.H + h)
                             : u32x2_t{0, 0};
#pragma unroll
      for (int r = 0; r < kRouterRows; ++r) {
        acc[r] = fma((double)bf16_bits_to_f32(xv[r][0] & 0xFFFFu), (double)w[0], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[r][0] >> 16), (double)w[1], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[r][1] & 0xFFFFu), (double)w[2], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[r][1] >> 16), (double)w[3], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r) {
      const double v = wave_sum(acc[r]);
      if (L.lane == 0) red[L.wave * kRouterRows + r] = v;
    }
    __syncthreads();
    const int r = threadIdx.x;
    if (r < kRouterRows && t0 + r < p.b) {
      double v = red[r];
      for (int q = 1; q < kWaves; ++q) v += red[q * kRouterRows + r];
      st_co8(part, (uint32_t)((((size_t)s * p.b + t0 + r) * p.E + e) * 8), __builtin_bit_cast(u32x2_t, v));
    }
    __syncthreads();
  }
  signal(d.ctr(kCtrLogits));
}

// ---------------------------------------------------------------- routing

// Candidate order of the top-k: a valid number beats a NaN, which beats an
// unavailable slot; larger keys first; equal keys (or two NaNs) to the lower id.
__device__ __forceinline__ bool beats(int c1, float k1, int id1, int c2, float k2, int id2) {
  if (c1 != c2) return c1 > c2;
  if (c1 == 2 && k1 != k2) return k1 > k2;
  return id1 < id2;
}

// fp32 logit (t, e): the fp64 slice partials added in slice order, or given.
__device__ __forceinline__ float logit_of(const BlockParams &p, rsrc_t part, int t, int e) {
  if (p.logits_in) return p.logits[(size_t)t * p.E + e];
  double acc = __builtin_bit_cast(double, ld_co8(part, (uint32_t)(((size_t)t * p.E + e) * 8)));
  for (int s = 1; s < p.rslices; ++s)
    acc += __builtin_bit_cast(double, ld_co8(part, (uint32_t)((((size_t)s * p.b + t) * p.E + e) * 8)));
  return (float)acc;
}

// One row's routing by one wave from its fp32 logits l[i] (expert lane + 64 i):
// multiplier, scores, keys = score + bias, k rounds of a wave-wide arg-max,
// then the fp32 weights in slot order.  Lane j < k gets slot j.
template <int PER>
__device__ __forceinline__ void route_one(const BlockParams &p, const float (&l)[PER], int &out_id,
                                          float &out_w) {
  const int lane = threadIdx.x % MB_WAVE;
  float g[PER], sc[PER], key[PER];
  bool live[PER];
  float gmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    live[i] = lane + MB_WAVE * i < p.E;
    g[i] = l[i] * p.mult;
    if (live[i]) gmax = fmaxf(gmax, g[i]);
  }
  if (p.scoring == MB_SCORING_SIGMOID) {
#pragma unroll
    for (int i = 0; i < PER; ++i) sc[i] = live[i] ? (float)(1.0 / (1.0 + exp(-(double)g[i]))) : 0.0f;
  } else {
    gmax = wave_max(gmax);
    double z[PER];
    double zs = 0.0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      z[i] = live[i] ? exp((double)g[i] - (double)gmax) : 0.0;
      zs += z[i];
    }
    zs = wave_sum(zs);
#pragma unroll
    for (int i = 0; i < PER; ++i) sc[i] = live[i] ? (float)(z[i] / zs) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i)
    key[i] = live[i] ? sc[i] + p.bias[min(lane + MB_WAVE * i, p.E - 1)] : 0.0f;

  out_id = 0;
  float my_sc = 0.0f;
  float chosen[kMaxTopK];
  for (int j = 0; j < p.k; ++j) {
    int bc = 0, bid = 0x7FFFFFFF;
    float bk = 0.0f, bs = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
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
    for (int i = 0; i < PER; ++i)
      if (live[i] && lane + MB_WAVE * i == bid) live[i] = false;
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj)
      if (jj == j) chosen[jj] = bs;
    if (lane == j) {
      out_id = bid;
      my_sc = bs;
    }
  }
  float sum = chosen[0];
#pragma unroll
  for (int jj = 1; jj < kMaxTopK; ++jj)
    if (jj < p.k) sum = sum + chosen[jj];
  const float den = sum + p.div_eps;
  const float q = my_sc / den;
  out_w = q * p.route_scale;
}

// Rows t_begin..t_end-1, one per wave in turn: logits from `lg` (LDS
// [rows][E], row t_begin first) when given, else from the partials; results
// to LDS and, when `out`, to the outputs.
template <int PER>
__device__ __forceinline__ void route_rows(const BlockParams &p, const RouteLds &R, const float *lg,
                                           int t_begin, int t_end, bool out) {
  const int lane = threadIdx.x % MB_WAVE;
  const rsrc_t part = make_rsrc(p.logit_part);
  for (int t = t_begin + threadIdx.x / MB_WAVE; t < t_end; t += kWaves) {
    float l[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + MB_WAVE * i;
      l[i] = 0.f;
      if (e < p.E) l[i] = lg ? lg[(size_t)(t - t_begin) * p.E + e] : logit_of(p, part, t, e);
    }
    int id;
    float w;
    route_one<PER>(p, l, id, w);
    if (lane < p.k) {
      R.ids[t * p.k + lane] = id;
      R.w[t * p.k + lane] = w;
      if (out) {
        p.ids[(size_t)t * p.k + lane] = id;
        p.wts[(size_t)t * p.k + lane] = w;
      }
    }
  }
}

__device__ __forceinline__ void route_dispatch(const BlockParams &p, const RouteLds &R, const float *lg,
                                               int t0, int t1, bool out) {
  // The host sends larger expert counts to the per-step kernels.
  if (p.E <= 64) route_rows<1>(p, R, lg, t0, t1, out);
  else if (p.E <= 128) route_rows<2>(p, R, lg, t0, t1, out);
  else route_rows<4>(p, R, lg, t0, t1, out);
}

// Exclusive prefix sum over the workgroup of one value per thread, in a fixed
// order; `total` receives the sum.  `red` holds kWaves ints.
__device__ __forceinline__ int wg_excl_scan(int v, int *red, int &total) {
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
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
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) pre += red[w];
    tot += red[w];
  }
  total = tot;
  return pre + x - v;
}

// Route grouping from R.ids: per-expert bitmaps over rows (LDS atomics, so
// independent of order), popcount counts, exclusive scans for offsets and
// the active list, and route (t, j) of expert e at offset[e] + the number of
// earlier rows that chose e (routes sorted by (expert, t*k + j)).
__device__ __forceinline__ void group_routes(const BlockParams &p, const RouteLds &R, bool out) {
  const int W = (p.b + 63) / 64;
  const int Rn = p.b * p.k;
  for (int i = threadIdx.x; i < p.E * W; i += kThreads) R.bits[i] = 0ull;
  __syncthreads();
  for (int r = threadIdx.x; r < Rn; r += kThreads) {
    const int t = r / p.k, e = R.ids[r];
    atomicOr(&R.bits[e * W + t / 64], 1ull << (t & 63));
  }
  __syncthreads();
  const int e0 = threadIdx.x * 4;
  int c[4], csum = 0, asum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = 0;
    const int e = e0 + q;
    if (e < p.E)
      for (int w = 0; w < W; ++w) c[q] += __popcll(R.bits[e * W + w]);
    csum += c[q];
    asum += c[q] > 0 ? 1 : 0;
  }
  int tot_c = 0, tot_a = 0;
  int oc = wg_excl_scan(csum, R.red, tot_c);
  int oa = wg_excl_scan(asum, R.red, tot_a);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = e0 + q;
    if (e < p.E) {
      R.off[e] = oc;
      if (out) {
        p.count[e] = c[q];
        p.offset[e] = oc;
      }
      if (c[q] > 0) {
        R.act[oa] = e;
        if (out) p.active[oa] = e;
        ++oa;
      }
      oc += c[q];
    }
  }
  if (threadIdx.x == 0) {
    R.off[p.E] = tot_c;
    *R.nact = tot_a;
    if (out) {
      p.offset[p.E] = tot_c;
      *p.n_active = tot_a;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < Rn; r += kThreads) {
    const int t = r / p.k, e = R.ids[r];
    const unsigned long long *b = R.bits + e * W;
    int rank = 0;
    for (int w = 0; w < t / 64; ++w) rank += __popcll(b[w]);
    rank += __popcll(b[t / 64] & ((1ull << (t & 63)) - 1ull));
    R.rl[R.off[e] + rank] = r;
    if (out) p.route_list[R.off[e] + rank] = r;
  }
  __syncthreads();
}

// Route task (many rows): rows 4 task .. +3, one per wave; their ids and
// weights go out coherently for every workgroup's grouping.
__device__ __noinline__ void route_task(const BlockParams &p, const Deps &d, const RouteLds &R,
                                           int task) {
  wait_ge(d, d.ctr(kCtrLogits), (unsigned)p.n_router);
  const int t0 = task * kWaves, t1 = min(p.b, t0 + kWaves);
  route_dispatch(p, R, nullptr, t0, t1, false);
  __syncthreads();
  const rsrc_t ri = make_rsrc(p.ids), rw = make_rsrc(p.wts);
  for (int i = threadIdx.x; i < (t1 - t0) * p.k; i += kThreads) {
    const int r = t0 * p.k + i;
    st_co4(ri, (uint32_t)(r * 4), (uint32_t)R.ids[r]);
    st_co4(rw, (uint32_t)(r * 4), __float_as_uint(R.w[r]));
  }
  if (p.logits && !p.logits_in) {
    const rsrc_t part = make_rsrc(p.logit_part);
    for (int i = threadIdx.x; i < (t1 - t0) * p.E; i += kThreads) {
      const int t = t0 + i / p.E, e = i % p.E;
      p.logits[(size_t)t * p.E + e] = logit_of(p, part, t, e);
    }
  }
  signal(d.ctr(kCtrRoute));
}

// The routing state a workgroup needs before its first expert task.
__device__ __noinline__ void prepare_routing(const BlockParams &p, const Deps &d, const RouteLds &R,
                                                unsigned char *scratch) {
  const bool out = p.routing_out && blockIdx.x == 0;
  if (p.route_given) {
    // From the caller (mb_experts).
    for (int i = threadIdx.x; i < p.b * p.k; i += kThreads) {
      R.ids[i] = p.ids[i];
      R.w[i] = p.wts[i];
      R.rl[i] = p.route_list[i];
    }
    for (int i = threadIdx.x; i <= p.E; i += kThreads) R.off[i] = p.offset[i];
    for (int i = threadIdx.x; i < p.E; i += kThreads) R.act[i] = p.active[i];
    if (threadIdx.x == 0) *R.nact = *p.n_active;
    __syncthreads();
    return;
  }
  if (p.n_route == 0) {
    // Few rows: every workgroup routes every row from logits staged in LDS.
    wait_ge(d, d.ctr(kCtrLogits), (unsigned)p.n_router);
    float *lg = reinterpret_cast<float *>(scratch);
    const rsrc_t part = make_rsrc(p.logit_part);
    for (int i = threadIdx.x; i < p.b * p.E; i += kThreads) lg[i] = logit_of(p, part, i / p.E, i % p.E);
    __syncthreads();
    route_dispatch(p, R, lg, 0, p.b, out);
    if (out && p.logits && !p.logits_in)
      for (int i = threadIdx.x; i < p.b * p.E; i += kThreads) p.logits[i] = lg[i];
  } else {
    wait_ge(d, d.ctr(kCtrRoute), (unsigned)p.n_route);
    const rsrc_t ri = make_rsrc(p.ids), rw = make_rsrc(p.wts);
    for (int i = threadIdx.x; i < p.b * p.k; i += kThreads) {
      R.ids[i] = (int)ld_co4(ri, (uint32_t)(i * 4));
      R.w[i] = __uint_as_float(ld_co4(rw, (uint32_t)(i * 4)));
    }
  }
  __syncthreads();
  group_routes(p, R, out);
}

// ---------------------------------------------------------------- projections

// One task of out[t, n] = bf16(sum_k a[t, k] w[n, k]): a 16-feature tile and
// contraction split ks of ks_count, the split's 32-element chunks dealt to the
// four waves; 16-row groups of activations share each weight fragment (weights
// in the MFMA A operand, activations in B).  The first weight fragments are
// requested before waiting for `a` (wait_ctr).  With ks_count > 1 the fp32
// partials go to `part` and the last split to finish (tile counter) adds them
// in split order and writes bf16.  Returns true in the workgroup that
// completed the tile.
__device__ __noinline__ bool proj_task(const Deps &d, const uint16_t *a, bool a_coherent,
                                          const uint16_t *w, uint16_t *out, int rows, int n_out,
                                          int kdim, int ks_count, float *part, unsigned *tile_ctr,
                                          const unsigned *wait_ctr, unsigned wait_target, int task,
                                          unsigned char *lds) {
  const Lane L;
  const int nchunks = kdim / 32;
  const int cpw = (nchunks + ks_count - 1) / ks_count;
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [kWaves][kPoolMG][64]
  int *s_last = reinterpret_cast<int *>(lds + kWaves * kPoolMG * MB_WAVE * sizeof(f32x4_t));
  const rsrc_t ra = make_rsrc(a), ro = make_rsrc(out), rp = make_rsrc(part);
  const int tile = task / ks_count, ks = task % ks_count;
  const int c_begin = ks * cpw, c_end = min(nchunks, c_begin + cpw);
  const uint16_t *wrow = w + (size_t)(tile * 16 + L.r16) * kdim + 8 * L.g;
  bool waited = false;
  for (int rb = 0; rb < rows; rb += 16 * kPoolMG) {
    f32x4_t acc[kPoolMG];
#pragma unroll
    for (int mg = 0; mg < kPoolMG; ++mg) acc[mg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t wv[4];
    const int c_first = c_begin + L.wave;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c_first + kWaves * u;
      wv[u] = cc < c_end ? ld16_nt(wrow + cc * 32) : u32x4_t{0, 0, 0, 0};
    }
    if (!waited) {
      wait_ge(d, wait_ctr, wait_target);
      waited = true;
    }
    for (int c = c_first; c < c_end; c += kWaves * 4) {
      if (c != c_first) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c + kWaves * u;
          wv[u] = cc < c_end ? ld16_nt(wrow + cc * 32) : u32x4_t{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int mg = 0; mg < kPoolMG; ++mg) {
        const int t = rb + mg * 16 + L.r16;
        if (rb + mg * 16 >= rows) break;
        u32x4_t av[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c + kWaves * u;
          const size_t off = (size_t)t * kdim + cc * 32 + 8 * L.g;
          if (cc < c_end && t < rows)
            av[u] = a_coherent ? ld_co16(ra, (uint32_t)(off * 2)) : ld16(a + off);
          else
            av[u] = u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c + kWaves * u < c_end) acc[mg] = mfma_bf16(as_bf16x8(wv[u]), as_bf16x8(av[u]), acc[mg]);
      }
    }
#pragma unroll
    for (int mg = 0; mg < kPoolMG; ++mg) red[(L.wave * kPoolMG + mg) * MB_WAVE + L.lane] = acc[mg];
    __syncthreads();
    for (int mg = L.wave; mg < kPoolMG; mg += kWaves) {
      const int t = rb + mg * 16 + L.r16;
      if (t >= rows) continue;
      f32x4_t v = red[(0 * kPoolMG + mg) * MB_WAVE + L.lane];
      for (int q = 1; q < kWaves; ++q) v += red[(q * kPoolMG + mg) * MB_WAVE + L.lane];
      const int n0 = tile * 16 + 4 * L.g;
      if (ks_count == 1)
        st_co8(ro, (uint32_t)(((size_t)t * n_out + n0) * 2),
               u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      else
        st_co16(rp, (uint32_t)((((size_t)ks * rows + t) * n_out + n0) * 4), __builtin_bit_cast(u32x4_t, v));
    }
    __syncthreads();
  }
  if (ks_count == 1) return true;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_last = __hip_atomic_fetch_add(&tile_ctr[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(ks_count - 1);
  __syncthreads();
  const bool last = *s_last != 0;
  if (last) {
    for (int idx = threadIdx.x; idx < rows * 4; idx += kThreads) {
      const int t = idx / 4, n0 = tile * 16 + 4 * (idx % 4);
      f32x4_t v = __builtin_bit_cast(f32x4_t, ld_co16(rp, (uint32_t)(((size_t)t * n_out + n0) * 4)));
      for (int q = 1; q < ks_count; ++q)
        v += __builtin_bit_cast(f32x4_t, ld_co16(rp, (uint32_t)((((size_t)q * rows + t) * n_out + n0) * 4)));
      st_co8(ro, (uint32_t)(((size_t)t * n_out + n0) * 2),
             u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    }
    if (threadIdx.x == 0) __hip_atomic_store(&tile_ctr[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last;
}

// Optional pre-expert norm of h row t.
__device__ __noinline__ void prenorm_task(const BlockParams &p, const Deps &d, int t,
                                             unsigned char *lds) {
  wait_ge(d, d.ctr(kCtrPool), (unsigned)p.n_pool_tiles);
  float *red = reinterpret_cast<float *>(lds);
  const rsrc_t rh = make_rsrc(p.h);
  float ss = 0.f;
  for (int i = threadIdx.x * 2; i < p.P; i += kThreads * 2) {
    const uint32_t v = ld_co4(rh, (uint32_t)(((size_t)t * p.P + i) * 2));
    const float a = bf16_bits_to_f32(v & 0xFFFFu), b = bf16_bits_to_f32(v >> 16);
    ss += a * a + b * b;
  }
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)p.P + p.norm_eps);
  for (int i = threadIdx.x * 2; i < p.P; i += kThreads * 2) {
    const uint32_t v = ld_co4(rh, (uint32_t)(((size_t)t * p.P + i) * 2));
    const float a = bf16_bits_to_f32(v & 0xFFFFu) * rs, b = bf16_bits_to_f32(v >> 16) * rs;
    const float wa = bf16_bits_to_f32(p.pre_norm_w[i]), wb = bf16_bits_to_f32(p.pre_norm_w[i + 1]);
    st_co4(rh, (uint32_t)(((size_t)t * p.P + i) * 2), pack_bf16x2(a * wa, b * wb));
  }
  signal(d.ctr(kCtrPrenorm));
}

// ---------------------------------------------------------------- experts

// w13 + gated activation for (active expert, 16 act columns): gate rows
// i0..i0+15 and up rows I+i0..I+i0+15, contraction over P in 128-element
// chunks dealt to the waves; per chunk a lane converts one 32-element MXFP4
// block (16 bytes + a scale byte) of its weight row to bf16 for four MFMAs.
__device__ __noinline__ void up_task(const BlockParams &p, const Deps &d, const RouteLds &R,
                                        int task, bool &h_ready, unsigned char *lds) {
  const Lane L;
  const int P = p.P, I = p.I;
  const int tiles = I / 16;
  const int nch = P / 128;
  const rsrc_t rh = make_rsrc(p.h), ract = make_rsrc(p.act);
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [kWaves][2][64]
  const int a = task / tiles, tile = task % tiles;
  const int e = R.act[a];
  const int row0 = R.off[e], nrows = R.off[e + 1] - row0;
  const int i0 = tile * 16;
  const size_t rg = (size_t)e * 2 * I + i0 + L.r16, ru = rg + I;
  const uint8_t *wg = p.w13 + rg * (P / 2) + 16 * L.g;
  const uint8_t *wu = p.w13 + ru * (P / 2) + 16 * L.g;
  const uint8_t *sg = p.w13s + rg * (P / 32) + L.g;
  const uint8_t *su = p.w13s + ru * (P / 32) + L.g;
  for (int m0 = 0; m0 < nrows; m0 += 16) {
    const int m = m0 + L.r16;
    const bool valid = m < nrows;
    const int t = valid ? R.rl[row0 + m] / p.k : 0;
    const uint32_t hoff = (uint32_t)(((size_t)t * P + 32 * L.g) * 2);
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    u32x4_t vg[4], vu[4];
    uint32_t bg[4], bu[4];
    const int c_first = L.wave;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c_first + kWaves * u;
      const bool ok = cc < nch;
      vg[u] = ok ? ld16_nt(wg + 64 * cc) : u32x4_t{0, 0, 0, 0};
      vu[u] = ok ? ld16_nt(wu + 64 * cc) : u32x4_t{0, 0, 0, 0};
      bg[u] = ok ? sg[4 * cc] : 0u;
      bu[u] = ok ? su[4 * cc] : 0u;
    }
    if (!h_ready) {
      wait_ge(d, d.ctr(p.pre_norm_w ? kCtrPrenorm : kCtrPool), (unsigned)p.h_producers);
      h_ready = true;
    }
    for (int c = c_first; c < nch; c += kWaves * 4) {
      if (c != c_first) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c + kWaves * u;
          const bool ok = cc < nch;
          vg[u] = ok ? ld16_nt(wg + 64 * cc) : u32x4_t{0, 0, 0, 0};
          vu[u] = ok ? ld16_nt(wu + 64 * cc) : u32x4_t{0, 0, 0, 0};
          bg[u] = ok ? sg[4 * cc] : 0u;
          bu[u] = ok ? su[4 * cc] : 0u;
        }
      }
      u32x4_t hv[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = c + kWaves * u;
        const bool ok = cc < nch && valid;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hv[u][i] = ok ? ld_co16(rh, hoff + (uint32_t)((128 * cc + 8 * i) * 2)) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c + kWaves * u < nch) {
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
    red[(L.wave * 2 + 0) * MB_WAVE + L.lane] = ag;
    red[(L.wave * 2 + 1) * MB_WAVE + L.lane] = au;
    __syncthreads();
    if (L.wave == 0 && valid) {
      f32x4_t gs = red[0 * MB_WAVE + L.lane], us = red[1 * MB_WAVE + L.lane];
      for (int q = 1; q < kWaves; ++q) {
        gs += red[(q * 2 + 0) * MB_WAVE + L.lane];
        us += red[(q * 2 + 1) * MB_WAVE + L.lane];
      }
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = gs[i];
        o[i] = (z / (1.0f + expf(-z))) * us[i];
      }
      st_co8(ract, (uint32_t)((((size_t)(row0 + m)) * I + i0 + 4 * L.g) * 2),
             u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
    }
    __syncthreads();
  }
  signal(d.up(e));
}

// w2 for (active expert, 32 output features): y in route order and the
// route's sum of squares over these 32 features.
__device__ __noinline__ void down_task(const BlockParams &p, const Deps &d, const RouteLds &R,
                                          int task, unsigned char *lds) {
  const Lane L;
  const int P = p.P, I = p.I;
  const int tiles = P / 32;
  const int nch = I / 128;
  const rsrc_t ract = make_rsrc(p.act), ry = make_rsrc(p.y), rss = make_rsrc(p.ssq);
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [kWaves][2][64]
  const int a = task / tiles, tile = task % tiles;
  const int e = R.act[a];
  const int row0 = R.off[e], nrows = R.off[e + 1] - row0;
  const int p0 = tile * 32;
  const size_t r0 = (size_t)e * P + p0 + L.r16, r1 = r0 + 16;
  const uint8_t *w0 = p.w2 + r0 * (I / 2) + 16 * L.g;
  const uint8_t *w1 = p.w2 + r1 * (I / 2) + 16 * L.g;
  const uint8_t *s0 = p.w2s + r0 * (I / 32) + L.g;
  const uint8_t *s1 = p.w2s + r1 * (I / 32) + L.g;
  bool ready = false;
  for (int m0 = 0; m0 < nrows; m0 += 16) {
    const int m = m0 + L.r16;
    const bool valid = m < nrows;
    const uint32_t aoff = (uint32_t)((((size_t)(row0 + (valid ? m : 0))) * I + 32 * L.g) * 2);
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    u32x4_t v0[4], v1[4];
    uint32_t b0[4], b1[4];
    const int c_first = L.wave;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cc = c_first + kWaves * u;
      const bool ok = cc < nch;
      v0[u] = ok ? ld16_nt(w0 + 64 * cc) : u32x4_t{0, 0, 0, 0};
      v1[u] = ok ? ld16_nt(w1 + 64 * cc) : u32x4_t{0, 0, 0, 0};
      b0[u] = ok ? s0[4 * cc] : 0u;
      b1[u] = ok ? s1[4 * cc] : 0u;
    }
    if (!ready) {
      wait_ge(d, d.up(e), p.has_up ? (unsigned)(I / 16) : 0u);
      ready = true;
    }
    for (int c = c_first; c < nch; c += kWaves * 4) {
      if (c != c_first) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cc = c + kWaves * u;
          const bool ok = cc < nch;
          v0[u] = ok ? ld16_nt(w0 + 64 * cc) : u32x4_t{0, 0, 0, 0};
          v1[u] = ok ? ld16_nt(w1 + 64 * cc) : u32x4_t{0, 0, 0, 0};
          b0[u] = ok ? s0[4 * cc] : 0u;
          b1[u] = ok ? s1[4 * cc] : 0u;
        }
      }
      u32x4_t av[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cc = c + kWaves * u;
        const bool ok = cc < nch && valid;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[u][i] = ok ? ld_co16(ract, aoff + (uint32_t)((128 * cc + 8 * i) * 2)) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c + kWaves * u < nch) {
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
    red[(L.wave * 2 + 0) * MB_WAVE + L.lane] = a0;
    red[(L.wave * 2 + 1) * MB_WAVE + L.lane] = a1;
    __syncthreads();
    if (L.wave == 0) {
      f32x4_t y0 = red[0 * MB_WAVE + L.lane], y1 = red[1 * MB_WAVE + L.lane];
      for (int q = 1; q < kWaves; ++q) {
        y0 += red[(q * 2 + 0) * MB_WAVE + L.lane];
        y1 += red[(q * 2 + 1) * MB_WAVE + L.lane];
      }
      float ss = 0.f;
      if (valid) {
        ss = y0[0] * y0[0] + y0[1] * y0[1] + y0[2] * y0[2] + y0[3] * y0[3];
        ss += y1[0] * y1[0] + y1[1] * y1[1] + y1[2] * y1[2] + y1[3] * y1[3];
      }
      ss += __shfl_xor(ss, 16, MB_WAVE);
      ss += __shfl_xor(ss, 32, MB_WAVE);
      if (valid) {
        const int r = R.rl[row0 + m];
        st_co16(ry, (uint32_t)(((size_t)r * P + p0 + 4 * L.g) * 4), __builtin_bit_cast(u32x4_t, y0));
        st_co16(ry, (uint32_t)(((size_t)r * P + p0 + 16 + 4 * L.g) * 4), __builtin_bit_cast(u32x4_t, y1));
        if (L.g == 0) st_co4(rss, (uint32_t)(((size_t)r * tiles + tile) * 4), __float_as_uint(ss));
      }
    }
    __syncthreads();
  }
  signal(d.down(e));
}

// ---------------------------------------------------------------- tail

// moe_out[t, p] = bf16(sum_j (w_j / sqrt(ss_j / P + eps)) y_j[p] * w_post[p]),
// ss_j = the route's per-tile sums of squares added in tile order, for the
// task's features of row t; waits for the down tasks of the row's experts.
__device__ __noinline__ void fin_task(const BlockParams &p, const Deps &d, const RouteLds &R,
                                         int task, unsigned char *lds) {
  const int P = p.P, k = p.k;
  const int tiles = P / 32;
  const int chunks = (P + kFinChunk - 1) / kFinChunk;
  const int t = task / chunks, p_begin = (task % chunks) * kFinChunk;
  const int p_end = min(P, p_begin + kFinChunk);
  const int lane = threadIdx.x % MB_WAVE, wave = threadIdx.x / MB_WAVE;
  if (p.has_up) {
    if (threadIdx.x < MB_WAVE) poll_ge(d, d.down(R.ids[t * k + (lane < k ? lane : 0)]), (unsigned)tiles);
    __syncthreads();
  }
  float *coef = reinterpret_cast<float *>(lds);  // [k]
  const rsrc_t rss = make_rsrc(p.ssq), ry = make_rsrc(p.y), ro = make_rsrc(p.moe_out);
  for (int j = wave; j < k; j += kWaves) {
    const int r = t * k + j;
    float s = 0.f;
    for (int c = lane; c < tiles; c += MB_WAVE)
      s += __uint_as_float(ld_co4(rss, (uint32_t)(((size_t)r * tiles + c) * 4)));
    s = wave_sum(s);
    if (lane == 0) coef[j] = R.w[r] * (1.0f / sqrtf(s / (float)P + p.norm_eps));
  }
  __syncthreads();
  for (int p4 = p_begin + threadIdx.x * 4; p4 < p_end; p4 += kThreads * 4) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const f32x4_t yv =
          __builtin_bit_cast(f32x4_t, ld_co16(ry, (uint32_t)(((size_t)(t * k + j) * P + p4) * 4)));
      acc += coef[j] * yv;
    }
    const u32x2_t pw = *reinterpret_cast<const u32x2_t *>(p.post_norm_w + p4);
    const float o0 = acc[0] * bf16_bits_to_f32(pw[0] & 0xFFFFu);
    const float o1 = acc[1] * bf16_bits_to_f32(pw[0] >> 16);
    const float o2 = acc[2] * bf16_bits_to_f32(pw[1] & 0xFFFFu);
    const float o3 = acc[3] * bf16_bits_to_f32(pw[1] >> 16);
    st_co8(ro, (uint32_t)(((size_t)t * P + p4) * 2), u32x2_t{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)});
  }
  signal(d.ctr(kCtrFin));
}

// ---------------------------------------------------------------- boundary

__device__ __forceinline__ void unpack4(u32x2_t v, float o[4]) {
  o[0] = bf16_bits_to_f32(v[0] & 0xFFFFu);
  o[1] = bf16_bits_to_f32(v[0] >> 16);
  o[2] = bf16_bits_to_f32(v[1] & 0xFFFFu);
  o[3] = bf16_bits_to_f32(v[1] >> 16);
}

// v = RMSNorm_H(u) * w_pff; stream = fp32(stream + g * v) (one fma);
// x_next = bf16(RMSNorm_H(stream) * w_in), for row t.
__device__ __noinline__ void boundary_task(const BlockParams &p, const Deps &d, int t,
                                              unsigned char *lds) {
  wait_ge(d, d.ctr(kCtrUnpool), (unsigned)p.n_unpool_tiles);
  float *red = reinterpret_cast<float *>(lds);
  const int H = p.H;
  const rsrc_t ru = make_rsrc(p.u);
  float *srow = p.stream + (size_t)t * H;
  float ss = 0.f;
  for (int h = threadIdx.x * 4; h < H; h += kThreads * 4) {
    float v[4];
    unpack4(ld_co8(ru, (uint32_t)(((size_t)t * H + h) * 2)), v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = block_sum(ss, red);
  const float rsu = 1.0f / sqrtf(ss / (float)H + p.norm_eps);
  float s2 = 0.f;
  for (int h = threadIdx.x * 4; h < H; h += kThreads * 4) {
    float v[4], gg[4], wf[4] = {1.f, 1.f, 1.f, 1.f};
    unpack4(ld_co8(ru, (uint32_t)(((size_t)t * H + h) * 2)), v);
    unpack4(*reinterpret_cast<const u32x2_t *>(p.gate + h), gg);
    if (p.ffn_norm_w) unpack4(*reinterpret_cast<const u32x2_t *>(p.ffn_norm_w + h), wf);
    f32x4_t s = *reinterpret_cast<const f32x4_t *>(srow + h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float vn = v[i] * rsu * wf[i];
      s[i] = fmaf(gg[i], vn, s[i]);
      s2 += s[i] * s[i];
    }
    *reinterpret_cast<f32x4_t *>(srow + h) = s;
  }
  s2 = block_sum(s2, red);
  const float rss = 1.0f / sqrtf(s2 / (float)H + p.norm_eps);
  for (int h = threadIdx.x * 4; h < H; h += kThreads * 4) {
    float wi[4] = {1.f, 1.f, 1.f, 1.f};
    if (p.next_norm_w) unpack4(*reinterpret_cast<const u32x2_t *>(p.next_norm_w + h), wi);
    const f32x4_t s = *reinterpret_cast<const f32x4_t *>(srow + h);
    *reinterpret_cast<u32x2_t *>(p.x_next + (size_t)t * H + h) =
        u32x2_t{pack_bf16x2(s[0] * rss * wi[0], s[1] * rss * wi[1]),
                pack_bf16x2(s[2] * rss * wi[2], s[3] * rss * wi[3])};
  }
  __syncthreads();
}

// ---------------------------------------------------------------- the kernel

// Tracing: workgroup thread 0 stamps the 100 MHz real-time counter at the
// start (slot 0), when routing is ready (5), when it enters its first task of
// each step (1..10 by step) and at the end (15).
__device__ __forceinline__ void stamp(const BlockParams &p, int slot) {
  if (p.timeline && threadIdx.x == 0)
    p.timeline[(size_t)blockIdx.x * kTimelineSlots + slot] = (int64_t)wall_clock64();
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void block_kernel(BlockParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  stamp(p, 0);
  const Deps d = deps_init(p);
  const RouteLds R = route_lds(p, lds);
  unsigned char *scratch = lds + p.lds_route_bytes;
  const int G = gridDim.x;
  const int nR = p.n_router, nRT = p.n_route, nP = p.n_pool, nPN = p.n_prenorm;
  const int nF = p.n_fin, nN = p.n_unpool, nB = p.n_boundary;
  bool routed = false, h_ready = p.h_producers == 0;
  int nU = 0, nD = 0;
  int last_step = -1;
  for (int idx = blockIdx.x;; idx += G) {
    int step, j = idx;
    if (j < nR) {
      step = 1;
    } else if ((j -= nR) < nRT) {
      step = 2;
    } else if ((j -= nRT) < nP) {
      step = 3;
    } else if ((j -= nP) < nPN) {
      step = 4;
    } else {
      j -= nPN;
      if (!routed && p.needs_routing) {
        prepare_routing(p, d, R, scratch);
        routed = true;
        stamp(p, 5);
        if (p.has_up) {
          nU = *R.nact * (p.I / 16);
          nD = *R.nact * (p.P / 32);
        }
      }
      if (j < nU) step = 6;
      else if ((j -= nU) < nD) step = 7;
      else if ((j -= nD) < nF) step = 8;
      else if ((j -= nF) < nN) step = 9;
      else if ((j -= nN) < nB) step = 10;
      else break;
    }
    if (step != last_step) {
      stamp(p, step);
      last_step = step;
    }
    switch (step) {
      case 1: router_task(p, d, j, scratch); break;
      case 2: route_task(p, d, R, j); break;
      case 3:
        if (proj_task(d, p.x, false, p.pool_w, p.h, p.b, p.P, p.H, p.pool_ks, p.pool_part, p.pool_cnt,
                      nullptr, 0u, j, scratch))
          signal(d.ctr(kCtrPool));
        break;
      case 4: prenorm_task(p, d, j, scratch); break;
      case 6: up_task(p, d, R, j, h_ready, scratch); break;
      case 7: down_task(p, d, R, j, scratch); break;
      case 8: fin_task(p, d, R, j, scratch); break;
      case 9:
        if (proj_task(d, p.moe_out, p.n_fin > 0, p.unpool_w, p.u, p.b, p.H, p.P, p.unpool_ks,
                      p.unpool_part, p.unpool_cnt, d.ctr(kCtrFin), (unsigned)p.n_fin, j, scratch))
          signal(d.ctr(kCtrUnpool));
        break;
      case 10: boundary_task(p, d, j, scratch); break;
      default: break;
    }
  }
  // Workgroup 0 writes the routing outputs even when it ran no routed step.
  if (!routed && p.needs_routing && p.routing_out && blockIdx.x == 0) prepare_routing(p, d, R, scratch);
  stamp(p, 15);
  // The last workgroup to finish ends the launch's epoch.
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned done =
        __hip_atomic_fetch_add(d.ctr(kCtrFinished), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (unsigned)G - 1) __hip_atomic_fetch_add(&p.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

hipError_t launch_block(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  void *args[] = {const_cast<BlockParams *>(&p)};
  return hipLaunchCooperativeKernel((const void *)block_kernel, dim3(grid), dim3(kThreads), args,
                                    (unsigned)lds, s);
}

int block_max_groups_per_cu(size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, block_kernel, kThreads, lds) != hipSuccess)
    return 0;
  return n;
}

}  // namespace mb
