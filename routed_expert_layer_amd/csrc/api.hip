// The C ABI of libmb.so (declared and documented in include/mb.h): argument
// checks, workspace layout and the launch sequence of each entry point.

#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "mb_block.h"
#include "mb_internal.h"
#include "mb_sync.h"

// The workspace of mb_moe_block_noalloc: a static device array, of which
// every GPU the library runs on holds its own copy (at its own address) until
// the process ends.  Host code uses the per-device address that
// hipGetSymbolAddress returns for it, never the array's name.
static __device__ __align__(256) unsigned char scratch[MB_NOALLOC_SCRATCH_BYTES];

namespace mb {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout layout_of(const mb_dims &d) {
  const size_t b = d.rows, H = d.hidden, P = d.pooled, I = d.inter, E = d.experts;
  const size_t R = b * d.top_k;
  const size_t wide = P > H ? P : H;
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  // The persistent launch's state (a fixed size), then the tile counters the
  // kernels leave at zero after every call, at offsets that depend only on H
  // and P, so one workspace serves calls of any row count.
  static_assert(kMaxRows <= kSyncMaxRows, "the counter sets cover every row count");
  L.sync = take(kSyncWords * 4);
  L.pool_cnt = take(((P + 63) / 64) * kMaxRowBlocks * 4);  // per pooler tile and 64-row block
  L.rtr_cnt = take((size_t)kMaxGrid * 4);  // the MFMA router's split counters
  L.qkv_cnt = take(kMaxQkvGroups * 4);
  L.logits = take(b * E * 4);
  L.ids = take(R * 4);
  L.wts = take(R * 4);
  L.count = take(E * 4);
  L.offset = take((E + 1) * 4);
  L.route_list = take(R * 4);
  L.active = take(E * 4);
  L.n_active = take(4);
  L.h = take(b * P * 2);
  L.act = take(R * I * 2);
  L.y = take(R * P * 4);
  L.ssq = take(R * (P / 32) * 4);
  L.moe_out = take(b * P * 2);
  L.moe_rep = take((size_t)kMoeReplicas * b * P * 2);
  L.u = take(b * H * 2);
  L.partial = take((size_t)kMaxSplitK * b * wide * 4);
  L.pool_part = take((size_t)kMaxPoolSplit * b * P * 4);
  L.unpool_part = take((size_t)kMaxSplitK * b * H * 4);
  L.qkv_part = take((size_t)kMaxSplitK * b * (size_t)d.qkv_rows * 4);
  // The fp64-MFMA router's split partials (splits x tiles never exceed the
  // grid; written before they are read).
  L.rtr_part = take((size_t)kMaxGrid * 256 * 8);
  // Tagged hand-off words of the block kernel (8 bytes each).
  size_t t = 0;
  auto ttake = [&](size_t bytes) {
    const size_t at = t;
    t = align256(t + bytes);
    return at;
  };
  L.t_logits = ttake(b * E * 8);
  L.t_routes = ttake((size_t)kRouteReps * 2 * R * 8);
  L.t_h = ttake(b * P * 4);
  L.t_hn = ttake(b * P * 4);
  L.t_act = ttake(R * I * 4);
  L.tagged = t;
  L.total = o + t;
  return L;
}

// The abort record (word 1 of the launch state, at the workspace start): read
// into *status as MB_OK / MB_ERR_ABORTED, or cleared (status NULL).  One
// thread; a kernel rather than a memset or copy, so that a captured graph
// replays it as it is.
__global__ void abort_word_kernel(unsigned *state, int32_t *status) {
  if (status) *status = __hip_atomic_load(state + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? MB_ERR_ABORTED : MB_OK;
  else __hip_atomic_store(state + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_abort_word(void *workspace, int32_t *status, hipStream_t s) {
  hipLaunchKernelGGL(abort_word_kernel, dim3(1), dim3(1), 0, s, static_cast<unsigned *>(workspace), status);
  return hipGetLastError();
}

// Zero n 16-byte words (a kernel, not a memset: a captured graph replays it
// as it is).
__global__ void zero16_kernel(uint4 *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace mb

using namespace mb;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims(const mb_dims *d) {
  if (!d) return MB_ERR_NULL;
  if (d->rows <= 0 || d->hidden <= 0 || d->pooled <= 0 || d->inter <= 0 || d->experts <= 0 ||
      d->top_k <= 0)
    return MB_ERR_DIMS;
  if (d->top_k > d->experts) return MB_ERR_DIMS;
  if (d->scoring != MB_SCORING_SIGMOID && d->scoring != MB_SCORING_SOFTMAX) return MB_ERR_DIMS;
  if (d->act_quant != 0 && d->act_quant != 1) return MB_ERR_DIMS;
  if (d->qkv_rows < 0) return MB_ERR_DIMS;
  if (d->qkv_rows % 16 || d->qkv_rows > 64 * kMaxQkvGroups) return MB_ERR_UNSUPPORTED;
  if (!(d->norm_eps >= 0.0f) || !isfinite(d->norm_eps) || !isfinite(d->route_scale) ||
      !isfinite(d->router_multiplier) || !isfinite(d->division_eps))
    return MB_ERR_DIMS;
  if (d->rows > kMaxRows || d->experts > kMaxExperts || d->top_k > kMaxTopK)
    return MB_ERR_UNSUPPORTED;
  if ((long)d->experts * ((d->rows + 63) / 64) > kMaxBitmapWords) return MB_ERR_UNSUPPORTED;
  if (d->hidden % 32 || d->pooled % 128 || d->inter % 128) return MB_ERR_UNSUPPORTED;
  return MB_OK;
}

int check_ws(const mb_dims *d, const void *ws, size_t bytes) {
  if (!ws) return MB_ERR_WORKSPACE;
  if (!aligned16(ws)) return MB_ERR_ALIGN;
  if (bytes < layout_of(*d).total) return MB_ERR_WORKSPACE;
  return MB_OK;
}

// The static scratch serves a call when its buffers fit before the last
// MB_NOALLOC_TAGGED_BYTES and its hand-off words fit in them: then the
// buffers of one call never overlap the hand-off words of another (whatever
// their sizes), so no stale buffer contents can pass for a hand-off word.
int check_scratch(const mb_dims *d) {
  const Layout L = layout_of(*d);
  if (L.tagged > (size_t)MB_NOALLOC_TAGGED_BYTES) return MB_ERR_SCRATCH;
  if (L.total - L.tagged > (size_t)MB_NOALLOC_SCRATCH_BYTES - MB_NOALLOC_TAGGED_BYTES) return MB_ERR_SCRATCH;
  return MB_OK;
}

// Required pointers must be non-NULL; every given pointer must be aligned.
int need(std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs)
    if (!p) return MB_ERR_NULL;
  for (const void *p : ptrs)
    if (!aligned16(p)) return MB_ERR_ALIGN;
  return MB_OK;
}

int maybe(std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return MB_ERR_ALIGN;
  return MB_OK;
}

#define MB_TRY(expr)            \
  do {                          \
    const int _st = (expr);     \
    if (_st != MB_OK) return _st; \
  } while (0)

#define MB_HIP(expr)                              \
  do {                                            \
    if ((expr) != hipSuccess) return MB_ERR_HIP;  \
  } while (0)

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current), when the array is also zero-filled on the
// caller's stream: the launch state, the tile counters and the hand-off words
// must start at zero, as in a zero-filled workspace.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int noalloc_scratch(hipStream_t s, void **out) {
  int dev = 0;
  MB_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    MB_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return MB_ERR_HIP;
    hipLaunchKernelGGL(zero16_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4 *>(ptr),
                       (size_t)MB_NOALLOC_SCRATCH_BYTES / 16);
    MB_HIP(hipGetLastError());
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MB_OK;
}

int check_weights_route(const mb_weights *w, int flags, const uint16_t *x) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->expert_bias}));
  if (!(flags & MB_LOGITS_IN)) MB_TRY(need({x, w->router_w}));
  return MB_OK;
}

// The experts come in the caller's layout, in the streaming layout, or both.
int check_weights_experts(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->post_norm_w}));
  MB_TRY(maybe({w->w13, w->w13_scale, w->w2, w->w2_scale, w->experts_packed}));
  if (w->experts_packed) return MB_OK;
  return need({w->w13, w->w13_scale, w->w2, w->w2_scale});
}

bool has_plain_experts(const mb_weights *w) { return w->w13 && w->w13_scale && w->w2 && w->w2_scale; }

// (With proj_packed, pool_w and unpool_w may be NULL: the block kernel reads
// the packed copy, the per-step kernels need the caller's.)
int check_weights_boundary(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->gate}));
  MB_TRY(maybe({w->unpool_w, w->proj_packed, w->ffn_norm_w, w->next_norm_w}));
  return w->proj_packed ? MB_OK : need({w->unpool_w});
}

int check_weights_pool(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(maybe({w->pool_w, w->proj_packed, w->pre_norm_w}));
  return w->proj_packed ? MB_OK : need({w->pool_w});
}

int run_route(const mb_dims &d, const uint16_t *x, const mb_weights *w, float *logits, int flags,
              int32_t *ids, float *wts, int32_t *count, int32_t *offset, int32_t *route_list,
              int32_t *active, int32_t *n_active, hipStream_t s) {
  if (!(flags & MB_LOGITS_IN)) MB_HIP(launch_router_logits(d, x, w->router_w, logits, s));
  MB_HIP(launch_route_select(d, logits, w->expert_bias, ids, wts, s));
  MB_HIP(launch_route_group(d, ids, count, offset, route_list, active, n_active, s));
  return MB_OK;
}

int run_pool(const mb_dims &d, const uint16_t *x, const mb_weights *w, uint16_t *h, void *ws,
             hipStream_t s) {
  if (!w->pool_w) return MB_ERR_UNSUPPORTED;  // (only proj_packed: the per-step kernels read the caller's layout)
  const Layout L = layout_of(d);
  MB_HIP(launch_gemm_bf16(x, w->pool_w, h, d.rows, d.pooled, d.hidden, at<float>(ws, L.partial),
                          nullptr, s));
  if (w->pre_norm_w) MB_HIP(launch_rownorm_bf16(h, w->pre_norm_w, d.rows, d.pooled, d.norm_eps, s));
  return MB_OK;
}

int run_experts(const mb_dims &d, const uint16_t *h, const float *wts, const int32_t *offset,
                const int32_t *route_list, const int32_t *active, const int32_t *n_active,
                const mb_weights *w, uint16_t *moe_out, void *ws, hipStream_t s, uint16_t *act_out = nullptr) {
  const Layout L = layout_of(d);
  uint16_t *act = act_out ? act_out : at<uint16_t>(ws, L.act);
  float *y = at<float>(ws, L.y), *ssq = at<float>(ws, L.ssq);
  MB_HIP(launch_experts_up(d, h, offset, route_list, active, n_active, w->w13, w->w13_scale, act, s));
  MB_HIP(launch_experts_down(d, act, offset, route_list, active, n_active, w->w2, w->w2_scale, y,
                             ssq, s));
  MB_HIP(launch_experts_finalize(d, y, ssq, wts, w->post_norm_w, moe_out, s));
  return MB_OK;
}

int run_unpool_boundary(const mb_dims &d, const uint16_t *moe_out, const mb_weights *w,
                        float *stream, uint16_t *x_next, uint16_t *u, void *ws, hipStream_t s) {
  if (!w->unpool_w) return MB_ERR_UNSUPPORTED;  // (only proj_packed, as in run_pool)
  const Layout L = layout_of(d);
  MB_HIP(launch_gemm_bf16(moe_out, w->unpool_w, u, d.rows, d.hidden, d.pooled,
                          at<float>(ws, L.partial), nullptr, s));
  MB_HIP(launch_boundary(d, u, stream, w->gate, w->ffn_norm_w, w->next_norm_w, x_next, s));
  return MB_OK;
}

// ---- the persistent block kernel (block.hip) --------------------------------

// Launch-shape queries, asked of the runtime once and kept: the current
// device's CU count, and the block kernel's resident workgroups per CU for
// each (device, kernel variant, LDS bytes).  0 = the query failed (not kept).
std::mutex g_shape_mu;
std::map<int, int> g_cus;
std::map<std::tuple<int, int, size_t>, int> g_occ;

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(g_shape_mu);
  const auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
  g_cus[dev] = n;
  return n;
}

int block_occupancy(size_t lds, bool w4a4, bool qkv, bool many) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(dev, (w4a4 ? 2 : 0) + (qkv ? 1 : 0) + (many ? 4 : 0), lds);
  {
    std::lock_guard<std::mutex> lock(g_shape_mu);
    const auto it = g_occ.find(key);
    if (it != g_occ.end()) return it->second;
  }
  const int n = block_max_groups_per_cu(lds, w4a4, qkv, many);
  if (n < 1) return 0;
  std::lock_guard<std::mutex> lock(g_shape_mu);
  g_occ[key] = n;
  return n;
}

// Fill the sizes, scalars and workspace pointers every phase set shares.
BlockParams base_params(const mb_dims &d, const mb_weights *w, void *ws, size_t ws_bytes) {
  const Layout L = layout_of(d);
  const size_t tb = tagged_base(L, ws_bytes);
  BlockParams p{};
  p.b = d.rows;
  p.H = d.hidden;
  p.P = d.pooled;
  p.I = d.inter;
  p.E = d.experts;
  p.k = d.top_k;
  p.scoring = d.scoring;
  p.mult = d.router_multiplier;
  p.div_eps = d.division_eps;
  p.route_scale = d.route_scale;
  p.norm_eps = d.norm_eps;
  p.w4a4 = d.act_quant;
  if (w) {
    p.router_w = w->router_w;
    p.bias = w->expert_bias;
    p.pool_w = w->pool_w;
    p.pre_norm_w = w->pre_norm_w;
    p.w13 = w->w13;
    p.w13s = w->w13_scale;
    p.w2 = w->w2;
    p.w2s = w->w2_scale;
    p.xp = w->experts_packed;
    const PackedExperts X = packed_experts(d.pooled, d.inter);
    p.xp_stride = X.stride;
    p.xp_up_s = X.up_s;
    p.xp_down = X.down;
    p.xp_down_s = X.down_s;
    p.post_norm_w = w->post_norm_w;
    p.unpool_w = w->unpool_w;
    if (w->proj_packed) {
      p.pool_wp = reinterpret_cast<const uint16_t *>(w->proj_packed);
      p.unpool_wp = reinterpret_cast<const uint16_t *>(w->proj_packed + packed_projections(d.pooled, d.hidden).unpool);
    }
    p.ffn_norm_w = w->ffn_norm_w;
    p.gate = w->gate;
    p.next_norm_w = w->next_norm_w;
  }
  p.logits_f = at<float>(ws, L.logits);
  p.pool_part = at<float>(ws, L.pool_part);
  p.unpool_part = at<float>(ws, L.unpool_part);
  p.y = at<float>(ws, L.y);
  p.ssq = at<float>(ws, L.ssq);
  p.act = at<uint16_t>(ws, L.act);
  p.moe_rep = at<uint16_t>(ws, L.moe_rep);
  p.pool_cnt = at<unsigned>(ws, L.pool_cnt);
  p.rtr_part = at<double>(ws, L.rtr_part);
  p.rtr_cnt = at<unsigned>(ws, L.rtr_cnt);
  p.sync = at<unsigned>(ws, L.sync);
  p.h = at<uint16_t>(ws, L.h);
  p.moe_out = at<uint16_t>(ws, L.moe_out);
  p.u = at<uint16_t>(ws, L.u);
  p.ids = at<int32_t>(ws, L.ids);
  p.wts = at<float>(ws, L.wts);
  p.count = at<int32_t>(ws, L.count);
  p.offset = at<int32_t>(ws, L.offset);
  p.route_list = at<int32_t>(ws, L.route_list);
  p.active = at<int32_t>(ws, L.active);
  p.n_active = at<int32_t>(ws, L.n_active);
  p.logits_t = at<uint32_t>(ws, tb + L.t_logits);
  p.routes_t = at<uint32_t>(ws, tb + L.t_routes);
  p.h_t = at<uint32_t>(ws, tb + L.t_h);
  p.hn_t = at<uint32_t>(ws, tb + L.t_hn);
  p.act_t = at<uint32_t>(ws, tb + L.t_act);
  return p;
}

// The next-QKV projection as a step of the persistent launch: 64-feature
// tiles, split along H to about fill the grid (each split a multiple of 32).
void set_qkv(BlockParams &p, const mb_dims &d, const uint16_t *w_qkvg, uint16_t *qkvg, void *ws) {
  const Layout L = layout_of(d);
  const int groups = (d.qkv_rows + 63) / 64;
  const int grid = device_cus() * kBlockGroupsPerCu;
  int ks = std::max(1, std::min(kMaxSplitK, grid / groups));
  while (ks > 1 && (d.hidden % ks != 0 || (d.hidden / ks) % 32 != 0)) --ks;
  p.qkv_w = w_qkvg;
  p.qkvg = qkvg;
  p.qkv_rows = d.qkv_rows;
  p.qkv_ks = ks;
  p.n_qkv = groups * ks;
  p.qkv_part = at<float>(ws, L.qkv_part);
  p.qkv_cnt = at<unsigned>(ws, L.qkv_cnt);
}

// Which steps one launch of the persistent kernel runs.
struct Steps {
  bool router = false;       // router logits (else given, or not needed)
  bool pool = false;         // pooler (and the pre-expert norm when weighted)
  bool experts = false;      // up, down, finalize
  bool unpool = false;       // unpooler and boundary
  bool routing_out = false;  // workgroup 0 writes the routing outputs
  bool route_given = false;  // routing arrays come from the caller
};

// Contraction split of a wide projection's tasks beyond 64 rows (64-feature
// tiles x 64-row blocks, the count rounded up to whole groups of eight, dealt
// to the workgroups in turn): each task streams its split in segments of 256
// elements, so the phase takes about (rounds of tasks over the grid) x
// (segments per task); the split with the fewest, then the fewest splits.
// Each split is a multiple of 32 elements.
int row_block_split(int groups, int kdim, int row_blocks, int grid, int max_ks) {
  int best = 1;
  long best_cost = -1;
  for (int ks = 1; ks <= max_ks; ++ks) {
    if (kdim % ks != 0 || (kdim / ks) % 32 != 0) continue;
    const long tasks = (long)((groups * ks + 7) / 8 * 8) * row_blocks;
    const long cost = (tasks + grid - 1) / grid * ((kdim / ks + 255) / 256);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ks;
    }
  }
  return best;
}

// Launch the persistent kernel for `st`.  *used = false (and nothing
// launched) when the sizes do not fit it; the caller then runs the per-step
// kernels instead.
int run_fused(BlockParams &p, const Steps &st, hipStream_t s, bool *used) {
  *used = false;
  // MXFP4 activations exist in the block kernel's streaming path only.
  const int none = (st.experts && p.w4a4) ? MB_ERR_UNSUPPORTED : MB_OK;
  if (st.experts && p.w4a4 && !p.xp) return MB_ERR_UNSUPPORTED;
  if (p.E > kBlockMaxExperts || p.H > 1024 * kBoundGroups) return none;
  const size_t route_bytes = route_lds_bytes(p.b, p.k, p.E);
  const size_t lds = route_bytes + kBlockScratchBytes;
  if (lds > 64 * 1024) return none;
  const int occ = block_occupancy(lds, p.w4a4 != 0, p.n_qkv > 0, false);
  const int cus = device_cus();
  if (occ < 1 || cus < 1) return none;
  int grid = cus * (occ < kBlockGroupsPerCu ? occ : kBlockGroupsPerCu);
  if (grid > kMaxGrid) grid = kMaxGrid;
  p.lds_route_bytes = (int)route_bytes;
  p.cus = cus;
  // Router tasks: one expert x 4 rows, or kRouterExperts experts x 4 rows
  // when one-expert tasks would take more than one and a half rounds of the
  // grid (against four-expert tasks, c3 b = 28 and 32, 896 and 1024
  // one-expert tasks: 190.2 -> 185.1 and 196.3 -> 194.0 us; b = 48, two
  // rounds: +0.9 us; b = 16, four-expert tasks to leave the pooler a round
  // to itself: +8.6 us).
  const int nrb = (p.b + kRouterRowBlock - 1) / kRouterRowBlock;
  p.router_multi = 2 * p.E * nrb > 3 * grid ? 1 : 0;
  // From 64 rows: tiles of 16 rows x 16 experts on fp64 MFMA, the
  // contraction split (in whole 32-element chunks) so that tiles x splits
  // fill at most half of the grid (below; at 32 rows the four-expert tasks
  // were as fast).
  const int rtiles = ((p.b + 15) / 16) * ((p.E + 15) / 16);
  p.router_mma = (st.router && p.router_multi && p.b >= 64) ? 1 : 0;
  // Beyond 64 rows the wide projections' tasks take one 64-row block each.
  p.row_blocks = p.b > 64 ? (p.b + 63) / 64 : 1;
  const bool many = (p.router_mma || p.row_blocks > 1) && !p.w4a4 && p.n_qkv == 0;
  if (many) {
    // The plain kernel's many-rows instance, with its own occupancy.
    const int occ_m = block_occupancy(lds, false, false, true);
    if (occ_m < 1) return none;
    if (occ_m < occ) grid = std::min(kMaxGrid, cus * std::min(occ_m, kBlockGroupsPerCu));
  }
  // In it, the expert units stage plain h and act behind counters: at many
  // rows every unit stages many rows, and tagged words would double the
  // bytes it reads and add the tag checks.
  p.plain_stage = (many && st.experts) ? 1 : 0;
  // The MFMA router's tasks take at most half of the grid, so that the
  // pooler's tasks start in the same round beside them (at c2 with the whole
  // grid: 512 router tasks, and 144 of the 384 pooler tasks ran after a
  // router task; c2 210 -> 206 us, c3 b = 64 221 -> 217, b = 256 329 -> 327).
  p.router_ks = 1;
  while (p.router_ks * 2 * rtiles <= grid / 2 && p.H % (p.router_ks * 2 * 32) == 0) p.router_ks *= 2;
  const int n_router =
      st.router ? (p.router_mma ? rtiles * p.router_ks
                                : (p.router_multi ? (p.E + kRouterExperts - 1) / kRouterExperts : p.E) * nrb)
                : 0;
  const int n_fin = st.experts ? p.b * ((p.P + kFinChunk - 1) / kFinChunk) : 0;
  const int n_boundary = st.unpool ? p.b : 0;
  const int n_prenorm = (st.pool && p.pre_norm_w) ? p.b : 0;
  const bool needs_routing = st.experts || st.routing_out;
  // Route tasks (4 rows each) publish ids and weights for every workgroup's
  // grouping.  (Every workgroup routing every row itself costs each of them
  // b/4 rows one after another, and has all of them read every logit.)
  const int n_route = (needs_routing && !st.route_given) ? (p.b + 3) / 4 : 0;
  // The pooler: wide tiles of 64 features, split along H so that the router,
  // route and pooler tasks fill the workgroups about once (at least half of
  // them for the pooler), each split a multiple of 32 elements.
  // Beyond 64 rows the tasks take one 64-row block each (the blocks of a
  // tile and split on one XCD), split by row_block_split: the pooler is then
  // most of the front.
  auto round8 = [](int v) { return (v + 7) / 8 * 8; };
  {
    const int groups = (p.P + 63) / 64;
    int ks;
    if (p.row_blocks > 1) {
      ks = row_block_split(groups, p.H, p.row_blocks, grid, kMaxPoolSplit);
    } else {
      const int slots = std::max(grid - n_router - n_route - n_prenorm, grid / 2);
      ks = std::min(kMaxPoolSplit, std::max(1, slots / groups));
      while (ks > 1 && (p.H % ks != 0 || (p.H / ks) % 32 != 0)) --ks;
    }
    p.pool_ks = ks;
  }
  // The unpooler: at few rows, tasks of kUnpoolTiles 16-feature tiles over
  // the fewest contraction splits that let every wave request all its
  // weights before the wait (at most kUnpoolChunks 32-element chunks each);
  // at many rows (or contractions too long for that) 64-feature tiles, so
  // that the MoE output is read once per 64 features, split along P to fill
  // the grid (its tasks follow the finalize tasks, which all end before any
  // unpooler work can start, so the whole grid is theirs).
  int narrow_ks = 1;
  while (narrow_ks < kMaxSplitK && (p.P / 32 + narrow_ks - 1) / narrow_ks > kBlockWaves * kUnpoolChunks) ++narrow_ks;
  p.unpool_wide = (p.b > 16 || (p.P / 32 + narrow_ks - 1) / narrow_ks > kBlockWaves * kUnpoolChunks) ? 1 : 0;
  if (p.unpool_wide) {
    const int groups = (p.H + 63) / 64;
    int ks;
    if (p.row_blocks > 1) {
      // Two splits (pooled % 128 == 0) up to three row blocks, one from
      // four: against the cost model's three, c3 b = 96 and 128 236.0 ->
      // 233.4 and 245.6 -> 243.3 us with two (one in between), b = 192 the
      // same with two (+0.7 with one); at b = 256 one split against two
      // 319.9 -> 308.9 us.
      ks = p.row_blocks >= 4 ? 1 : 2;
    } else {
      // At most three splits: against min(8, grid / tiles) (six at H 7168),
      // c2 206.2 -> 201.2 us, c3 b = 64 217.3 -> 212.6, b = 32 195.1 ->
      // 191.8 (two and four splits in between).
      ks = std::min(3, std::max(1, grid / groups));
      while (ks > 1 && (p.P % ks != 0 || (p.P / ks) % 32 != 0)) --ks;
    }
    p.unpool_ks = ks;
  } else {
    p.unpool_ks = narrow_ks;
  }
  p.n_pool_tiles = (p.P + 63) / 64;
  p.needs_routing = needs_routing ? 1 : 0;
  p.routing_out = st.routing_out ? 1 : 0;
  p.route_given = st.route_given ? 1 : 0;
  p.n_router = n_router;
  p.n_logit_producers = p.n_router;
  p.n_route = n_route;
  p.n_pool = st.pool ? (p.row_blocks > 1 ? round8(p.n_pool_tiles * p.pool_ks) * p.row_blocks
                                         : p.n_pool_tiles * p.pool_ks)
                     : 0;
  p.n_prenorm = n_prenorm;
  p.h_tagged = st.pool ? 1 : 0;
  // Signals that make h complete under plain staging: every pooler tile (each
  // 64-row block of it beyond 64 rows), or every pre-norm row, which then
  // writes h in bf16 itself.
  p.n_h_ready = !st.pool ? 0 : n_prenorm > 0 ? n_prenorm
                                             : p.n_pool_tiles * (p.row_blocks > 1 ? p.row_blocks : 1);
  if (p.plain_stage && n_prenorm > 0) p.h_plain = 1;
  p.has_up = st.experts ? 1 : 0;
  p.n_fin = n_fin;
  if (!st.unpool) {
    p.n_unpool = 0;
  } else if (p.unpool_wide) {
    const int gq = ((p.H + 63) / 64) * p.unpool_ks;
    p.n_unpool = p.row_blocks > 1 ? round8(gq) * p.row_blocks : gq;
  } else {
    p.n_unpool = p.H / (16 * kUnpoolTiles) * p.unpool_ks;
  }
  p.n_boundary = n_boundary;
  MB_HIP(launch_block(p, grid, lds, s));
  *used = true;
  return MB_OK;
}

// The arguments of the whole-block call (both forms of it).
int check_block_args(const mb_dims *dims, const uint16_t *x, const mb_weights *w, float *stream,
                     uint16_t *x_next, const mb_block_taps *taps) {
  MB_TRY(check_dims(dims));
  MB_TRY(check_weights_route(w, 0, x));
  MB_TRY(check_weights_pool(w));
  MB_TRY(check_weights_experts(w));
  MB_TRY(check_weights_boundary(w));
  MB_TRY(need({stream, x_next}));
  if (taps)
    MB_TRY(maybe({taps->logits, taps->topk_ids, taps->topk_w, taps->count, taps->offset, taps->route_list,
                  taps->active, taps->n_active, taps->h, taps->moe_out, taps->u, taps->timeline, taps->act,
                  taps->qkvg}));
  return MB_OK;
}

// The whole block on a checked workspace `ws` of ws_bytes bytes.
int run_block_call(const mb_dims &d, const uint16_t *x, const mb_weights *w, float *stream, uint16_t *x_next,
                   const mb_block_taps *taps, void *ws, size_t ws_bytes, hipStream_t s) {
  mb_block_taps tp{};
  if (taps) tp = *taps;
  const Layout L = layout_of(d);
  float *logits = tp.logits ? tp.logits : at<float>(ws, L.logits);
  int32_t *ids = tp.topk_ids ? tp.topk_ids : at<int32_t>(ws, L.ids);
  float *wts = tp.topk_w ? tp.topk_w : at<float>(ws, L.wts);
  int32_t *count = tp.count ? tp.count : at<int32_t>(ws, L.count);
  int32_t *offset = tp.offset ? tp.offset : at<int32_t>(ws, L.offset);
  int32_t *route_list = tp.route_list ? tp.route_list : at<int32_t>(ws, L.route_list);
  int32_t *active = tp.active ? tp.active : at<int32_t>(ws, L.active);
  int32_t *n_active = tp.n_active ? tp.n_active : at<int32_t>(ws, L.n_active);
  uint16_t *h = tp.h ? tp.h : at<uint16_t>(ws, L.h);
  uint16_t *moe_out = tp.moe_out ? tp.moe_out : at<uint16_t>(ws, L.moe_out);
  uint16_t *u = tp.u ? tp.u : at<uint16_t>(ws, L.u);
  BlockParams p = base_params(d, w, ws, ws_bytes);
  Steps st;
  st.router = st.pool = st.experts = st.unpool = true;
  st.routing_out = tp.topk_ids || tp.topk_w || tp.count || tp.offset || tp.route_list || tp.active ||
                   tp.n_active || tp.logits;
  p.x = x;
  p.logits = tp.logits;
  p.ids = ids;
  p.wts = wts;
  p.count = count;
  p.offset = offset;
  p.route_list = route_list;
  p.active = active;
  p.n_active = n_active;
  p.h = h;
  p.moe_out = moe_out;
  p.u = u;
  p.stream = stream;
  p.x_next = x_next;
  p.timeline = tp.timeline;
  p.act_tap = tp.act;
  p.h_plain = tp.h ? 1 : 0;
  if (d.qkv_rows > 0) {
    // The next-QKV projection fused after the boundary.
    MB_TRY(need({w->next_qkv_w, tp.qkvg}));
    set_qkv(p, d, w->next_qkv_w, tp.qkvg, ws);
  }
  bool used = false;
  MB_TRY(run_fused(p, st, s, &used));
  if (used) return MB_OK;
  // The per-step kernels read the caller's layouts.
  if (!has_plain_experts(w) || !w->pool_w || !w->unpool_w) return MB_ERR_UNSUPPORTED;
  MB_TRY(run_route(d, x, w, logits, 0, ids, wts, count, offset, route_list, active, n_active, s));
  MB_TRY(run_pool(d, x, w, h, ws, s));
  MB_TRY(run_experts(d, h, wts, offset, route_list, active, n_active, w, moe_out, ws, s, tp.act));
  MB_TRY(run_unpool_boundary(d, moe_out, w, stream, x_next, u, ws, s));
  if (d.qkv_rows > 0)
    MB_HIP(launch_gemm_bf16(x_next, w->next_qkv_w, tp.qkvg, d.rows, d.qkv_rows, d.hidden, at<float>(ws, L.qkv_part),
                            nullptr, s));
  return MB_OK;
}

}  // namespace

extern "C" {

int mb_workspace_bytes(const mb_dims *dims, size_t *bytes) {
  if (!bytes) return MB_ERR_NULL;
  MB_TRY(check_dims(dims));
  *bytes = layout_of(*dims).total;
  return MB_OK;
}

int mb_route(const mb_dims *dims, const uint16_t *x, const mb_weights *w, float *logits,
             int flags, int32_t *topk_ids, float *topk_w, int32_t *count, int32_t *offset,
             int32_t *route_list, int32_t *active, int32_t *n_active, void *workspace,
             size_t workspace_bytes, void *stream) {
  MB_TRY(check_dims(dims));
  if ((flags & ~(MB_LOGITS_IN | MB_LOGITS_OUT)) != 0 ||
      ((flags & MB_LOGITS_IN) && (flags & MB_LOGITS_OUT)))
    return MB_ERR_DIMS;
  MB_TRY(check_weights_route(w, flags, x));
  MB_TRY(need({topk_ids, topk_w, count, offset, route_list, active, n_active}));
  if (flags) MB_TRY(need({logits}));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  BlockParams p = base_params(*dims, w, workspace, workspace_bytes);
  Steps st;
  st.router = !(flags & MB_LOGITS_IN);
  st.routing_out = true;
  p.x = x;
  p.logits_in = (flags & MB_LOGITS_IN) ? 1 : 0;
  p.logits = flags ? logits : nullptr;
  p.ids = topk_ids;
  p.wts = topk_w;
  p.count = count;
  p.offset = offset;
  p.route_list = route_list;
  p.active = active;
  p.n_active = n_active;
  bool used = false;
  MB_TRY(run_fused(p, st, (hipStream_t)stream, &used));
  if (used) return MB_OK;
  float *lg = flags ? logits : at<float>(workspace, layout_of(*dims).logits);
  return run_route(*dims, x, w, lg, flags, topk_ids, topk_w, count, offset, route_list, active,
                   n_active, (hipStream_t)stream);
}

int mb_pool(const mb_dims *dims, const uint16_t *x, const mb_weights *w, uint16_t *h,
            void *workspace, size_t workspace_bytes, void *stream) {
  MB_TRY(check_dims(dims));
  MB_TRY(check_weights_pool(w));
  MB_TRY(need({x, h}));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  BlockParams p = base_params(*dims, w, workspace, workspace_bytes);
  Steps st;
  st.pool = true;
  p.x = x;
  p.h = h;
  p.h_plain = 1;
  bool used = false;
  MB_TRY(run_fused(p, st, (hipStream_t)stream, &used));
  if (used) return MB_OK;
  return run_pool(*dims, x, w, h, workspace, (hipStream_t)stream);
}

int mb_experts(const mb_dims *dims, const uint16_t *h, const int32_t *topk_ids,
               const float *topk_w, const int32_t *count, const int32_t *offset,
               const int32_t *route_list, const int32_t *active, const int32_t *n_active,
               const mb_weights *w, uint16_t *moe_out, void *workspace, size_t workspace_bytes,
               void *stream) {
  MB_TRY(check_dims(dims));
  MB_TRY(check_weights_experts(w));
  MB_TRY(need({h, topk_ids, topk_w, count, offset, route_list, active, n_active, moe_out}));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  BlockParams p = base_params(*dims, w, workspace, workspace_bytes);
  Steps st;
  st.experts = true;
  st.route_given = true;
  p.h = const_cast<uint16_t *>(h);
  p.ids = const_cast<int32_t *>(topk_ids);
  p.wts = const_cast<float *>(topk_w);
  p.count = const_cast<int32_t *>(count);
  p.offset = const_cast<int32_t *>(offset);
  p.route_list = const_cast<int32_t *>(route_list);
  p.active = const_cast<int32_t *>(active);
  p.n_active = const_cast<int32_t *>(n_active);
  p.moe_out = moe_out;
  bool used = false;
  MB_TRY(run_fused(p, st, (hipStream_t)stream, &used));
  if (used) return MB_OK;
  if (!has_plain_experts(w)) return MB_ERR_UNSUPPORTED;  // the per-step kernels read the caller's layout
  return run_experts(*dims, h, topk_w, offset, route_list, active, n_active, w, moe_out, workspace,
                     (hipStream_t)stream);
}

int mb_unpool_boundary(const mb_dims *dims, const uint16_t *moe_out, const mb_weights *w,
                       float *stream, uint16_t *x_next, uint16_t *u_out, void *workspace,
                       size_t workspace_bytes, void *stream_handle) {
  MB_TRY(check_dims(dims));
  MB_TRY(check_weights_boundary(w));
  MB_TRY(need({moe_out, stream, x_next}));
  MB_TRY(maybe({u_out}));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  uint16_t *u = u_out ? u_out : at<uint16_t>(workspace, layout_of(*dims).u);
  BlockParams p = base_params(*dims, w, workspace, workspace_bytes);
  Steps st;
  st.unpool = true;
  p.moe_out = const_cast<uint16_t *>(moe_out);
  p.u = u;
  p.stream = stream;
  p.x_next = x_next;
  bool used = false;
  MB_TRY(run_fused(p, st, (hipStream_t)stream_handle, &used));
  if (used) return MB_OK;
  return run_unpool_boundary(*dims, moe_out, w, stream, x_next, u, workspace,
                             (hipStream_t)stream_handle);
}

int mb_moe_block(const mb_dims *dims, const uint16_t *x, const mb_weights *w, float *stream,
                 uint16_t *x_next, const mb_block_taps *taps, void *workspace,
                 size_t workspace_bytes, void *stream_handle) {
  MB_TRY(check_block_args(dims, x, w, stream, x_next, taps));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  return run_block_call(*dims, x, w, stream, x_next, taps, workspace, workspace_bytes,
                        (hipStream_t)stream_handle);
}

int mb_moe_block_noalloc(const mb_dims *dims, const uint16_t *x, const mb_weights *w, float *stream,
                         uint16_t *x_next, const mb_block_taps *taps, void *stream_handle) {
  MB_TRY(check_block_args(dims, x, w, stream, x_next, taps));
  MB_TRY(check_scratch(dims));
  const hipStream_t s = (hipStream_t)stream_handle;
  void *ws = nullptr;
  MB_TRY(noalloc_scratch(s, &ws));
  return run_block_call(*dims, x, w, stream, x_next, taps, ws, (size_t)MB_NOALLOC_SCRATCH_BYTES, s);
}

int mb_packed_experts_bytes(const mb_dims *dims, size_t *bytes) {
  MB_TRY(check_dims(dims));
  if (!bytes) return MB_ERR_NULL;
  *bytes = (size_t)dims->experts * packed_experts(dims->pooled, dims->inter).stride;
  return MB_OK;
}

int mb_pack_experts(const mb_dims *dims, const mb_weights *w, uint8_t *packed, size_t packed_bytes,
                    void *stream) {
  MB_TRY(check_dims(dims));
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->w13, w->w13_scale, w->w2, w->w2_scale, packed}));
  size_t bytes = 0;
  MB_TRY(mb_packed_experts_bytes(dims, &bytes));
  if (packed_bytes < bytes) return MB_ERR_WORKSPACE;
  MB_HIP(launch_pack_experts(*dims, w->w13, w->w13_scale, w->w2, w->w2_scale, packed, (hipStream_t)stream));
  return MB_OK;
}

int mb_packed_projections_bytes(const mb_dims *dims, size_t *bytes) {
  MB_TRY(check_dims(dims));
  if (!bytes) return MB_ERR_NULL;
  *bytes = packed_projections(dims->pooled, dims->hidden).bytes;
  return MB_OK;
}

int mb_pack_projections(const mb_dims *dims, const mb_weights *w, uint8_t *packed, size_t packed_bytes,
                        void *stream) {
  MB_TRY(check_dims(dims));
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->pool_w, w->unpool_w, packed}));
  size_t bytes = 0;
  MB_TRY(mb_packed_projections_bytes(dims, &bytes));
  if (packed_bytes < bytes) return MB_ERR_WORKSPACE;
  MB_HIP(launch_pack_projections(*dims, w->pool_w, w->unpool_w, packed, (hipStream_t)stream));
  return MB_OK;
}

int mb_attn_boundary(const mb_dims *dims, const uint16_t *partial, const uint16_t *post_attn_norm_w,
                     const uint16_t *gate, const uint16_t *pre_ffn_norm_w, float *stream, uint16_t *out,
                     void *stream_handle) {
  MB_TRY(check_dims(dims));
  MB_TRY(need({partial, gate, stream, out}));
  MB_TRY(maybe({post_attn_norm_w, pre_ffn_norm_w}));
  MB_HIP(launch_boundary(*dims, partial, stream, gate, post_attn_norm_w, pre_ffn_norm_w, out,
                         (hipStream_t)stream_handle));
  return MB_OK;
}

int mb_next_qkv(const mb_dims *dims, const uint16_t *x_next, const uint16_t *w_qkvg, int32_t n_out,
                uint16_t *qkvg, void *workspace, size_t workspace_bytes, void *stream) {
  MB_TRY(check_dims(dims));
  if (n_out <= 0) return MB_ERR_DIMS;
  if (n_out % 16) return MB_ERR_UNSUPPORTED;
  MB_TRY(need({x_next, w_qkvg, qkvg}));
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  // The persistent kernel's projection step alone (no boundary to wait for),
  // with its partials in the workspace sized for these dims and n_out.
  {
    mb_dims dq = *dims;
    dq.qkv_rows = n_out;
    if (dq.act_quant == 0 && layout_of(dq).total <= workspace_bytes && n_out <= 64 * kMaxQkvGroups) {
      BlockParams p = base_params(dq, nullptr, workspace, workspace_bytes);
      p.x_next = const_cast<uint16_t *>(x_next);
      set_qkv(p, dq, w_qkvg, qkvg, workspace);
      bool used = false;
      MB_TRY(run_fused(p, Steps{}, (hipStream_t)stream, &used));
      if (used) return MB_OK;
    }
  }
  // Else the split-K GEMM, its partials [ks][b][n_out] fp32 in the partial area.
  const Layout L = layout_of(*dims);
  const size_t per_split = (size_t)dims->rows * n_out * 4;
  const size_t room = (size_t)kMaxSplitK * dims->rows * std::max(dims->pooled, dims->hidden) * 4;  // its size
  const int cap = (int)std::min<size_t>(kMaxSplitK, room / per_split);
  MB_HIP(launch_gemm_bf16(x_next, w_qkvg, qkvg, dims->rows, n_out, dims->hidden, at<float>(workspace, L.partial),
                          nullptr, (hipStream_t)stream, cap < 1 ? 1 : cap));
  return MB_OK;
}

int mb_effective_norm_weight(const float *weight, int32_t n, float gain_center, int32_t zero_centered,
                             uint16_t *out, void *stream) {
  if (n <= 0 || !isfinite(gain_center)) return MB_ERR_DIMS;
  if (!weight || !out) return MB_ERR_NULL;
  MB_HIP(launch_norm_weight(weight, n, zero_centered ? gain_center : 0.0f, out, (hipStream_t)stream));
  return MB_OK;
}

int mb_workspace_status(const void *workspace, size_t workspace_bytes, int32_t *status, void *stream) {
  if (!workspace || !status) return MB_ERR_NULL;
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(status) & 3u)) return MB_ERR_ALIGN;
  if (workspace_bytes < kSyncWords * 4) return MB_ERR_WORKSPACE;
  MB_HIP(launch_abort_word(const_cast<void *>(workspace), status, (hipStream_t)stream));
  return MB_OK;
}

int mb_workspace_reset(void *workspace, size_t workspace_bytes, void *stream) {
  if (!workspace) return MB_ERR_NULL;
  if (!aligned16(workspace)) return MB_ERR_ALIGN;
  if (workspace_bytes < kSyncWords * 4) return MB_ERR_WORKSPACE;
  MB_HIP(launch_abort_word(workspace, nullptr, (hipStream_t)stream));
  return MB_OK;
}

const char *mb_status_string(int status) {
  switch (status) {
    case MB_OK: return "ok";
    case MB_ERR_NULL: return "a required pointer is NULL";
    case MB_ERR_DIMS: return "invalid dims: a size is not positive, top_k exceeds experts, "
                             "scoring is not sigmoid/softmax, a scalar is not finite, or flags "
                             "are invalid";
    case MB_ERR_UNSUPPORTED: return "dims outside the supported limits (rows <= 1024, experts <= "
                                    "1024, top_k <= 16, experts*ceil(rows/64) <= 4096, hidden % 32, "
                                    "pooled % 128, inter % 128)";
    case MB_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case MB_ERR_WORKSPACE: return "workspace (or packed-weights buffer) missing or smaller than "
                                  "mb_workspace_bytes (mb_packed_experts_bytes, mb_packed_projections_bytes)";
    case MB_ERR_HIP: return "a kernel launch failed";
    case MB_ERR_SCRATCH: return "(mb_moe_block_noalloc) the sizes need more than its static scratch: "
                                "over 56 MiB of buffers or 8 MiB of hand-off words (mb_moe_block "
                                "with a workspace serves them)";
    case MB_ERR_ABORTED: return "a launch on this workspace gave up a wait between its workgroups (not all "
                                "of them were resident together): its results are not to be trusted; "
                                "mb_workspace_reset clears the record";
    default: return "unknown status";
  }
}

}  // extern "C"
