// The routed-MoE block as one persistent launch.
//
// The block's steps ([providers] MoEProvider: router, routing, pooler, routed
// experts, tail, unpooler; BoundaryProvider: the boundary; [mono.decoder]
// _K3Bucket runs the whole layer as one launch at small row counts) run as
// four lists of work, in this order, in every workgroup:
//
//   1. workgroup tasks before routing
//        router   (expert, 4 rows)         fp32 logits (fp64 sums)         [Wr]
//        route    (4 rows)                 top-k and weights
//        pool     (64 features, K split)   h = bf16(x Wp^T); the last
//                                          split of a tile adds them       [Wp]
//        prenorm  (row)                    optional RMSNorm of h
//   2. the routing state, rebuilt in the workgroup's LDS
//   3. wave units (each wave on its own: no workgroup barrier)
//        up       (expert, 16 act columns) act = bf16(silu(g) * u)        [w13]
//        down     (expert, 32 features)    y, per-tile sums of squares    [w2]
//   4. workgroup tasks after the experts
//        finalize (row, 1024 features)     moe_out = bf16(sum_j w_j yn_j)
//        unpool   (16 or 64 features,      u = moe_out Wu^T, K-split
//                  K split)                  partials                      [Wu]
//        boundary (row)                    stream, x_next
//
// Workgroup w takes workgroup tasks w, w + G, ... of lists 1 and 4; wave v
// (global index) takes up units v, v + 4G, ..., then down units v, v + 4G, ...  A task or unit waits
// only for the work whose output it reads: routing for the logits (or the
// route tasks), up for the pooler (or pre-norm), down for the up units of its
// expert, finalize for the down units of its row's experts, unpool for the
// finalize tasks, boundary for the unpool tasks.  The logits, the routes, h
// and act go from producer to consumer as tagged words (payload and the
// launch's tag in one 8-byte store), which the consumer polls directly; the
// later steps use dependency counters that producers add to after their
// coherent stores completed (mb_block.h: the layout, the two counter sets
// that alternate from launch to launch, and copies of widely awaited
// counters).  Every dependency points to earlier work in this order and the
// grid is what the device holds at once, so the earliest unfinished work can
// always run and the launch completes; every wait is also bounded.
//
// Data one workgroup hands to another goes through coherent (sc1) buffer
// accesses; weights are streamed with non-temporal loads, each wave keeping
// several chunks of its weight rows in flight.  Arithmetic: fp64-accumulated
// router logits rounded once to fp32, the fp32 routing recipe, bf16 MFMA with
// exact MXFP4 -> bf16 weight conversion and fp32 accumulation, fixed-order
// reductions (results do not depend on timing).

#include "mb_block.h"
#include "mb_device.h"
#include "mb_sync.h"

namespace mb {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MB_WAVE;
static_assert(kWaves == kBlockWaves, "routing LDS is laid out per wave");
static_assert(kRouterRowBlock == kWaves, "a router task covers as many rows as it has waves");
// 128-element weight chunks a wave keeps in flight in an up / a down unit.
constexpr int kRingUp = 4, kRingDown = 4;
// Down units of at most this many chunks (in the streaming layout, passes of
// up to 16 rows) request all their weights before waiting for the up units.
constexpr int kDownAll = 8;
static_assert(kRingUp % 4 == 0 && kRingDown % 4 == 0, "one scale load covers four chunks");
static_assert((kStageChunkRows / 32) % kRingUp == 0 && (kStageChunkRows / 32) % kRingDown == 0,
              "activation segments hold whole rounds of chunks");
constexpr int kRouterBatch = 4;   // router element blocks a thread requests at once (x 4 rows)
constexpr int kBoundBatch = 4;   // pre-norm element groups a thread requests at once

// A value the wave holds in every lane (LDS reads, the wave index), moved to
// a scalar register so that addresses and resources built from it are too.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

struct Lane {
  int lane, wave, g, r16;
  __device__ Lane()
      : lane(threadIdx.x % MB_WAVE), wave(threadIdx.x / MB_WAVE), g((threadIdx.x % MB_WAVE) >> 4),
        r16(threadIdx.x & 15) {}
};

// ---------------------------------------------------------------- dependencies

// threadIdx.x, read afresh at each use: values derived from it are then not
// kept in registers from one phase of the kernel to the next.
__device__ __forceinline__ unsigned tid() {
  unsigned t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

struct Deps {
  unsigned *s;   // the launch state (layout in mb_block.h)
  unsigned gen;  // this launch's generation (every lane): its counter set is gen % 2

  __device__ unsigned *line(size_t i) const {
    const unsigned set = (unsigned)__builtin_amdgcn_readfirstlane((int)gen) & 1u;
    return s + (sync_line_set((int)set) + i) * kLine;
  }
  __device__ unsigned *abort_word() const { return s + 1; }
  // The tag of this launch's hand-off words (the generation + 1, never the
  // 0 of a zero-filled workspace within 2^32 launches).
  __device__ unsigned tag() const { return gen + 1u; }
  __device__ unsigned *ctr(int i, int rep = 0) const { return line(sync_line_ctr(i, rep)); }
  // The first stripe of the copy of counter i that this workgroup (or wave:
  // index w) polls.
  __device__ unsigned *mine(int i, int w) const { return ctr(i, (w % replicas(i)) * stripes(i)); }
  __device__ unsigned *up(int e) const { return line(sync_line_up(e)); }
  __device__ unsigned *down(int e) const { return line(sync_line_down(e)); }
  __device__ unsigned *logits(int rb) const { return line(sync_line_logits(rb)); }
};

__device__ __forceinline__ unsigned atomic_inc(unsigned *c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_co(unsigned *w, unsigned v) {
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Generation not yet requested: a workgroup that starts with a router task
// requests it inside that task (should the generation itself equal this
// value, a later router task of the workgroup merely requests it again).
constexpr unsigned kGenPending = 0xFFFFFFFFu;

// This workgroup's generation word (coherent: the previous launch wrote it).
// The offset is opaque to the compiler, so the value stays in a vector
// register and is first waited for where a counter is used, not here.
__device__ __forceinline__ unsigned load_generation(const unsigned *state) {
  uint32_t off = (uint32_t)(kLine + blockIdx.x) * 4u;
  asm volatile("" : "+v"(off));
  return ld_co4(make_rsrc(state), off);
}

// For the next launch, at the end of a workgroup: clear its share of the
// other counter set (16-byte stores) and advance the generation words it
// owns (b, b + G, ..).  Nothing reads either during this launch.
__device__ __forceinline__ void prepare_next_launch(unsigned *state, unsigned gen) {
  const unsigned G = gridDim.x;
  const rsrc_t rs = make_rsrc(state);
  const uint32_t other = (uint32_t)(sync_line_set((int)((gen + 1u) & 1u)) * kLine * 4);
  constexpr uint32_t kPieces = (uint32_t)(kSetLines * kLine / 4);
  for (uint32_t i = blockIdx.x * kThreads + tid(); i < kPieces; i += G * kThreads)
    st_co16(rs, other + 16u * i, u32x4_t{0u, 0u, 0u, 0u});
  for (unsigned w = blockIdx.x + G * tid(); w < (unsigned)kMaxGrid; w += G * kThreads)
    st_co4(rs, (uint32_t)(kLine + w) * 4u, gen + 1u);
}

// Workgroup: every wave's coherent stores complete, then one increment.
__device__ __forceinline__ void signal(unsigned *c) {
  wait_stores();
  __syncthreads();
  if (tid() == 0) atomic_inc(c);
}

// Workgroup: every wave's coherent stores complete, then one increment of
// this workgroup's stripe in every copy of step counter i.
__device__ __forceinline__ void signal_step(const Deps &d, int i) {
  wait_stores();
  __syncthreads();
  if (tid() < replicas(i)) atomic_inc(d.ctr(i, tid() * stripes(i) + (int)(blockIdx.x % stripes(i))));
}

// Workgroup after expert units: every wave's coherent stores complete, then
// one increment by the workgroup's kWaves units.  (Units go to workgroups
// four at a time, consecutive tiles of one expert, so a workgroup's waves
// take their units together and the expert's counter sees a quarter of the
// increments -- and of the polls -- it would see from every wave.)
__device__ __forceinline__ void signal_units(unsigned *c) {
  wait_stores();
  __syncthreads();
  if (tid() == 0) __hip_atomic_fetch_add(c, (unsigned)kWaves, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup: after its coherent stores, add one to counter c; true in the
// workgroup whose increment made it `of` (the last of `of` arrivals).
__device__ __forceinline__ bool last_arrival(unsigned *c, unsigned of, int *flag) {
  wait_stores();
  __syncthreads();
  if (tid() == 0) *flag = atomic_inc(c) == of - 1u;
  __syncthreads();
  const bool last = *flag != 0;
  __syncthreads();
  return last;
}

// A polling wave, every 256 polls: whether to stop waiting.  Every wait is
// bounded: after kSpinLimit polls it gives up and raises the abort word (word
// 1 of the launch state) to this launch's tag, and every wait of the launch
// that sees it gives up too, so the grid drains.  The word keeps the tag (it
// only changes when a later launch times out, or when mb_workspace_reset
// clears it), so the caller can learn that a launch's results are not to be
// trusted (mb_workspace_status); later launches compare it with their own
// tag, so they wait and compute as usual.
__device__ __forceinline__ bool give_up(const Deps &d, unsigned &spins) {
  if ((++spins & 255u) != 0) return false;
  if (__hip_atomic_load(d.abort_word(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == d.tag()) return true;
  if (spins > kSpinLimit) {
    if (tid() % MB_WAVE == 0) store_co(d.abort_word(), d.tag());
    return true;
  }
  return false;
}

// One wave polls, each lane its own word, until every lane's has reached
// `target`.  Bounded (give_up).
__device__ __forceinline__ void poll_ge(const Deps &d, const unsigned *mine, unsigned target) {
  unsigned spins = 0;
  while (true) {
    const unsigned have = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all((int)(have >= target)) || give_up(d, spins)) return;
    __builtin_amdgcn_s_sleep(2);
  }
}

// One wave polls the n stripes (consecutive lines from `first`, one per
// lane) until their sum reached `target`.  Bounded like poll_ge.
__device__ __forceinline__ void poll_sum_ge(const Deps &d, const unsigned *first, int n, unsigned target) {
  const int lane = tid() % MB_WAVE;
  const unsigned *mine = first + (lane < n ? lane : 0) * kLine;
  unsigned spins = 0;
  while (true) {
    const unsigned have = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned sum = 0;
    for (int l = 0; l < n; ++l) sum += __builtin_amdgcn_readlane(have, l);
    if (sum >= target || give_up(d, spins)) return;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Workgroup wait on one counter.
__device__ __forceinline__ void wait_ge(const Deps &d, const unsigned *c, unsigned target) {
  if (target == 0) return;
  if (tid() < MB_WAVE) poll_ge(d, c, target);
  __syncthreads();
}

// Workgroup / one wave waits until step counter i reached `target`.
__device__ __forceinline__ void wait_step(const Deps &d, int i, int target) {
  if (target == 0) return;
  if (tid() < MB_WAVE) poll_sum_ge(d, d.mine(i, blockIdx.x), stripes(i), (unsigned)target);
  __syncthreads();
}
__device__ __forceinline__ void wave_wait_step(const Deps &d, int i, int target) {
  if (target > 0)
    poll_sum_ge(d, d.mine(i, blockIdx.x * kWaves + tid() / MB_WAVE), stripes(i), (unsigned)target);
}

// Tagged hand-off words: 8 bytes, the payload first and then the tag of the
// launch that wrote it, stored and loaded whole with coherent accesses (an
// aligned 8-byte access is single-copy atomic), so a consumer that reads this
// launch's tag reads the payload stored with it.  A consumer polls the data
// itself: no store-completion wait, counter or second load on the way.  Words
// of earlier launches carry their own (older) tags.
__device__ __forceinline__ void st_tagged(rsrc_t r, uint32_t off, uint32_t v, uint32_t tag) {
  st_co8(r, off, u32x2_t{v, tag});
}

// One wave: until every word its lanes hold (v[i] from offset off[i]; kOob:
// no word) carries this launch's tag, request again the words that do not.
// Bounded like poll_ge.
template <int N>
__device__ __forceinline__ void await_tagged(const Deps &d, rsrc_t r, const uint32_t (&off)[N], u32x2_t (&v)[N]) {
  const uint32_t tag = d.tag();
  unsigned spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && (off[i] == kOob || v[i][1] == tag);
    if (__all((int)ok) || give_up(d, spins)) return;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (off[i] != kOob && v[i][1] != tag) v[i] = ld_co8(r, off[i]);
  }
}

// Tracing: workgroup thread 0 stamps the 100 MHz real-time counter at the
// start (slot 0), when it enters its first task of each step (router 1,
// route 2, pool 3, prenorm 4, finalize 8, unpool 9, boundary 10), when its
// routing state is ready (5), when its waves start (6) and finish (11) their
// expert units, and at the end (15); inside the steps: pool task done (7),
// logits seen by a route task (12), its rows routed (14), routes seen by the
// workgroup (13), unpool task done (16), boundary's unpooler wait over (17),
// boundary done (18), finalize's expert wait over (19), wave 0's up units
// done (20), finalize done (21), router task done (22), router products
// summed in wave 0 (23).
// The workgroup's stamps are kept in LDS and written out at its end: a
// store to memory at each stamp would count in the wave's outstanding memory
// operations, and every later wait for a load would wait for it too.
__shared__ int64_t g_stamps[kTimelineSlots];

__device__ __forceinline__ void stamp(const BlockParams &p, int slot) {
  if (p.timeline && tid() == 0) {
    asm volatile("" ::: "memory");
    g_stamps[slot] = (int64_t)wall_clock64();
    asm volatile("" ::: "memory");
  }
}

// (Wave 0, which also takes every stamp: LDS accesses of one wave are in order.)
__device__ __forceinline__ void stamps_begin(const BlockParams &p) {
  if (p.timeline && tid() < kTimelineSlots) g_stamps[tid()] = 0;
}
__device__ __forceinline__ void stamps_end(const BlockParams &p) {
  if (p.timeline && tid() < kTimelineSlots)
    p.timeline[(size_t)blockIdx.x * kTimelineSlots + tid()] = g_stamps[tid()];
}

// ---------------------------------------------------------------- router

// fp64 sum over the wave's 64 lanes, in lane 63 and returned to every lane:
// DPP row shifts by 1, 2, 4, 8 and the row broadcasts 15 and 31 (each 64-bit
// value moved as its two halves), a fixed order.
template <int CTRL, int ROWS>
__device__ __forceinline__ double sum_step64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, false);
  return v + __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_dpp64(double v) {
  v = sum_step64<0x111, 0xF>(v);
  v = sum_step64<0x112, 0xF>(v);
  v = sum_step64<0x114, 0xF>(v);
  v = sum_step64<0x118, 0xF>(v);
  v = sum_step64<0x142, 0xA>(v);
  v = sum_step64<0x143, 0xC>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Logits of expert e for a block of kRouterRowBlock (4) rows, in fp64 (bf16 x
// fp32 products are exact in fp64), rounded once to fp32.  The expert's
// router row is read once per workgroup: wave w takes hidden elements in
// 256-element blocks w, w + 4, w + 8, ..; its lane q adds, for each of the
// four rows, the products of elements 4q .. 4q + 3 of those blocks in order,
// requesting kRouterBatch blocks at once.  Each wave then sums its lanes
// (wave_sum_dpp64, the four rows' trees interleaved), and the four wave sums
// are added in wave order.
__device__ __forceinline__ void router_task(const BlockParams &p, unsigned &gen, int task, unsigned char *lds) {
  constexpr int RB = kRouterRowBlock;
  const int nrb = (p.b + RB - 1) / RB;
  const int e = task / nrb, t0 = (task % nrb) * RB;
  const int w = tid() / MB_WAVE, q = tid() % MB_WAVE;
  double *red = reinterpret_cast<double *>(lds);  // [kWaves][RB]
  // Padding elements (past H, or rows past b) load zeros and add nothing.
  double acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.0;
  const rsrc_t rw = make_rsrc(p.router_w + (size_t)e * p.H), rx = make_rsrc(p.x);
  uint32_t xrow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) xrow[r] = t0 + r < p.b ? (uint32_t)(t0 + r) * (uint32_t)p.H * 2u : kOob;
  bool need_gen = gen == kGenPending;
  for (int h0 = 4 * q + 256 * w; h0 < p.H; h0 += 256 * kWaves * kRouterBatch) {
    f32x4_t wv[kRouterBatch];
    u32x2_t xv[kRouterBatch][RB];
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      const uint32_t h = (uint32_t)(h0 + 256 * kWaves * u);
      const bool in = h < (uint32_t)p.H;
      wv[u] = __builtin_bit_cast(f32x4_t, ld_b128(rw, in ? h * 4 : kOob));
#pragma unroll
      for (int r = 0; r < RB; ++r) xv[u][r] = ld_b64(rx, (in && xrow[r] != kOob) ? xrow[r] + h * 2 : kOob);
    }
    // The workgroup's generation, behind the wave's first router requests
    // (its waits for them do not include it).
    if (need_gen) {
      gen = load_generation(p.sync);
      need_gen = false;
    }
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        acc[r] = fma((double)bf16_bits_to_f32(xv[u][r][0] & 0xFFFFu), (double)wv[u][0], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[u][r][0] >> 16), (double)wv[u][1], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[u][r][1] & 0xFFFFu), (double)wv[u][2], acc[r]);
        acc[r] = fma((double)bf16_bits_to_f32(xv[u][r][1] >> 16), (double)wv[u][3], acc[r]);
      }
    }
  }
  // (A wave with no hidden elements here requests it now.)
  if (need_gen) gen = load_generation(p.sync);
  stamp(p, 23);
  double ws[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) ws[r] = wave_sum_dpp64(acc[r]);
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) red[w * RB + r] = ws[r];
  }
  __syncthreads();
  if (tid() < RB && t0 + (int)tid() < p.b) {
    double v = red[tid()];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) v += red[ww * RB + tid()];
    const size_t te = (size_t)(t0 + tid()) * p.E + e;
    const Deps d{p.sync, gen};
    st_tagged(make_rsrc(p.logits_t), (uint32_t)(te * 8), __float_as_uint((float)v), d.tag());
  }
  __syncthreads();  // (the workgroup's next task reuses the LDS)
  stamp(p, 22);
}

// Many rows: the logits of a tile of 16 rows x 16 experts over the
// contraction split q of router_ks (32-element chunks, dealt to the waves in
// turn), on the fp64 MFMA (bf16 x fp32 products are exact in fp64; each
// product added in fp64).  For a chunk, lane l (r = l % 16, g = l / 16)
// loads elements 8g .. 8g + 7 of row r's x and of expert r's router row;
// step s of eight multiplies element s: A[r][g] = x, B[g][r] = w, so the
// steps together sum the chunk.  The four waves' tiles are added in wave
// order; with several splits the last to finish adds the partials in split
// order; the sum is rounded once to fp32 and goes out as tagged logits.
constexpr int kRouterMmaAhead = 4;  // chunks requested ahead per wave
__device__ __forceinline__ void router_mma_task(const BlockParams &p, unsigned &gen, int task, unsigned char *lds) {
  const int lane = tid() % MB_WAVE, w = tid() / MB_WAVE, r = lane % 16, g = lane / 16;
  const int ks = p.router_ks, ET = (p.E + 15) / 16;
  const int tile = task / ks, q = task % ks, rt = tile / ET, et = tile % ET;
  const int kr = p.H / ks, k0 = q * kr, nchk = kr / 32;
  const int nw = (nchk - w + kWaves - 1) / kWaves;  // this wave's chunks: w, w + 4, ..
  const int row = rt * 16 + r, e = et * 16 + r;
  const uint32_t xrow = row < p.b ? (uint32_t)(((size_t)row * p.H + k0 + 8 * g) * 2) : kOob;
  const uint32_t wrow = e < p.E ? (uint32_t)(((size_t)e * p.H + k0 + 8 * g) * 4) : kOob;
  const rsrc_t rx = make_rsrc(p.x), rw = make_rsrc(p.router_w);
  u32x4_t xv[kRouterMmaAhead], w0[kRouterMmaAhead], w1[kRouterMmaAhead];
  auto req = [&](int c, int i) {
    const bool ok = c < nw;
    const uint32_t cw = (uint32_t)(w + kWaves * c) * 32u;
    xv[i] = ld_b128(rx, (ok && xrow != kOob) ? xrow + cw * 2u : kOob);
    w0[i] = ld_b128(rw, (ok && wrow != kOob) ? wrow + cw * 4u : kOob);
    w1[i] = ld_b128(rw, (ok && wrow != kOob) ? wrow + cw * 4u + 16u : kOob);
  };
#pragma unroll
  for (int i = 0; i < kRouterMmaAhead; ++i) req(i, i);
  if (gen == kGenPending) gen = load_generation(p.sync);
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < nw; c0 += kRouterMmaAhead) {
#pragma unroll
    for (int i = 0; i < kRouterMmaAhead; ++i) {
      if (c0 + i < nw) {
        const float wf[8] = {__uint_as_float(w0[i][0]), __uint_as_float(w0[i][1]), __uint_as_float(w0[i][2]),
                             __uint_as_float(w0[i][3]), __uint_as_float(w1[i][0]), __uint_as_float(w1[i][1]),
                             __uint_as_float(w1[i][2]), __uint_as_float(w1[i][3])};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint32_t xb = (s & 1) ? (xv[i][s / 2] >> 16) : (xv[i][s / 2] & 0xFFFFu);
          acc = mfma_f64(bf16_bits_to_f32(xb), wf[s], acc);
        }
      }
      req(c0 + kRouterMmaAhead + i, i);
    }
  }
  stamp(p, 23);
  // Lane l's element v is D[4 v + l / 16][l % 16]; added over the waves in order.
  double *red = reinterpret_cast<double *>(lds);  // [kWaves][4][64]
  int *flag = reinterpret_cast<int *>(lds + kWaves * 4 * MB_WAVE * sizeof(double));
#pragma unroll
  for (int v = 0; v < 4; ++v) red[(w * 4 + v) * MB_WAVE + lane] = acc[v];
  __syncthreads();
  const int i = tid() / 16, j = tid() % 16;  // this thread's tile element
  const int src = (i % 4) * 16 + j, v = i / 4;
  double sum = red[v * MB_WAVE + src];
#pragma unroll
  for (int ww = 1; ww < kWaves; ++ww) sum += red[(ww * 4 + v) * MB_WAVE + src];
  const int trow = rt * 16 + i, te = et * 16 + j;
  const Deps d{p.sync, gen};
  bool out = true;
  if (ks > 1) {
    const rsrc_t rp = make_rsrc(p.rtr_part);
    const uint64_t bits = __builtin_bit_cast(uint64_t, sum);
    st_co8(rp, (uint32_t)((((size_t)q * ((p.b + 15) / 16) * ET + tile) * 256 + tid()) * 8),
           u32x2_t{(uint32_t)bits, (uint32_t)(bits >> 32)});
    out = last_arrival(&p.rtr_cnt[tile], (unsigned)ks, flag);
    if (out) {
      u32x2_t pv[8];
      for (int q0 = 0; q0 < ks; q0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[u] = ld_co8(rp, q0 + u < ks
                                 ? (uint32_t)((((size_t)(q0 + u) * ((p.b + 15) / 16) * ET + tile) * 256 + tid()) * 8)
                                 : kOob);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const double pu = __builtin_bit_cast(double, ((uint64_t)pv[u][1] << 32) | pv[u][0]);
          if (q0 + u < ks) sum = (q0 + u == 0) ? pu : sum + pu;
        }
      }
      if (tid() == 0) __hip_atomic_store(&p.rtr_cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (out && trow < p.b && te < p.E) {
    const size_t idx = (size_t)trow * p.E + te;
    st_tagged(make_rsrc(p.logits_t), (uint32_t)(idx * 8), __float_as_uint((float)sum), d.tag());
  }
  __syncthreads();  // (the workgroup's next task reuses the LDS)
  stamp(p, 22);
}

// Many rows (more router tasks than workgroups at one expert each): the
// logits of kRouterExperts (4) experts for a block of 4 rows.  Same split of
// the hidden elements over the waves and lanes as router_task, the lane
// holding 16 fp64 sums; each (expert, row) sum is reduced across the wave
// (butterfly, the same in every lane) and then over the four waves in wave
// order, and rounded once to fp32.  The hidden states are read once per four
// experts instead of once per expert.
__device__ __forceinline__ void router_task_multi(const BlockParams &p, unsigned &gen, int task,
                                                  unsigned char *lds) {
  constexpr int RB = kRouterRowBlock, XE = kRouterExperts, kB = 2;  // blocks per request batch
  const int nrb = (p.b + RB - 1) / RB;
  const int e0 = (task / nrb) * XE, t0 = (task % nrb) * RB;
  const int w = tid() / MB_WAVE, q = tid() % MB_WAVE;
  double *red = reinterpret_cast<double *>(lds);  // [kWaves][XE * RB]
  double acc[XE][RB];
#pragma unroll
  for (int j = 0; j < XE; ++j)
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[j][r] = 0.0;
  const rsrc_t rw = make_rsrc(p.router_w), rx = make_rsrc(p.x);
  uint32_t xrow[RB], wrow[XE];
#pragma unroll
  for (int r = 0; r < RB; ++r) xrow[r] = t0 + r < p.b ? (uint32_t)(t0 + r) * (uint32_t)p.H * 2u : kOob;
#pragma unroll
  for (int j = 0; j < XE; ++j) wrow[j] = e0 + j < p.E ? (uint32_t)(e0 + j) * (uint32_t)p.H * 4u : kOob;
  bool need_gen = gen == kGenPending;
  for (int h0 = 4 * q + 256 * w; h0 < p.H; h0 += 256 * kWaves * kB) {
    f32x4_t wv[kB][XE];
    u32x2_t xv[kB][RB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const uint32_t h = (uint32_t)(h0 + 256 * kWaves * u);
      const bool in = h < (uint32_t)p.H;
#pragma unroll
      for (int j = 0; j < XE; ++j)
        wv[u][j] = __builtin_bit_cast(f32x4_t, ld_b128(rw, (in && wrow[j] != kOob) ? wrow[j] + h * 4 : kOob));
#pragma unroll
      for (int r = 0; r < RB; ++r) xv[u][r] = ld_b64(rx, (in && xrow[r] != kOob) ? xrow[r] + h * 2 : kOob);
    }
    if (need_gen) {
      gen = load_generation(p.sync);
      need_gen = false;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u)
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const double x0 = bf16_bits_to_f32(xv[u][r][0] & 0xFFFFu), x1 = bf16_bits_to_f32(xv[u][r][0] >> 16);
        const double x2 = bf16_bits_to_f32(xv[u][r][1] & 0xFFFFu), x3 = bf16_bits_to_f32(xv[u][r][1] >> 16);
#pragma unroll
        for (int j = 0; j < XE; ++j) {
          acc[j][r] = fma(x0, (double)wv[u][j][0], acc[j][r]);
          acc[j][r] = fma(x1, (double)wv[u][j][1], acc[j][r]);
          acc[j][r] = fma(x2, (double)wv[u][j][2], acc[j][r]);
          acc[j][r] = fma(x3, (double)wv[u][j][3], acc[j][r]);
        }
      }
  }
  if (need_gen) gen = load_generation(p.sync);
  stamp(p, 23);
#pragma unroll
  for (int j = 0; j < XE; ++j)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const double v = wave_sum(acc[j][r]);
      if (q == 0) red[w * XE * RB + j * RB + r] = v;
    }
  __syncthreads();
  if (tid() < XE * RB) {
    const int j = tid() / RB, r = tid() % RB;
    double v = red[tid()];
    for (int ww = 1; ww < kWaves; ++ww) v += red[ww * XE * RB + tid()];
    if (t0 + r < p.b && e0 + j < p.E) {
      const size_t te = (size_t)(t0 + r) * p.E + e0 + j;
      const Deps d{p.sync, gen};
      st_tagged(make_rsrc(p.logits_t), (uint32_t)(te * 8), __float_as_uint((float)v), d.tag());
    }
  }
  __syncthreads();  // (the workgroup's next task reuses the LDS)
  stamp(p, 22);
}

// ---------------------------------------------------------------- routing

// Order key of a candidate: larger is better.  Valid numbers above NaN, then
// the larger selection key, then the lower expert id; -0 counts as +0.
__device__ __forceinline__ unsigned long long order_key(float key, int e) {
  const float k = key + 0.0f;
  uint32_t u = 0;
  if (!isnan(k)) {
    const uint32_t bits = __float_as_uint(k);
    u = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  }
  return ((unsigned long long)u << 32) | (uint32_t)~(uint32_t)e;
}

// Wave-wide maximum of a 64-bit key, on every lane: DPP row shifts by 1, 2,
// 4, 8 leave each 16-lane row's maximum in its last lane, and two row
// broadcasts (15, 31) carry it to lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ void key_max_step(uint32_t &hi, uint32_t &lo) {
  const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWS, 0xF, false);
  const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWS, 0xF, false);
  const bool gt = h > hi || (h == hi && l > lo);
  hi = gt ? h : hi;
  lo = gt ? l : lo;
}
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long key) {
  uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
  key_max_step<0x111, 0xF>(hi, lo);  // row_shr:1
  key_max_step<0x112, 0xF>(hi, lo);  // row_shr:2
  key_max_step<0x114, 0xF>(hi, lo);  // row_shr:4
  key_max_step<0x118, 0xF>(hi, lo);  // row_shr:8
  key_max_step<0x142, 0xA>(hi, lo);  // row_bcast:15
  key_max_step<0x143, 0xC>(hi, lo);  // row_bcast:31
  return ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)hi, 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
}

// Wave-wide fp32 sum on every lane, by the same DPP tree as wave_max_key.
template <int CTRL, int ROWS>
__device__ __forceinline__ float sum_step(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF,
                                                                   false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = sum_step<0x111, 0xF>(v);
  v = sum_step<0x112, 0xF>(v);
  v = sum_step<0x114, 0xF>(v);
  v = sum_step<0x118, 0xF>(v);
  v = sum_step<0x142, 0xA>(v);
  v = sum_step<0x143, 0xC>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Workgroup fp32 sum (fixed order: the wave trees, then the waves in order)
// through red[slot * kWaves ..]; calls with different slots need no barrier
// between them.
__device__ __forceinline__ float wg_sum(float v, float *red, int slot) {
  v = wave_sum_dpp(v);
  if (tid() % MB_WAVE == 0) red[slot * kWaves + tid() / MB_WAVE] = v;
  __syncthreads();
  float t = red[slot * kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t += red[slot * kWaves + w];
  return t;
}

// One row's routing by one wave from its fp32 logits l[i] and expert biases
// bias[i] (expert lane + 64 i): multiplier, scores, keys = score + bias; then
// k rounds, each taking the largest remaining order key (the keys are
// distinct) into the next slot.  Then the fp32 weights in slot order.  Lane
// j < k gets slot j.
template <int PER>
__device__ __forceinline__ void route_one(const BlockParams &p, const float (&l)[PER], const float (&bias)[PER],
                                          int &out_id, float &out_w) {
  const int lane = tid() % MB_WAVE;
  float g[PER], sc[PER];
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
  // Order keys; lanes past E hold 0, below every candidate's key.
  unsigned long long key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = live[i] ? order_key(sc[i] + bias[i], lane + MB_WAVE * i) : 0ull;
  int my_id = 0;
  float my_sc = 0.f, sum = 0.f;
  for (int j = 0; j < p.k; ++j) {
    unsigned long long best = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) best = key[i] > best ? key[i] : best;
    const unsigned long long m = wave_max_key(best);
    const int id = uniform((int)~(uint32_t)m);
    const int src = id % MB_WAVE, part = id / MB_WAVE;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (i == part) {
        s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[i]), src));
        if (lane == src) key[i] = 0ull;  // taken
      }
    }
    sum = j == 0 ? s : sum + s;
    if (lane == j) {
      my_id = id;
      my_sc = s;
    }
  }
  out_id = my_id;
  const float den = sum + p.div_eps;
  const float q = my_sc / den;
  out_w = q * p.route_scale;
}

// Rows t_begin..t_end-1, one per wave in turn, from their fp32 logits: the
// caller's, or the router's tagged words, polled until this launch's are all
// there (the expert biases are requested first).  The ids and weights go out
// as tagged words to every copy of the routes, and to the caller's routing
// outputs (ids, weights, logits) when it asked for them.
template <int PER>
__device__ __forceinline__ void route_rows(const BlockParams &p, const Deps &d, int t_begin, int t_end) {
  const int lane = tid() % MB_WAVE;
  const rsrc_t rl = make_rsrc(p.logits_t), rb = make_rsrc(p.bias), rr = make_rsrc(p.routes_t);
  float bias[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + MB_WAVE * i;
    bias[i] = __uint_as_float(ld_b32(rb, e < p.E ? (uint32_t)e * 4u : kOob));
  }
  const int R2 = 2 * p.b * p.k;
  for (int t = t_begin + (int)(tid() / MB_WAVE); t < t_end; t += kWaves) {
    float l[PER];
    if (p.logits_in) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + MB_WAVE * i;
        l[i] = e < p.E ? p.logits[(size_t)t * p.E + e] : 0.f;
      }
    } else {
      uint32_t off[PER];
      u32x2_t v[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + MB_WAVE * i;
        off[i] = e < p.E ? (uint32_t)(((size_t)t * p.E + e) * 8) : kOob;
        v[i] = ld_co8(rl, off[i]);
      }
      await_tagged(d, rl, off, v);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        l[i] = __uint_as_float(v[i][0]);
        const int e = lane + MB_WAVE * i;
        if (p.logits && e < p.E) p.logits[(size_t)t * p.E + e] = l[i];
      }
    }
    stamp(p, 12);
    int id;
    float w;
    route_one<PER>(p, l, bias, id, w);
    // The kRouteReps copies of the row's ids and weights, one word per lane:
    // lane l stores slot l % k of copy (l / k) % kRouteReps, an id below
    // kRouteReps k and a weight above (the slot's values from lane l % k).
    const uint32_t tag = d.tag();
    const int nst = 2 * kRouteReps * p.k;
#pragma unroll 1
    for (int s0 = 0; s0 < nst; s0 += MB_WAVE) {
      const int si = s0 + lane, j = si % p.k, c = (si / p.k) % kRouteReps, kind = si / (kRouteReps * p.k);
      const int sid = __shfl(id, j, MB_WAVE);
      const float sw = __shfl(w, j, MB_WAVE);
      if (si < nst)
        st_tagged(rr, (uint32_t)(((size_t)c * R2 + kind * (R2 / 2) + t * p.k + j) * 8),
                  kind ? __float_as_uint(sw) : (uint32_t)sid, tag);
    }
    if (lane < p.k && p.routing_out) {
      const int r = t * p.k + lane;
      p.ids[r] = id;
      p.wts[r] = w;
    }
  }
}

__device__ __forceinline__ void route_dispatch(const BlockParams &p, const Deps &d, int t0, int t1) {
  // The host sends larger expert counts to the per-step kernels.
  if (p.E <= 64) route_rows<1>(p, d, t0, t1);
  else if (p.E <= 128) route_rows<2>(p, d, t0, t1);
  else route_rows<4>(p, d, t0, t1);
}

// Inclusive prefix sum over the wave's 64 lanes (DPP: row shifts 1, 2, 4, 8,
// then the row broadcasts 15 and 31 add the earlier rows' totals).
template <int CTRL, int ROWS>
__device__ __forceinline__ int scan_step(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v = scan_step<0x111, 0xF>(v);
  v = scan_step<0x112, 0xF>(v);
  v = scan_step<0x114, 0xF>(v);
  v = scan_step<0x118, 0xF>(v);
  v = scan_step<0x142, 0xA>(v);
  v = scan_step<0x143, 0xC>(v);
  return v;
}

// Exclusive prefix sum over the workgroup of one value per thread, in a fixed
// order; `total` receives the sum.  `red` holds kWaves ints.
__device__ __forceinline__ int wg_excl_scan(int v, int *red, int &total) {
  const int lane = tid() % MB_WAVE, wave = tid() / MB_WAVE;
  const int x = wave_incl_scan(v);
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

// Many-rows instance: each active expert's rows in passes of up to 32 (the
// units' two 16-column MFMA blocks), every pass an entry of vact with units
// of its own, in the order of act: an expert with more rows than one pass
// takes more workgroups, where a unit covering all its rows would stream the
// expert's weights once per pass.
__device__ __forceinline__ void build_passes(const RouteLds &R) {
  const int na = uniform(*R.nact), a = tid();
  int e = 0, np = 0;
  if (a < na) {
    e = R.act[a];
    np = (R.off[e + 1] - R.off[e] + 31) / 32;
  }
  int tot = 0;
  const int pos = wg_excl_scan(np, R.red, tot);
  for (int j = 0; j < np; ++j) R.vact[pos + j] = (uint16_t)(e | (j << 8));
  if (tid() == 0) R.nact[2] = tot;
  __syncthreads();
}

// Route grouping from R.ids: per-expert bitmaps over rows (LDS atomics, so
// independent of order), popcount counts, exclusive scans for offsets and
// the active list, and route (t, j) of expert e at offset[e] + the number of
// earlier rows that chose e (routes sorted by (expert, t*k + j)).
// Row t of route r = t k + j joins expert e's bitmap (R.bits zeroed at the
// start of the launch).
__device__ __forceinline__ void mark_route(const BlockParams &p, const RouteLds &R, int r, int e) {
  const int W = (p.b + 63) / 64, t = r / p.k;
  atomicOr(&R.bits[e * W + t / 64], 1ull << (t & 63));
}

// (Expects every route marked, and a barrier since.)  by_count: the
// workgroup's own list of active experts (R.act) in descending order of
// their route counts, ties by id (the routing outputs keep id order): the
// many-rows instance claims its rounds of up units, then of down units, in
// list order, the costliest first, each expert's rows in passes of up to 32
// (build_passes).  (Measured against ascending order and against down units
// in the reverse order: faster at every size but the literal skew's, where
// ascending is ~3 us faster.)
__device__ __forceinline__ void group_routes(const BlockParams &p, const RouteLds &R, bool out,
                                             bool by_count = false) {
  const int W = (p.b + 63) / 64;
  const int Rn = p.b * p.k;
  const int e0 = tid() * 4;
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
  // Counts (< 2^16) and active flags in one scan: count in the low half.
  int tot = 0;
  const int packed = wg_excl_scan(csum | (asum << 16), R.red, tot);
  int oc = packed & 0xFFFF, oa = packed >> 16;
  const int tot_c = tot & 0xFFFF, tot_a = tot >> 16;
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
  if (tid() == 0) {
    R.off[p.E] = tot_c;
    *R.nact = tot_a;
    if (out) {
      p.offset[p.E] = tot_c;
      *p.n_active = tot_a;
    }
  }
  __syncthreads();
  for (int r = tid(); r < Rn; r += kThreads) {
    const int t = r / p.k, e = R.ids[r];
    const unsigned long long *b = R.bits + e * W;
    int rank = 0;
    for (int w = 0; w < t / 64; ++w) rank += __popcll(b[w]);
    rank += __popcll(b[t / 64] & ((1ull << (t & 63)) - 1ull));
    R.rl[R.off[e] + rank] = r;
    if (out) p.route_list[R.off[e] + rank] = r;
  }
  __syncthreads();
  if (by_count) {
    static_assert(kBlockMaxExperts <= kThreads, "one active expert per thread");
    const int na = tot_a, a = tid();
    int e = -1, rk = 0;
    if (a < na) {
      e = R.act[a];
      const int c = R.off[e + 1] - R.off[e];
      for (int a2 = 0; a2 < na; ++a2) {
        const int e2 = R.act[a2], c2 = R.off[e2 + 1] - R.off[e2];
        rk += (c2 > c || (c2 == c && e2 < e)) ? 1 : 0;
      }
    }
    __syncthreads();
    if (e >= 0) R.act[rk] = e;
    __syncthreads();
    build_passes(R);
  }
}

// Route task: rows 4 task .. +3, one per wave.
__device__ __forceinline__ void route_task(const BlockParams &p, const Deps &d, int task) {
  const int t0 = task * kWaves, t1 = min(p.b, t0 + kWaves);
  route_dispatch(p, d, t0, t1);
  stamp(p, 14);
}

// Words of the tagged routes each thread polls at once.
constexpr int kRouteBatch = 2;

// The routing state a workgroup needs before its first expert unit: the
// routes (from the caller, or polled from this workgroup's copy of the tagged
// routes), then the grouping; by_count: the many-rows instance's order and
// passes (group_routes).
__device__ __forceinline__ void prepare_routing(const BlockParams &p, const Deps &d, const RouteLds &R,
                                                bool by_count = false) {
  const bool out = p.routing_out && blockIdx.x == 0;
  if (p.route_given) {
    // From the caller (mb_experts).
    for (int i = tid(); i < p.b * p.k; i += kThreads) {
      R.ids[i] = (unsigned)p.ids[i] < (unsigned)p.E ? p.ids[i] : 0;  // (the caller's ids are below E)
      R.w[i] = p.wts[i];
      R.rl[i] = p.route_list[i];
    }
    for (int i = tid(); i <= p.E; i += kThreads) R.off[i] = p.offset[i];
    for (int i = tid(); i < p.E; i += kThreads) R.act[i] = p.active[i];
    if (tid() == 0) *R.nact = *p.n_active;
    __syncthreads();
    if (by_count) build_passes(R);
    return;
  }
  const int Rn = p.b * p.k, R2 = 2 * Rn;
  const rsrc_t rr = make_rsrc(p.routes_t + (size_t)(blockIdx.x % kRouteReps) * R2 * 2);
  for (int w0 = 0; w0 < R2; w0 += kThreads * kRouteBatch) {
    uint32_t off[kRouteBatch];
    u32x2_t v[kRouteBatch];
#pragma unroll
    for (int i = 0; i < kRouteBatch; ++i) {
      const int w = w0 + (int)tid() + kThreads * i;
      off[i] = w < R2 ? (uint32_t)w * 8u : kOob;
      v[i] = ld_co8(rr, off[i]);
    }
    await_tagged(d, rr, off, v);
    stamp(p, 13);
#pragma unroll
    for (int i = 0; i < kRouteBatch; ++i) {
      const int w = w0 + (int)tid() + kThreads * i;
      if (w < Rn) {
        // (An id is below E unless a wait gave up and the word is stale or
        // never written: then expert 0, so that every index stays in range.)
        const int e = v[i][0] < (uint32_t)p.E ? (int)v[i][0] : 0;
        R.ids[w] = e;
        mark_route(p, R, w, e);
      } else if (w < R2) {
        R.w[w - Rn] = __uint_as_float(v[i][0]);
      }
    }
  }
  __syncthreads();
  group_routes(p, R, out, by_count);
}

// ---------------------------------------------------------------- projections

constexpr size_t kProjRedBytes = 4 * kWaves * MB_WAVE * sizeof(f32x4_t);
__device__ __forceinline__ int *proj_flag(unsigned char *lds) {
  return reinterpret_cast<int *>(lds + kProjRedBytes);
}

// Wide projection tile: out[t, n] over features n0 = 64 gi .. +63 (wave w:
// n0 + 16 w .. +15, its weights in the MFMA A operand), every row t, and the
// contraction split q of ks (elements q kr .. + kr, kr = kdim / ks).  The
// workgroup stages the activations a[t, k] of the split once, in segments,
// in `stage` (read coherently when another workgroup of the launch wrote
// them: kCoherentA); each wave streams its own weights kWideRing chunks of
// 32 elements ahead.  Rows go in passes of up to 64 (four 16-row MFMA
// blocks); features and rows past the ends load zeros and are not stored.
// With ks == 1 the result goes to `out` in bf16 (when not NULL) and to out_t
// as tagged words (when not NULL: two bf16 per word), else the fp32 partial
// to part[q].  `wait` runs after the first weight requests, before the first
// activation request.
// Tasks of the wide projections beyond 64 rows: (tile, split) gq and 64-row
// block rb, numbered so that the row blocks of one (tile, split) are eight
// task numbers apart -- on workgroups of the same XCD (the grid is a
// multiple of eight), whose L2 then serves their common weights.  The count
// is rounded up to whole groups of eight: gq past the last is no task.
__device__ __forceinline__ void row_block_task(int i, int row_blocks, int &gq, int &rb) {
  const int hi = i / 8;
  rb = hi % row_blocks;
  gq = (hi / row_blocks) * 8 + i % 8;
}

constexpr int kWideRing = 8;
constexpr int kWideCols = 16 * kWaves;
// 16-byte activation pieces per thread and segment: the stage holds 64 rows
// x 256, 32 x 512 or 16 x 1024 elements, 2048 pieces.
constexpr int kWidePieces = 2048 / kThreads;
//
// kRB (the kernel's many-rows instances): only rows t_begin .. t_end - 1
// (one 64-row block of a task of its own), the weights read cached when
// `cached` (other blocks' tasks read them too).  Without it, every row and
// nontemporal weights, and none of that bookkeeping in the registers.
template <bool kCoherentA, bool kRB = false, typename Wait>
__device__ __forceinline__ void proj_wide(rsrc_t ra, const uint16_t *w, bool wpk, int rows, int n_out, int kdim,
                                          int gi, int q, int ks, float *part, uint16_t *out, uint32_t *out_t,
                                          uint32_t tag, unsigned char *stage, Wait wait, int t_begin = 0,
                                          int t_end = 0, bool cached = false) {
  const int lane = (int)(tid() % MB_WAVE), wave = (int)(tid() / MB_WAVE), g = lane >> 4, r16 = lane & 15;
  const int kr = kdim / ks, k0 = q * kr, nch = kr / 32;
  const int f = gi * kWideCols + 16 * wave + r16;  // this lane's weight row
  const rsrc_t rw = make_rsrc(w);
  // (wpk: w in the streaming layout, each chunk's wave load one kilobyte.)
  const uint32_t wrow = f >= n_out ? kOob
                        : wpk      ? (uint32_t)packed_offset(gi * kWaves + wave, kdim, k0, lane)
                                   : (uint32_t)(((size_t)f * kdim + k0 + 8 * g) * 2);
  const uint32_t wstep = wpk ? 1024u : 64u;
  auto wload = [&](int c) {
    const uint32_t o = (wrow != kOob && c < nch) ? wrow + (uint32_t)c * wstep : kOob;
    return (kRB && cached) ? ld_b128(rw, o) : ld_nt16(rw, o);
  };
  const int tb = kRB ? t_begin : 0, te = kRB ? min(rows, t_end) : rows;
  const rsrc_t ro = make_rsrc(out), rp = make_rsrc(part), rt = make_rsrc(out_t);
  for (int t0 = tb; t0 < te; t0 += 64) {
    // (kRB: always four 16-row blocks -- rows past the end are staged as
    // zeros and not stored -- so the products have no branches.)
    const int rp_ = min(64, rows - t0), nb = kRB ? 4 : (rp_ + 15) / 16;
    // Segment length (elements, a multiple of 32 kWideRing): rows x segment fits the stage.
    const int seg = kRB ? 256 : min((rp_ <= 16 ? 1024 : rp_ <= 32 ? 512 : 256), ((kr + 255) / 256) * 256);
    const int srow = seg * 2 + 16;
    u32x4_t W[kWideRing];
#pragma unroll
    for (int r = 0; r < kWideRing; ++r) W[r] = wload(r);
    if (t0 == tb) wait();
    f32x4_t acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Rows t0 .. t0 + 16 nb, elements k0 + 32 s0 .. + seg, in 16-byte
    // pieces (at most kWidePieces per thread): requested into registers one
    // segment ahead, so that a segment's loads overlap the one before.
    const int ppr = seg / 8, pieces = 16 * nb * ppr;
    u32x4_t v[kWidePieces];
    auto act_req = [&](int s0) {
#pragma unroll
      for (int u = 0; u < kWidePieces; ++u) {
        const int i = (int)tid() + kThreads * u;
        const int m = i / ppr, pc = i % ppr;
        const int t = t0 + m, k = 32 * s0 + 8 * pc;
        const bool in = i < pieces && t < rows && k < kr;
        const uint32_t off = in ? (uint32_t)(((size_t)t * kdim + k0 + k) * 2) : kOob;
        v[u] = kCoherentA ? ld_co16(ra, off) : ld_b128(ra, off);
      }
    };
    act_req(0);
    for (int s0 = 0; s0 < nch; s0 += seg / 32) {
#pragma unroll
      for (int u = 0; u < kWidePieces; ++u) {
        const int i = (int)tid() + kThreads * u;
        if (i < pieces) *reinterpret_cast<u32x4_t *>(stage + (i / ppr) * srow + (i % ppr) * 16) = v[u];
      }
      __syncthreads();
      if (s0 + seg / 32 < nch) act_req(s0 + seg / 32);
      for (int c0 = s0; c0 < s0 + seg / 32 && c0 < nch; c0 += kWideRing) {
#pragma unroll
        for (int r = 0; r < kWideRing; ++r) {
          const unsigned char *bp = stage + r16 * srow + ((c0 + r - s0) * 32 + 8 * g) * 2;
          if constexpr (kRB) {
            // The four blocks' operands read together, then the products.
            u32x4_t B[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) B[b] = *reinterpret_cast<const u32x4_t *>(bp + 16 * b * srow);
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = mfma_bf16(as_bf16x8(W[r]), as_bf16x8(B[b]), acc[b]);
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (b < nb)
                acc[b] = mfma_bf16(as_bf16x8(W[r]),
                                   as_bf16x8(*reinterpret_cast<const u32x4_t *>(bp + 16 * b * srow)), acc[b]);
          }
          W[r] = wload(c0 + kWideRing + r);
        }
      }
      __syncthreads();
    }
    // Lane: features 4 g .. + 3 of the wave's 16 (rows of D), row r16 of each block.
    const int n = gi * kWideCols + 16 * wave + 4 * g;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int t = t0 + 16 * b + r16;
      if (b >= nb || t >= rows || n >= n_out) continue;
      if (ks == 1) {
        const uint32_t lo = pack_bf16x2(acc[b][0], acc[b][1]), hi = pack_bf16x2(acc[b][2], acc[b][3]);
        if (out) st_co8(ro, (uint32_t)(((size_t)t * n_out + n) * 2), u32x2_t{lo, hi});
        if (out_t) st_co16(rt, (uint32_t)(((size_t)t * n_out + n) * 4), u32x4_t{lo, tag, hi, tag});
      } else
        st_co16(rp, (uint32_t)((((size_t)q * rows + t) * n_out + n) * 4), __builtin_bit_cast(u32x4_t, acc[b]));
    }
  }
}

// The last split of a wide tile: out[t, n] = bf16(sum over q of part[q][t][n]),
// in split order, for the tile's 64 features and every row; to `out` (when
// not NULL) and as tagged words to out_t (when not NULL).
__device__ __forceinline__ void proj_wide_sum(const float *part, uint16_t *out, uint32_t *out_t, uint32_t tag,
                                              int rows, int n_out, int gi, int ks, int t_begin = 0,
                                              int t_end = 1 << 30) {
  const rsrc_t rp = make_rsrc(part), ro = make_rsrc(out), rt = make_rsrc(out_t);
  const int tb = t_begin, te = min(rows, t_end);
  for (int idx = (int)tid(); idx < (te - tb) * (kWideCols / 4); idx += kThreads) {
    const int t = tb + idx / (kWideCols / 4), n = gi * kWideCols + 4 * (idx % (kWideCols / 4));
    if (n >= n_out) continue;
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < ks; q0 += 8) {
      f32x4_t pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pv[u] = __builtin_bit_cast(
            f32x4_t, ld_co16(rp, q0 + u < ks ? (uint32_t)((((size_t)(q0 + u) * rows + t) * n_out + n) * 4) : kOob));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u < ks) v = (q0 + u == 0) ? pv[u] : v + pv[u];
    }
    const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
    if (out) st_co8(ro, (uint32_t)(((size_t)t * n_out + n) * 2), u32x2_t{lo, hi});
    if (out_t) st_co16(rt, (uint32_t)(((size_t)t * n_out + n) * 4), u32x4_t{lo, tag, hi, tag});
  }
}

// Unpooler task at few rows (b <= 16): u[t, n] = sum_k moe_out[t, k] Wu[n, k]
// over features n0 = 32 grp .. + 31 (two 16-feature MFMA tiles, the weights
// in the A operand) and the contraction split q of ks (32-element chunks
// [q cps, (q + 1) cps), dealt to the waves in turn), for every row t (the B
// operand: lane r16 reads row r16 of the MoE output, from the copy `mo`,
// which the finalize tasks of the launch write chunk by chunk).
// Every weight chunk of the task is requested before the wait for the
// finalize tasks (kUnpoolChunks per wave at most: the host sizes the split
// so), so that only the MoE output is read after it.  The waves' sums are
// added in wave order through LDS; the fp32 partial goes to part[q]
// ([ks][b][H]), or u in bf16 when ks == 1.
constexpr int kUnpoolActBatch = 4;  // activation chunks a wave requests at once
__device__ __forceinline__ void unpool_task(const BlockParams &p, const Deps &d, const uint16_t *mo, int task,
                                            unsigned char *lds) {
  const Lane L;
  const int P = p.P, H = p.H, ks = p.unpool_ks;
  const int grp = task / ks, q = task % ks;
  const int nch = P / 32, cps = (nch + ks - 1) / ks;
  const int c_begin = q * cps, c_end = min(nch, c_begin + cps);
  const int n0 = grp * 16 * kUnpoolTiles;
  const bool wpk = p.unpool_wp != nullptr;  // (the streaming layout)
  const rsrc_t rw = make_rsrc(wpk ? p.unpool_wp : p.unpool_w), ra = make_rsrc(mo);
  const uint32_t wstep = wpk ? 1024u : 64u;
  u32x4_t W[kUnpoolTiles][kUnpoolChunks];
#pragma unroll
  for (int t = 0; t < kUnpoolTiles; ++t) {
    const int row = n0 + 16 * t + L.r16;
    const uint32_t wrow = row >= H ? kOob
                          : wpk    ? (uint32_t)packed_offset(n0 / 16 + t, P, 0, L.lane)
                                   : (uint32_t)(((size_t)row * P + 8 * L.g) * 2);
#pragma unroll
    for (int i = 0; i < kUnpoolChunks; ++i) {
      const int c = c_begin + L.wave + kWaves * i;
      W[t][i] = ld_nt16(rw, (wrow != kOob && c < c_end) ? wrow + (uint32_t)c * wstep : kOob);
    }
  }
  wait_step(d, kCtrFin, p.n_fin);
  f32x4_t acc[kUnpoolTiles];
#pragma unroll
  for (int t = 0; t < kUnpoolTiles; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // (mpk: the finalize tasks' copy, chunk by chunk: moe_rep_off.)
  const bool mpk = p.n_fin > 0;
  const uint32_t arow = L.r16 >= p.b ? kOob
                        : mpk         ? (uint32_t)(L.r16 * 64 + L.g * 16)
                                      : (uint32_t)(((size_t)L.r16 * P + 8 * L.g) * 2);
  const uint32_t astep = mpk ? (uint32_t)p.b * 64u : 64u;
  // Activations in batches, the next batch requested before the current
  // one's products (so the requests overlap); batches past this wave's last
  // chunk are skipped.
  constexpr int NB = kUnpoolChunks / kUnpoolActBatch;
  static_assert(kUnpoolChunks % kUnpoolActBatch == 0, "whole batches");
  const int nbw = uniform((c_end - c_begin - L.wave + kWaves * kUnpoolActBatch - 1) / (kWaves * kUnpoolActBatch));
  u32x4_t A[2][kUnpoolActBatch];
  auto act_batch = [&](int b, u32x4_t(&dst)[kUnpoolActBatch]) {
#pragma unroll
    for (int i = 0; i < kUnpoolActBatch; ++i) {
      const int c = c_begin + L.wave + kWaves * (b * kUnpoolActBatch + i);
      dst[i] = ld_co16(ra, (arow != kOob && c < c_end) ? arow + (uint32_t)c * astep : kOob);
    }
  };
  act_batch(0, A[0]);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= nbw) break;
    if (b + 1 < NB && b + 1 < nbw) act_batch(b + 1, A[(b + 1) % 2]);
#pragma unroll
    for (int i = 0; i < kUnpoolActBatch; ++i)
#pragma unroll
      for (int t = 0; t < kUnpoolTiles; ++t)
        acc[t] = mfma_bf16(as_bf16x8(W[t][b * kUnpoolActBatch + i]), as_bf16x8(A[b % 2][i]), acc[t]);
  }
  f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);  // [kWaves][kUnpoolTiles][64]
#pragma unroll
  for (int t = 0; t < kUnpoolTiles; ++t) red[(L.wave * kUnpoolTiles + t) * MB_WAVE + L.lane] = acc[t];
  __syncthreads();
  // Wave t (< kUnpoolTiles): tile t; lane: row r16, features 4 g .. + 3.
  if (L.wave < kUnpoolTiles && L.r16 < p.b) {
    const int t = L.wave;
    f32x4_t v = red[t * MB_WAVE + L.lane];
    for (int w = 1; w < kWaves; ++w) v += red[(w * kUnpoolTiles + t) * MB_WAVE + L.lane];
    const int n = n0 + 16 * t + 4 * L.g;
    if (n < H) {
      if (ks == 1)
        st_co8(make_rsrc(p.u), (uint32_t)(((size_t)L.r16 * H + n) * 2),
               u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      else
        st_co16(make_rsrc(p.unpool_part), (uint32_t)((((size_t)q * p.b + L.r16) * H + n) * 4),
                __builtin_bit_cast(u32x4_t, v));
    }
  }
}

// Optional pre-expert norm of h row t: thread i takes elements 2i + 512 m,
// +1 (one tagged word of the pooler's output), kBoundBatch of them per
// request, polled until this launch's.  The normed row goes out as tagged
// words (hn_t) and, when asked for, in bf16 to h.
__device__ __forceinline__ void prenorm_task(const BlockParams &p, const Deps &d, int t,
                                             unsigned char *lds) {
  float *red = reinterpret_cast<float *>(lds);
  const uint32_t W = (uint32_t)p.P / 2;  // words per row
  const rsrc_t rh = make_rsrc(p.h_t + (size_t)t * W * 2), rn = make_rsrc(p.hn_t + (size_t)t * W * 2),
               rw = make_rsrc(p.pre_norm_w), ro = make_rsrc(p.h + (size_t)t * p.P);
  float ss = 0.f;
  for (uint32_t w0 = tid(); w0 < W; w0 += kThreads * kBoundBatch) {
    uint32_t off[kBoundBatch];
    u32x2_t v[kBoundBatch];
#pragma unroll
    for (int m = 0; m < kBoundBatch; ++m) {
      const uint32_t w = w0 + kThreads * m;
      off[m] = w < W ? w * 8u : kOob;
      v[m] = ld_co8(rh, off[m]);
    }
    await_tagged(d, rh, off, v);
#pragma unroll
    for (int m = 0; m < kBoundBatch; ++m) {
      const float a = bf16_bits_to_f32(v[m][0] & 0xFFFFu), b = bf16_bits_to_f32(v[m][0] >> 16);
      ss += a * a + b * b;
    }
  }
  ss = wg_sum(ss, red, 0);
  const float rs = 1.0f / sqrtf(ss / (float)p.P + p.norm_eps);
  const uint32_t tag = d.tag();
  for (uint32_t w0 = tid(); w0 < W; w0 += kThreads * kBoundBatch) {
    uint32_t v[kBoundBatch], wv[kBoundBatch];
#pragma unroll
    for (int m = 0; m < kBoundBatch; ++m) {
      const uint32_t w = w0 + kThreads * m;
      v[m] = ld_co4(rh, w < W ? w * 8u : kOob);  // (this thread saw these words tagged above)
      wv[m] = ld_b32(rw, w < W ? w * 4u : kOob);
    }
#pragma unroll
    for (int m = 0; m < kBoundBatch; ++m) {
      const uint32_t w = w0 + kThreads * m;
      if (w >= W) break;
      const float a = bf16_bits_to_f32(v[m] & 0xFFFFu) * rs, b = bf16_bits_to_f32(v[m] >> 16) * rs;
      const float wa = bf16_bits_to_f32(wv[m] & 0xFFFFu), wb = bf16_bits_to_f32(wv[m] >> 16);
      const uint32_t o = pack_bf16x2(a * wa, b * wb);
      st_tagged(rn, w * 8u, o, tag);
      if (p.h_plain) st_co4(ro, w * 4u, o);
    }
  }
  __syncthreads();  // (the workgroup's next task reuses the LDS)
}

// ---------------------------------------------------------------- experts

// Issue priority of the waves streaming expert units: the workgroups
// sharing a CU are launched one after another (slot = blockIdx / CUs), and
// among waves of equal priority the oldest issues first, which leaves the
// waves of the later workgroups on a CU behind -- and a down unit waits for
// the slowest up unit of its expert.  So from its first round of chunks on,
// the later a workgroup's slot, the higher its waves' priority (1, 2, 3); the
// first requests of the units phase go out oldest first, at priority 0.
__device__ __forceinline__ void set_slot_priority(int slot) {
  if (slot <= 0) __builtin_amdgcn_s_setprio(1);
  else if (slot == 1) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
}

// Where a wave finds the two 16-row MXFP4 tiles of a unit: codes of chunk c
// of tile 0 / 1 at o0 / o1 + wstride * c in rw (o0 / o1 already at this
// lane's 16 bytes), the scales of chunks c .. c + 3 at so0 / so1 + sstride * c
// in rs (vec: one 16-byte load per 4 chunks, else one 4-byte load per chunk).
struct MxTiles {
  rsrc_t rw, rs;
  uint32_t o0, o1, so0, so1, wstride, sstride;
  int smode;  // kScalesRow4, kScalesRow16 or kScalesLane (what one scale load holds)
};
// A lane's scale load per four chunks: the row's four 4-byte words (one per
// chunk, byte g = block g), as one 16-byte load or four 4-byte loads; or the
// lane's own 4-byte word (byte j = its block of chunk j).
constexpr int kScalesRow4 = 0, kScalesRow16 = 1, kScalesLane = 2;

// The tiles of rows r0 .. r0 + 15 and r1 .. r1 + 15 of one expert's matrix of
// `kdim`-element rows, in the caller's row-major layout: lane l reads row
// l % 16, bytes 64 c + 16 (l / 16) of each 64-byte chunk c.
__device__ __forceinline__ MxTiles mx_plain(const uint8_t *codes, const uint8_t *scales, int r0, int r1, int kdim,
                                            int lane) {
  const uint32_t r16 = (uint32_t)(lane & 15), g = (uint32_t)(lane >> 4);
  const uint32_t rb = (uint32_t)kdim / 2, sb = (uint32_t)kdim / 32;
  return MxTiles{make_rsrc(codes), make_rsrc(scales), (r0 + r16) * rb + 16 * g, (r1 + r16) * rb + 16 * g,
                 (r0 + r16) * sb, (r1 + r16) * sb, 64u, 4u, (kdim / 128) % 4 == 0 ? kScalesRow16 : kScalesRow4};
}

// Unit `unit` of one section of the streaming layout (mb_pack_experts): per
// chunk the two tiles' 1 KB wave loads follow each other, lane l at 16 l;
// per group of four chunks the two tiles' 256-byte wave loads of scales, lane
// l at 4 l (the scales its codes need: row l % 16, block l / 16, four chunks).
__device__ __forceinline__ MxTiles mx_packed(const uint8_t *codes, const uint8_t *scales, int unit, int kdim,
                                             int lane) {
  const uint32_t nch = (uint32_t)kdim / 128, ngr = (nch + 3) / 4;
  const uint32_t o = (uint32_t)unit * nch * 2048u + 16u * (uint32_t)lane;
  const uint32_t so = (uint32_t)unit * ngr * 512u + 4u * (uint32_t)lane;
  return MxTiles{make_rsrc(codes), make_rsrc(scales), o, o + 1024u, so, so + 256u, 2048u, 128u, kScalesLane};
}

// Activation rows per pass over a unit's weights: 8, 16 or 32 (as one or two
// 16-column MFMA blocks); more rows take several passes.
__device__ __forceinline__ int pass_rows(int nrows) { return nrows <= 8 ? 8 : nrows <= 16 ? 16 : 32; }

// ---- activation staging

// Where the activation rows of a unit come from: a bf16 matrix, read
// coherently (the caller wrote it, or another workgroup did before counter
// `ready` reached `target`: the workgroup waits for that once its weights
// are requested), or the same matrix as tagged words (two bf16 and the
// writer's tag per 8 bytes: the pooler's h, the up units' act), polled until
// every word the unit reads carries this launch's tag.
struct ActSrc {
  rsrc_t r;
  bool tagged;
  const unsigned *ready = nullptr;
  unsigned target = 0;
};

// One batch of staging loads in flight: kStagePieces pieces of 8 elements
// per thread, piece n being elements e[n] .. + 8 of the matrix (kOob:
// padding, which loads zeros).  (Small batches: a tagged piece takes 8
// registers until it arrives, and a down unit holds all its weights then.)
constexpr int kStagePieces = 2;
static_assert(kSegLoads % kStagePieces == 0, "whole batches per segment");
struct StageBatch {
  uint32_t e[kStagePieces];
  u32x4_t a[kStagePieces], b[kStagePieces];
};

// Whether batch n0 (its first piece index per thread) holds a piece of one of
// the pass's vrows valid rows (ppr pieces per row); the other batches are
// padding only and skipped (their rows' columns are not stored).
__device__ __forceinline__ bool batch_needed(int n0, int ppr, int vrows) { return (kThreads * n0) / ppr < vrows; }

// Request batch n0 of the staging of the segment from chunk seg0 (segn
// chunks, ppr 16-byte pieces per row): piece q = tid + kThreads (n0 + n) is
// pass row m = q / ppr, elements 128 seg0 + 8 (q % ppr) .. + 8 of it; row_e(m)
// is the matrix element of row m's element 0, or kOob.  Pieces past the
// segment's chunks, and rows past pr or without a row, are padding.
template <typename RowE>
__device__ __forceinline__ void stage_issue(const ActSrc &A, RowE row_e, int pr, int seg0, int segn, int ppr, int n0,
                                            StageBatch &S) {
#pragma unroll
  for (int n = 0; n < kStagePieces; ++n) {
    const int q = (int)tid() + kThreads * (n0 + n);
    const int m = q / ppr, pc = q % ppr;
    const uint32_t ro = m < pr ? row_e(m) : kOob;
    S.e[n] = (ro != kOob && pc < segn * 16) ? ro + (uint32_t)(seg0 * 128 + pc * 8) : kOob;
    if (A.tagged) {
      S.a[n] = ld_co16(A.r, S.e[n] != kOob ? S.e[n] * 4u : kOob);
      S.b[n] = ld_co16(A.r, S.e[n] != kOob ? S.e[n] * 4u + 16u : kOob);
    } else {
      S.a[n] = ld_co16(A.r, S.e[n] != kOob ? S.e[n] * 2u : kOob);
    }
  }
}

__device__ __forceinline__ bool stage_piece_ready(const StageBatch &S, int n, uint32_t tag) {
  return S.e[n] == kOob || (S.a[n][1] == tag && S.a[n][3] == tag && S.b[n][1] == tag && S.b[n][3] == tag);
}

// The batch's pieces (8 bf16 each) once they arrived; tagged, once every word
// carries this launch's tag (the others requested again).  Bounded like
// poll_ge.
__device__ __forceinline__ void stage_complete(const Deps &d, const ActSrc &A, StageBatch &S,
                                               u32x4_t (&v)[kStagePieces]) {
  if (A.tagged) {
    const uint32_t tag = d.tag();
    unsigned spins = 0;
    while (true) {
      bool ok = true;
#pragma unroll
      for (int n = 0; n < kStagePieces; ++n) ok = ok && stage_piece_ready(S, n, tag);
      if (__all((int)ok) || give_up(d, spins)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int n = 0; n < kStagePieces; ++n)
        if (!stage_piece_ready(S, n, tag)) {
          S.a[n] = ld_co16(A.r, S.e[n] * 4u);
          S.b[n] = ld_co16(A.r, S.e[n] * 4u + 16u);
        }
    }
#pragma unroll
    for (int n = 0; n < kStagePieces; ++n) v[n] = u32x4_t{S.a[n][0], S.a[n][2], S.b[n][0], S.b[n][2]};
  } else {
#pragma unroll
    for (int n = 0; n < kStagePieces; ++n) v[n] = S.a[n];
  }
}

// Batch n0 of the staging into `stage` (rows of srow bytes): complete it,
// then write its pieces of the pass's pr rows.
__device__ __forceinline__ void stage_store(const Deps &d, const ActSrc &A, StageBatch &S, int pr, int ppr, int n0,
                                            int srow, unsigned char *stage) {
  u32x4_t v[kStagePieces];
  stage_complete(d, A, S, v);
#pragma unroll
  for (int n = 0; n < kStagePieces; ++n) {
    const int q = (int)tid() + kThreads * (n0 + n);
    const int m = q / ppr, pc = q % ppr;
    if (m < pr) *reinterpret_cast<u32x4_t *>(stage + m * srow + pc * 16) = v[n];
  }
}

// One wave: D0 = W0 B and D1 = W1 B for two 16-row MXFP4 weight tiles over
// nch 128-element chunks and a pass of pr activation rows (bf16).  The
// four waves of a workgroup call this together for units of the same expert
// (so with the same rows): the activations are staged once per workgroup.
//
// Weights: see MxTiles.  Lane l gets output rows 4*(l/16)..+3 of column
// l % 16; columns past the pass's rows are zero.  Per chunk a lane converts
// its MX block of each tile row to bf16 in registers for four 16x16x32
// MFMAs; kRing chunks are in flight.
//
// Activations (stage_issue / stage_complete): the rows' elements of up to
// kStageChunkRows / pr chunks at a time are loaded by the whole workgroup in
// 16-byte pieces into `stage` (row m at m * (its chunks * 256 + 16); chunks
// past nch as zeros; rows past the pass's vrows valid rows hold whatever the
// stage held -- their columns are never stored), then each wave reads its
// MFMA operand from there: lane l reads row l % 8 (pr 8) or l % 16 (of each
// 16-row block).  The first batch is requested before the weights when
// `early` (the activations are normally complete: the up units), else after
// them (the down units, whose activations are being written meanwhile).  The
// order matters because a wait for a load completes in request order: staging
// loads behind a wave's ring would be held up until the whole ring arrived.
//
// Chunks past nch have zero weights and zero activations and add nothing,
// so the loop has no branches on the data.  Each round of chunks runs at the
// issue priority of the workgroup's slot (set_slot_priority).  kLane: the
// scales in the streaming layout's per-lane words.
template <bool kLane> struct ScaleWord { using type = u32x4_t; };
template <> struct ScaleWord<true> { using type = uint32_t; };

template <int kRing, bool kLane, typename RowE>
__device__ __forceinline__ void mx_pair(const Deps &d, const MxTiles &T, int nch, int pr, int vrows, const ActSrc &A,
                                        RowE row_e, unsigned char *stage, f32x4_t (&d0)[2], f32x4_t (&d1)[2],
                                        int slot, bool early) {
  const int lane = tid() % MB_WAVE, g = lane >> 4;
  const rsrc_t rw = T.rw, rs = T.rs;
  const uint32_t o0 = T.o0, o1 = T.o1, so0 = T.so0, so1 = T.so1, ws = T.wstride, ss = T.sstride;
  const bool row16 = T.smode == kScalesRow16;
  u32x4_t W0[kRing], W1[kRing];
  using SW = typename ScaleWord<kLane>::type;
  auto scales = [&](uint32_t so, int c0) {
    if constexpr (kLane) {
      return ld_b32(rs, c0 < nch ? so + ss * c0 : kOob);
    } else {
      if (row16) return ld_b128(rs, c0 < nch ? so + ss * c0 : kOob);
      u32x4_t v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = ld_b32(rs, c0 + r < nch ? so + 4u * (c0 + r) : kOob);
      return v;
    }
  };
  // The lane's scale of chunk r of a group.
  auto scale_of = [&](const SW &v, int r) {
    if constexpr (kLane) return e8m0_to_f32((v >> (8 * r)) & 0xFFu);
    else return e8m0_to_f32((v[r] >> (8 * g)) & 0xFFu);
  };
  // pr rows (8, 16 or 32) in segments of seg chunks: pr * seg = 128.
  const int seg = kStageChunkRows / pr, srow = seg * 256 + 16;  // row stride in the stage
  const int nb = pr > 16 ? 2 : 1;                             // 16-row column blocks
  // The first two batches of the first segment: requested before the
  // weights when early, else right after them.
  const int segn_first = min(seg, nch), ppr_first = ((segn_first + kRing - 1) / kRing) * kRing * 16;
  const bool need1 = batch_needed(kStagePieces, ppr_first, vrows);
  StageBatch first[2];
  if (early) {
    stage_issue(A, row_e, pr, 0, segn_first, ppr_first, 0, first[0]);
    if (need1) stage_issue(A, row_e, pr, 0, segn_first, ppr_first, kStagePieces, first[1]);
  }
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    const bool ok = r < nch;
    W0[r] = ld_nt16(rw, ok ? o0 + ws * r : kOob);
    W1[r] = ld_nt16(rw, ok ? o1 + ws * r : kOob);
  }
  SW S0[kRing / 4], S1[kRing / 4];
#pragma unroll
  for (int q = 0; q < kRing / 4; ++q) {
    S0[q] = scales(so0, 4 * q);
    S1[q] = scales(so1, 4 * q);
  }
  if (!early) {
    if (A.ready) wait_ge(d, A.ready, A.target);
    stage_issue(A, row_e, pr, 0, segn_first, ppr_first, 0, first[0]);
    if (need1) stage_issue(A, row_e, pr, 0, segn_first, ppr_first, kStagePieces, first[1]);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    d0[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    d1[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t rd_off = (uint32_t)((lane & (pr == 8 ? 7 : 15)) * srow + 64 * g);
  for (int seg0 = 0; seg0 < nch; seg0 += seg) {
    // This segment's activations, chunks rounded up to whole rounds.
    const int segn = min(seg, nch - seg0);
    const int ppr = ((segn + kRing - 1) / kRing) * kRing * 16;  // 16-byte pieces per row
    // In batches of kStagePieces pieces per thread, each only if it holds
    // one of the pass's vrows rows (the batches in row order, so the needed
    // ones come first); batch k in buf[k % 2], requested one batch ahead of
    // its completion so that consecutive batches' requests overlap (the
    // first segment's first two were requested with the weights, into the
    // same two buffers).
    StageBatch (&buf)[2] = first;
    if (seg0 != 0) stage_issue(A, row_e, pr, seg0, segn, ppr, 0, buf[0]);
#pragma unroll
    for (int k = 0; k < kSegLoads / kStagePieces; ++k) {
      const int n0 = k * kStagePieces, n1 = n0 + kStagePieces;
      if (k > 0 && !batch_needed(n0, ppr, vrows)) break;
      if (n1 < kSegLoads && batch_needed(n1, ppr, vrows) && !(seg0 == 0 && k + 1 < 2))
        stage_issue(A, row_e, pr, seg0, segn, ppr, n1, buf[(k + 1) % 2]);
      stage_store(d, A, buf[k % 2], pr, ppr, n0, srow, stage);
    }
    __syncthreads();
    for (int c0 = seg0; c0 < seg0 + segn; c0 += kRing) {
      set_slot_priority(slot);
      SW N0[kRing / 4], N1[kRing / 4];
#pragma unroll
      for (int q = 0; q < kRing / 4; ++q) {
        N0[q] = scales(so0, c0 + kRing + 4 * q);
        N1[q] = scales(so1, c0 + kRing + 4 * q);
      }
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        const float s0 = scale_of(S0[r / 4], r % 4), s1 = scale_of(S1[r / 4], r % 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned char *bp = stage + rd_off + (c0 + r - seg0) * 256 + 16 * i;
          const bf16x8_t x0 = dequant_fp4x8(W0[r][i], s0), x1 = dequant_fp4x8(W1[r][i], s1);
          const u32x4_t B = *reinterpret_cast<const u32x4_t *>(bp);
          d0[0] = mfma_bf16(x0, as_bf16x8(B), d0[0]);
          d1[0] = mfma_bf16(x1, as_bf16x8(B), d1[0]);
          if (nb > 1) {
            const u32x4_t B1 = *reinterpret_cast<const u32x4_t *>(bp + 16 * srow);
            d0[1] = mfma_bf16(x0, as_bf16x8(B1), d0[1]);
            d1[1] = mfma_bf16(x1, as_bf16x8(B1), d1[1]);
          }
        }
        const int cn = c0 + kRing + r;
        const bool ok = cn < nch;
        W0[r] = ld_nt16(rw, ok ? o0 + ws * cn : kOob);
        W1[r] = ld_nt16(rw, ok ? o1 + ws * cn : kOob);
      }
#pragma unroll
      for (int q = 0; q < kRing / 4; ++q) {
        S0[q] = N0[q];
        S1[q] = N1[q];
      }
    }
    __syncthreads();
  }
}

// mx_pair for units of at most kAll chunks and passes of at most 16 rows, in
// the streaming layout: all of the unit's weights and scales are requested
// first (a down unit's activations are being written by its expert's up units
// meanwhile), then the activations are staged in one segment and every chunk
// is computed with no further weight requests.  Same operands, staging and
// results as mx_pair (block 0 of d0 / d1 only).
template <int kAll, typename RowE>
__device__ __forceinline__ void mx_pair_all(const Deps &d, const MxTiles &T, int nch, int pr, int vrows,
                                            const ActSrc &A, RowE row_e, unsigned char *stage, f32x4_t (&d0)[2],
                                            f32x4_t (&d1)[2]) {
  static_assert(kAll % 4 == 0 && 16 * kAll <= kStageChunkRows, "whole scale words; 16 rows x kAll chunks staged");
  const int lane = tid() % MB_WAVE, g = lane >> 4;
  const rsrc_t rw = T.rw, rs = T.rs;
  const uint32_t o0 = T.o0, o1 = T.o1, so0 = T.so0, so1 = T.so1, ws = T.wstride, ss = T.sstride;
  u32x4_t W0[kAll], W1[kAll];
  uint32_t S0[kAll / 4], S1[kAll / 4];
#pragma unroll
  for (int r = 0; r < kAll; ++r) {
    const bool ok = r < nch;
    W0[r] = ld_nt16(rw, ok ? o0 + ws * r : kOob);
    W1[r] = ld_nt16(rw, ok ? o1 + ws * r : kOob);
  }
#pragma unroll
  for (int q = 0; q < kAll / 4; ++q) {
    S0[q] = ld_b32(rs, 4 * q < nch ? so0 + ss * (4 * q) : kOob);
    S1[q] = ld_b32(rs, 4 * q < nch ? so1 + ss * (4 * q) : kOob);
  }
  const int srow = kAll * 256 + 16;  // row stride in the stage
  d0[0] = d1[0] = d0[1] = d1[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (A.ready) wait_ge(d, A.ready, A.target);
  // Chunks past nch are staged as zeros; a batch only if it holds one of the
  // pass's vrows rows.
  constexpr int ppr = kAll * 16;  // 16-byte pieces per row
#pragma unroll
  for (int n0 = 0; n0 < kSegLoads; n0 += kStagePieces) {
    if (n0 > 0 && !batch_needed(n0, ppr, vrows)) continue;
    StageBatch S;
    stage_issue(A, row_e, pr, 0, nch, ppr, n0, S);
    stage_store(d, A, S, pr, ppr, n0, srow, stage);
  }
  __syncthreads();
  const uint32_t rd_off = (uint32_t)((lane & (pr == 8 ? 7 : 15)) * srow + 64 * g);
#pragma unroll
  for (int r = 0; r < kAll; ++r) {
    const float s0 = e8m0_to_f32((S0[r / 4] >> (8 * (r % 4))) & 0xFFu);
    const float s1 = e8m0_to_f32((S1[r / 4] >> (8 * (r % 4))) & 0xFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t B = *reinterpret_cast<const u32x4_t *>(stage + rd_off + r * 256 + 16 * i);
      d0[0] = mfma_bf16(dequant_fp4x8(W0[r][i], s0), as_bf16x8(B), d0[0]);
      d1[0] = mfma_bf16(dequant_fp4x8(W1[r][i], s1), as_bf16x8(B), d1[0]);
    }
  }
  __syncthreads();
}

// ---- MXFP4 activations (the W4A4 variant), streaming layout only

// Quantized staging of one segment: pass rows 0 .. pr - 1 (row_e(m)), bf16
// elements of chunks seg0 .. seg0 + segn (segc >= segn chunks, a multiple of
// 4), fetched in 16-byte pieces of 8 elements as the bf16 staging does
// (stage_issue / stage_complete), quantized per 32-element block (four
// consecutive lanes hold a block: their amax by two butterfly steps; then the
// block's E8M0 byte by mx_scale_byte and the elements' E2M1 codes by the
// hardware's scaled conversion) and written to `stage` rows of srowq bytes:
// chunk c's block g's 16 code bytes at (4c + g) * 16, its scale byte at
// segc * 64 + g * segc + c (so a lane's scales of four chunks form one word).
// Rows past vrows are left as they are (their columns are not stored).
template <typename RowE>
__device__ __forceinline__ void mxq_stage(const Deps &d, const ActSrc &A, RowE row_e, int pr, int vrows, int seg0,
                                          int segn, int segc, int srowq, unsigned char *stage) {
  const int ppr = segc * 16;  // bf16 pieces (8 elements) per row
#pragma unroll
  for (int n0 = 0; n0 < kSegLoads; n0 += kStagePieces) {
    if (n0 > 0 && !batch_needed(n0, ppr, vrows)) continue;
    StageBatch S;
    u32x4_t v[kStagePieces];
    stage_issue(A, row_e, pr, seg0, segn, ppr, n0, S);
    stage_complete(d, A, S, v);
#pragma unroll
    for (int n = 0; n < kStagePieces; ++n) {
      const int q = (int)tid() + kThreads * (n0 + n);
      const int m = q / ppr, pc = q % ppr;
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_bits_to_f32(v[n][i] & 0xFFFFu);
        f[2 * i + 1] = bf16_bits_to_f32(v[n][i] >> 16);
      }
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(f[i]));
      am = fmaxf(am, __shfl_xor(am, 1, MB_WAVE));
      am = fmaxf(am, __shfl_xor(am, 2, MB_WAVE));
      const uint32_t sb = mx_scale_byte(am);
      uint32_t w = 0;
      if (sb == 0u && am > 0.f) {
        // Scale 2^-127 (a block below 2^-124): no normal fp32 divisor.
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= e2m1_code(ldexpf(f[i], 127)) << (4 * i);
      } else {
        // The hardware conversion divides by the scale and rounds to
        // nearest even, saturating at 6: the rule above, exactly.  (An
        // all-zero block converts to zeros with any scale.)  Each writes
        // two codes into byte i of w.  (The fp32-input form: the compiler
        // at hand merges the bf16-input form's four calls into one.)
        const float scl = __uint_as_float((sb > 0u ? sb : 1u) << 23);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], scl, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], scl, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], scl, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], scl, 3);
      }
      if (m < pr) {
        const int c = pc / 16, gq = (pc % 16) / 4, pw = pc % 4;
        *reinterpret_cast<uint32_t *>(stage + m * srowq + (4 * c + gq) * 16 + 4 * pw) = w;
        if (pw == 0) stage[m * srowq + segc * 64 + gq * segc + c] = (unsigned char)sb;
      }
    }
  }
}

// One scaled MFMA per 128-element chunk of each tile, the chunk's byte r of
// the lanes' scale words selecting its scales.
__device__ __forceinline__ f32x4_t mfma_fp4_r(int r, u32x4_t a, u32x4_t b, f32x4_t c, uint32_t sa, uint32_t sb) {
  switch (r & 3) {
    case 0: return mfma_fp4<0>(a, b, c, sa, sb);
    case 1: return mfma_fp4<1>(a, b, c, sa, sb);
    case 2: return mfma_fp4<2>(a, b, c, sa, sb);
    default: return mfma_fp4<3>(a, b, c, sa, sb);
  }
}

// mx_pair with MXFP4 activations: the same weight ring, scales, passes and
// results' layout, but the activations staged as MXFP4 (mxq_stage, after
// the weights are requested) and each chunk of a tile one scaled fp4 x fp4
// MFMA with the weights' codes as loaded (no conversion to bf16).
template <int kRing, typename RowE>
__device__ __forceinline__ void mxq_pair(const Deps &d, const MxTiles &T, int nch, int pr, int vrows,
                                         const ActSrc &A, RowE row_e, unsigned char *stage, f32x4_t (&d0)[2],
                                         f32x4_t (&d1)[2], int slot) {
  static_assert(kRing == 4, "one scale word covers the four chunks of a round");
  const int lane = tid() % MB_WAVE, g = lane >> 4;
  const rsrc_t rw = T.rw, rs = T.rs;
  const uint32_t o0 = T.o0, o1 = T.o1, so0 = T.so0, so1 = T.so1, ws = T.wstride, ss = T.sstride;
  u32x4_t W0[kRing], W1[kRing];
#pragma unroll
  for (int r = 0; r < kRing; ++r) {
    const bool ok = r < nch;
    W0[r] = ld_nt16(rw, ok ? o0 + ws * r : kOob);
    W1[r] = ld_nt16(rw, ok ? o1 + ws * r : kOob);
  }
  uint32_t S0 = ld_b32(rs, so0), S1 = ld_b32(rs, so1);
  const int seg = kStageChunkRows / pr, nb = pr > 16 ? 2 : 1;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    d0[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    d1[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int rrow = lane & (pr == 8 ? 7 : 15);
  for (int seg0 = 0; seg0 < nch; seg0 += seg) {
    const int segn = min(seg, nch - seg0), segc = ((segn + 3) / 4) * 4, srowq = segc * 68 + 16;
    mxq_stage(d, A, row_e, pr, vrows, seg0, segn, segc, srowq, stage);
    __syncthreads();
    for (int c0 = seg0; c0 < seg0 + segn; c0 += kRing) {
      set_slot_priority(slot);
      const uint32_t N0 = ld_b32(rs, c0 + kRing < nch ? so0 + ss * (c0 + kRing) : kOob);
      const uint32_t N1 = ld_b32(rs, c0 + kRing < nch ? so1 + ss * (c0 + kRing) : kOob);
      uint32_t sbw[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
        sbw[b] = b < nb ? *reinterpret_cast<const uint32_t *>(stage + (rrow + 16 * b) * srowq + segc * 64 +
                                                               g * segc + (c0 - seg0))
                        : 0u;
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        const int cr = c0 + r - seg0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (b >= nb) break;
          const u32x4_t B = *reinterpret_cast<const u32x4_t *>(stage + (rrow + 16 * b) * srowq + (4 * cr + g) * 16);
          d0[b] = mfma_fp4_r(r, W0[r], B, d0[b], S0, sbw[b]);
          d1[b] = mfma_fp4_r(r, W1[r], B, d1[b], S1, sbw[b]);
        }
        const int cn = c0 + kRing + r;
        const bool ok = cn < nch;
        W0[r] = ld_nt16(rw, ok ? o0 + ws * cn : kOob);
        W1[r] = ld_nt16(rw, ok ? o1 + ws * cn : kOob);
      }
      S0 = N0;
      S1 = N1;
    }
    __syncthreads();
  }
}

// mx_pair_all with MXFP4 activations (as mxq_pair is to mx_pair).
template <int kAll, typename RowE>
__device__ __forceinline__ void mxq_pair_all(const Deps &d, const MxTiles &T, int nch, int pr, int vrows,
                                             const ActSrc &A, RowE row_e, unsigned char *stage, f32x4_t (&d0)[2],
                                             f32x4_t (&d1)[2]) {
  static_assert(kAll % 4 == 0, "whole scale words");
  const int lane = tid() % MB_WAVE, g = lane >> 4;
  const rsrc_t rw = T.rw, rs = T.rs;
  const uint32_t o0 = T.o0, o1 = T.o1, so0 = T.so0, so1 = T.so1, ws = T.wstride, ss = T.sstride;
  u32x4_t W0[kAll], W1[kAll];
  uint32_t S0[kAll / 4], S1[kAll / 4];
#pragma unroll
  for (int r = 0; r < kAll; ++r) {
    const bool ok = r < nch;
    W0[r] = ld_nt16(rw, ok ? o0 + ws * r : kOob);
    W1[r] = ld_nt16(rw, ok ? o1 + ws * r : kOob);
  }
#pragma unroll
  for (int q = 0; q < kAll / 4; ++q) {
    S0[q] = ld_b32(rs, 4 * q < nch ? so0 + ss * (4 * q) : kOob);
    S1[q] = ld_b32(rs, 4 * q < nch ? so1 + ss * (4 * q) : kOob);
  }
  constexpr int segc = kAll, srowq = segc * 68 + 16;
  d0[0] = d1[0] = d0[1] = d1[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  mxq_stage(d, A, row_e, pr, vrows, 0, nch, segc, srowq, stage);
  __syncthreads();
  const int rrow = lane & (pr == 8 ? 7 : 15);
  uint32_t sbw[kAll / 4];
#pragma unroll
  for (int q = 0; q < kAll / 4; ++q)
    sbw[q] = *reinterpret_cast<const uint32_t *>(stage + rrow * srowq + segc * 64 + g * segc + 4 * q);
#pragma unroll
  for (int r = 0; r < kAll; ++r) {
    const u32x4_t B = *reinterpret_cast<const u32x4_t *>(stage + rrow * srowq + (4 * r + g) * 16);
    d0[0] = mfma_fp4_r(r, W0[r], B, d0[0], S0[r / 4], sbw[r / 4]);
    d1[0] = mfma_fp4_r(r, W1[r], B, d1[0], S1[r / 4], sbw[r / 4]);
  }
  __syncthreads();
}

// Up unit: w13 and the gated activation for (active expert, 16 act columns):
// gate rows i0..i0+15 and up rows I+i0..I+i0+15 of the expert, over P, for
// the expert's routes in passes of pass_rows.  h: the pooler's (or the
// pre-norm's) tagged words of this launch, or the caller's bf16 matrix.  act
// goes out as tagged words, and in bf16 to act_tap when asked for.  kPS with
// plain staging (the many-rows instance): h and act in bf16 (the units
// phase waited for h), each round of units signalled on the expert's up
// counter.
template <bool kPacked, bool kQ, bool kPS = false>
__device__ __forceinline__ void up_unit(const BlockParams &p, const Deps &d, const RouteLds &R, int unit,
                                        unsigned char *stage) {
  const int lane = tid() % MB_WAVE, g = lane >> 4, r16 = lane & 15;
  const int P = p.P, I = p.I;
  const int tiles = I / 16;
  const int a = unit / tiles, tile = unit % tiles;
  // Many rows: the unit covers one pass of its expert's rows (build_passes).
  const int ev = kPS ? uniform((int)R.vact[a]) : uniform(R.act[a]);
  const int e = kPS ? ev & 0xFF : ev, m_begin = kPS ? 32 * (ev >> 8) : 0;
  const int row0 = uniform(R.off[e]), rows_e = uniform(R.off[e + 1]) - row0;
  const int nrows = kPS ? min(rows_e, m_begin + 32) : rows_e;
  const int i0 = tile * 16;
  const MxTiles T =
      kPacked ? mx_packed(p.xp + (size_t)e * p.xp_stride, p.xp + (size_t)e * p.xp_stride + p.xp_up_s, tile, P, lane)
           : mx_plain(p.w13 + (size_t)e * 2 * I * (P / 2), p.w13s + (size_t)e * 2 * I * (P / 32), i0, I + i0, P,
                      lane);
  // (Plain staging: h is complete -- the units phase waited for it.)
  const bool plain = kPS && p.plain_stage;
  const ActSrc A{(p.h_tagged && !plain) ? make_rsrc(p.pre_norm_w ? p.hn_t : p.h_t) : make_rsrc(p.h),
                 p.h_tagged != 0 && !plain};
  const rsrc_t rat = make_rsrc(p.act_t), rap = make_rsrc(p.act_tap), rpl = make_rsrc(p.act);
  const uint32_t tag = d.tag();
  const int nch = P / 128;
  const int pr = pass_rows(nrows - m_begin);
  for (int m0 = m_begin; m0 < nrows; m0 += pr) {
    f32x4_t gs[2], us[2];
    auto row_e = [&](int m) { return m0 + m < nrows ? (uint32_t)((R.rl[row0 + m0 + m] / p.k) * P) : kOob; };
    if constexpr (kQ)
      mxq_pair<kRingUp>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, gs, us, (int)blockIdx.x / p.cus);
    else
      mx_pair<kRingUp, kPacked>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, gs, us,
                                (int)blockIdx.x / p.cus, true);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int m = m0 + 16 * b + r16;
      if ((b == 0 || pr > 16) && (pr > 8 || r16 < 8) && m < nrows) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = gs[b][i];
          o[i] = (z / (1.0f + expf(-z))) * us[b][i];
        }
        const uint32_t lo = pack_bf16x2(o[0], o[1]), hi = pack_bf16x2(o[2], o[3]);
        const size_t el = (size_t)(row0 + m) * I + i0 + 4 * g;
        if (plain) st_co8(rpl, (uint32_t)(el * 2), u32x2_t{lo, hi});
        else st_co16(rat, (uint32_t)(el * 4), u32x4_t{lo, tag, hi, tag});
        if (p.act_tap) st_co8(rap, (uint32_t)(el * 2), u32x2_t{lo, hi});
      }
    }
  }
  if (plain) signal_units(d.up(e));
}

// Down unit: w2 for (active expert, 32 output features): y in route order and
// the route's sum of squares over these 32 features, from the up units'
// tagged act (the staging polls it), or under plain staging from their bf16
// act once the expert's up counter is complete.
template <bool kPacked, bool kQ, bool kPS = false>
__device__ __forceinline__ void down_unit(const BlockParams &p, const Deps &d, const RouteLds &R, int unit,
                                          unsigned char *stage) {
  const int lane = tid() % MB_WAVE, g = lane >> 4, r16 = lane & 15;
  const int P = p.P, I = p.I;
  const int tiles = P / 32;
  const int a = unit / tiles, tile = unit % tiles;
  const int ev = kPS ? uniform((int)R.vact[a]) : uniform(R.act[a]);
  const int e = kPS ? ev & 0xFF : ev, m_begin = kPS ? 32 * (ev >> 8) : 0;
  const int row0 = uniform(R.off[e]), rows_e = uniform(R.off[e + 1]) - row0;
  const int nrows = kPS ? min(rows_e, m_begin + 32) : rows_e;
  const int p0 = tile * 32;
  const MxTiles T =
      kPacked ? mx_packed(p.xp + (size_t)e * p.xp_stride + p.xp_down, p.xp + (size_t)e * p.xp_stride + p.xp_down_s,
                       tile, I, lane)
           : mx_plain(p.w2 + (size_t)e * P * (I / 2), p.w2s + (size_t)e * P * (I / 32), p0, p0 + 16, I, lane);
  // Plain staging: act once the expert's up units (I / 16 per pass, four
  // per signal) signalled.
  const ActSrc A = (kPS && p.plain_stage)
                       ? ActSrc{make_rsrc(p.act), false, d.up(e), (unsigned)(I / 16 * ((rows_e + 31) / 32))}
                       : ActSrc{make_rsrc(p.act_t), true};
  const rsrc_t ry = make_rsrc(p.y), rss = make_rsrc(p.ssq);
  const int nch = I / 128;
  const int pr = pass_rows(nrows - m_begin);
  for (int m0 = m_begin; m0 < nrows; m0 += pr) {
    f32x4_t y0[2], y1[2];
    auto row_e = [&](int m) { return m0 + m < nrows ? (uint32_t)((row0 + m0 + m) * I) : kOob; };
    if constexpr (kQ) {
      if (nch <= kDownAll && pr <= 16)
        mxq_pair_all<kDownAll>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, y0, y1);
      else
        mxq_pair<kRingDown>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, y0, y1, (int)blockIdx.x / p.cus);
    } else if (kPacked && nch <= kDownAll && pr <= 16)
      mx_pair_all<kDownAll>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, y0, y1);
    else
      mx_pair<kRingDown, kPacked>(d, T, nch, pr, min(pr, nrows - m0), A, row_e, stage, y0, y1,
                                  (int)blockIdx.x / p.cus, false);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b == 1 && pr <= 16) break;
      const int m = m0 + 16 * b + r16;
      const bool valid = (pr > 8 || r16 < 8) && m < nrows;
      float ss = 0.f;
      if (valid) {
        ss = y0[b][0] * y0[b][0] + y0[b][1] * y0[b][1] + y0[b][2] * y0[b][2] + y0[b][3] * y0[b][3];
        ss += y1[b][0] * y1[b][0] + y1[b][1] * y1[b][1] + y1[b][2] * y1[b][2] + y1[b][3] * y1[b][3];
      }
      ss += __shfl_xor(ss, 16, MB_WAVE);
      ss += __shfl_xor(ss, 32, MB_WAVE);
      if (valid) {
        const int r = R.rl[row0 + m];
        st_co16(ry, (uint32_t)(((size_t)r * P + p0 + 4 * g) * 4), __builtin_bit_cast(u32x4_t, y0[b]));
        st_co16(ry, (uint32_t)(((size_t)r * P + p0 + 16 + 4 * g) * 4), __builtin_bit_cast(u32x4_t, y1[b]));
        if (g == 0) st_co4(rss, (uint32_t)(((size_t)r * tiles + tile) * 4), __float_as_uint(ss));
      }
    }
  }
  signal_units(d.down(e));
}

// ---------------------------------------------------------------- tail

// Byte offset of element p of row t in a copy of the MoE output [b][P] laid
// out chunk by chunk for the few-row unpooler: per 32-element chunk, the b
// rows' 64 bytes one after another, so that a chunk's wave load is b * 64
// contiguous bytes.
__device__ __forceinline__ uint32_t moe_rep_off(int t, int p, int b) {
  return (uint32_t)(((p / 32) * b + t) * 64 + (p % 32) * 2);
}

// moe_out[t, p] = bf16(sum_j (w_j / sqrt(ss_j / P + eps)) y_j[p] * w_post[p]),
// ss_j = the route's per-tile sums of squares added in tile order, for the
// task's features of row t (4 per thread); waits for the down units of the
// row's experts.  The post-norm weights are requested before the wait, the
// route rows of y and the sums of squares together after it.
template <bool kPasses>
__device__ __forceinline__ void fin_task(const BlockParams &p, const Deps &d, const RouteLds &R,
                                         int task, unsigned char *lds) {
  const int P = p.P, k = p.k;
  const int tiles = P / 32;
  const int chunks = (P + kFinChunk - 1) / kFinChunk;
  const int t = task / chunks, p_begin = (task % chunks) * kFinChunk;
  const int p_end = min(P, p_begin + kFinChunk);
  const int lane = tid() % MB_WAVE, wave = tid() / MB_WAVE;
  const int p4 = p_begin + tid() * 4;
  const bool mine = p4 < p_end;
  const u32x2_t pw = ld_b64(make_rsrc(p.post_norm_w), mine ? (uint32_t)p4 * 2 : kOob);
  if (tid() < MB_WAVE) {
    // (kPasses: the expert's down units come per pass of 32 rows.)
    const int e = R.ids[t * k + (lane < k ? lane : 0)];
    const unsigned passes = kPasses ? (unsigned)(R.off[e + 1] - R.off[e] + 31) / 32u : 1u;
    poll_ge(d, d.down(e), (unsigned)tiles * passes);
  }
  __syncthreads();
  stamp(p, 19);
  float *coef = reinterpret_cast<float *>(lds);  // [k]
  const rsrc_t rss = make_rsrc(p.ssq), ry = make_rsrc(p.y);
  f32x4_t yv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    yv[j] = __builtin_bit_cast(
        f32x4_t, ld_co16(ry, (mine && j < k) ? (uint32_t)(((size_t)(t * k + j) * P + p4) * 4) : kOob));
  for (int j = wave; j < k; j += kWaves) {
    const int r = t * k + j;
    float sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lane + MB_WAVE * q;
      sv[q] = __uint_as_float(ld_co4(rss, c < tiles ? (uint32_t)(((size_t)r * tiles + c) * 4) : kOob));
    }
    float s = sv[0] + sv[1] + sv[2] + sv[3];
    for (int c0 = MB_WAVE * 4; c0 < tiles; c0 += MB_WAVE)
      s += __uint_as_float(ld_co4(rss, lane + c0 < tiles ? (uint32_t)(((size_t)r * tiles + lane + c0) * 4) : kOob));
    s = wave_sum(s);
    if (lane == 0) coef[j] = R.w[r] * (1.0f / sqrtf(s / (float)P + p.norm_eps));
  }
  __syncthreads();
  if (mine) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) acc += coef[j] * yv[j];
    const float o0 = acc[0] * bf16_bits_to_f32(pw[0] & 0xFFFFu);
    const float o1 = acc[1] * bf16_bits_to_f32(pw[0] >> 16);
    const float o2 = acc[2] * bf16_bits_to_f32(pw[1] & 0xFFFFu);
    const float o3 = acc[3] * bf16_bits_to_f32(pw[1] >> 16);
    const u32x2_t v = u32x2_t{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
    const uint32_t off = (uint32_t)(((size_t)t * P + p4) * 2);
    if (p.unpool_wide) {
      // The wide unpooler's tasks read moe_out itself (each 64-row block
      // task a slice of it): kMoeReplicas copies of b x P cost the finalize
      // more stores than they save the readers beyond 16 rows (c3 b = 256
      // 322.9 -> 318.1 us, b = 128 244.2 -> 241.8, c2 201.1 -> 200.1).
      st_co8(make_rsrc(p.moe_out), off, v);
    } else {
      *reinterpret_cast<u32x2_t *>(reinterpret_cast<unsigned char *>(p.moe_out) + off) = v;
      // Copies for the few-row unpooler's tasks, each reading the one its
      // workgroup index selects (hundreds of workgroups reading one copy
      // queue on it), chunk by chunk (moe_rep_off).
      const rsrc_t rr = make_rsrc(p.moe_rep);
      const uint32_t rep_bytes = (uint32_t)(p.b * P * 2);
      const uint32_t roff = moe_rep_off(t, p4, p.b);
#pragma unroll
      for (int c = 0; c < kMoeReplicas; ++c) st_co8(rr, roff + rep_bytes * c, v);
    }
  }
  signal_step(d, kCtrFin);
  stamp(p, 21);
}

// ---------------------------------------------------------------- boundary

__device__ __forceinline__ void unpack4(u32x2_t v, float o[4]) {
  o[0] = bf16_bits_to_f32(v[0] & 0xFFFFu);
  o[1] = bf16_bits_to_f32(v[0] >> 16);
  o[2] = bf16_bits_to_f32(v[1] & 0xFFFFu);
  o[3] = bf16_bits_to_f32(v[1] >> 16);
}

// v = RMSNorm_H(u) * w_pff; stream = fp32(stream + g * v) (one fma);
// x_next = bf16(RMSNorm_H(stream) * w_in), for row t.  Thread i holds
// elements 4i + 1024 m .. +3 (m < NG, so H <= 1024 NG)
// in registers across the passes; the gate and the stream are requested
// before the wait.  With a split unpooler, u = bf16 of its fp32 partials added here in
// split order (and written out).
//
// kSignal (the next-QKV projection follows in the launch): x_next is written
// coherently and the row signals kCtrBound.
template <int NG, bool kSignal = false>
__device__ __forceinline__ void boundary_task(const BlockParams &p, const Deps &d, int t,
                                              unsigned char *lds) {
  float *red = reinterpret_cast<float *>(lds);
  const int H = p.H;
  const uint32_t H2 = (uint32_t)H * 2;
  const rsrc_t rg = make_rsrc(p.gate), rs = make_rsrc(p.stream + (size_t)t * H);
  u32x2_t gv[NG], fv[NG], wv[NG];
  f32x4_t sv[NG];
  // Everything but the unpooler's output is requested before the wait (the
  // next norm's weights later for wide rows: registers).
  constexpr bool kEarlyNext = NG <= 4;
  auto next_norm = [&](bool in, uint32_t h) {
    return p.next_norm_w ? ld_b64(make_rsrc(p.next_norm_w), in ? h * 2 : kOob) : u32x2_t{0x3F803F80u, 0x3F803F80u};
  };
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    const uint32_t h = (uint32_t)(4 * tid() + 1024 * m);
    const bool in = h * 2 < H2;
    gv[m] = ld_b64(rg, in ? h * 2 : kOob);
    sv[m] = __builtin_bit_cast(f32x4_t, ld_b128(rs, in ? h * 4 : kOob));
    fv[m] = p.ffn_norm_w ? ld_b64(make_rsrc(p.ffn_norm_w), in ? h * 2 : kOob) : u32x2_t{0x3F803F80u, 0x3F803F80u};
    if (kEarlyNext) wv[m] = next_norm(in, h);
  }
  wait_step(d, kCtrUnpool, p.n_unpool);
  stamp(p, 17);
  u32x2_t uv[NG];
  if (p.unpool_ks > 1) {
    // u = bf16(sum of the split partials in split order).
    const rsrc_t rp = make_rsrc(p.unpool_part), ru = make_rsrc(p.u + (size_t)t * H);
    // Partials requested QB splits at a time (fewer when the row is wide).
    constexpr int QB = NG <= 4 ? 2 : 1;
    f32x4_t av[NG];
    for (int q0 = 0; q0 < p.unpool_ks; q0 += QB) {
      f32x4_t pv[QB][NG];
#pragma unroll
      for (int q = 0; q < QB; ++q)
#pragma unroll
        for (int m = 0; m < NG; ++m) {
          const uint32_t h = (uint32_t)(4 * tid() + 1024 * m);
          const bool in = h * 2 < H2 && q0 + q < p.unpool_ks;
          pv[q][m] = __builtin_bit_cast(
              f32x4_t, ld_co16(rp, in ? (uint32_t)((((size_t)(q0 + q) * p.b + t) * H + h) * 4) : kOob));
        }
#pragma unroll
      for (int m = 0; m < NG; ++m) {
        av[m] = q0 == 0 ? pv[0][m] : av[m] + pv[0][m];
#pragma unroll
        for (int q = 1; q < QB; ++q)
          if (q0 + q < p.unpool_ks) av[m] += pv[q][m];
      }
    }
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const uint32_t h = (uint32_t)(4 * tid() + 1024 * m);
      uv[m] = u32x2_t{pack_bf16x2(av[m][0], av[m][1]), pack_bf16x2(av[m][2], av[m][3])};
      if (h * 2 < H2) st_co8(ru, h * 2, uv[m]);
    }
  } else {
    const rsrc_t ru = make_rsrc(p.u + (size_t)t * H);
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const uint32_t h = (uint32_t)(4 * tid() + 1024 * m);
      uv[m] = ld_co8(ru, h * 2 < H2 ? h * 2 : kOob);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    float v[4];
    unpack4(uv[m], v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  if (!kEarlyNext) {
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const uint32_t h = (uint32_t)(4 * tid() + 1024 * m);
      wv[m] = next_norm(h * 2 < H2, h);
    }
  }
  ss = wg_sum(ss, red, 0);
  const float rsu = 1.0f / sqrtf(ss / (float)H + p.norm_eps);
  float s2 = 0.f;
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    float v[4], gg[4], wf[4];
    unpack4(uv[m], v);
    unpack4(gv[m], gg);
    unpack4(fv[m], wf);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float vn = v[i] * rsu * wf[i];
      sv[m][i] = fmaf(gg[i], vn, sv[m][i]);
      s2 += sv[m][i] * sv[m][i];
    }
  }
  s2 = wg_sum(s2, red, 1);
  const float rss = 1.0f / sqrtf(s2 / (float)H + p.norm_eps);
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    const int h = 4 * tid() + 1024 * m;
    if (h >= H) break;
    float wi[4];
    unpack4(wv[m], wi);
    const f32x4_t sn = sv[m];
    *reinterpret_cast<f32x4_t *>(p.stream + (size_t)t * H + h) = sn;
    const u32x2_t xv = u32x2_t{pack_bf16x2(sn[0] * rss * wi[0], sn[1] * rss * wi[1]),
                               pack_bf16x2(sn[2] * rss * wi[2], sn[3] * rss * wi[3])};
    if constexpr (kSignal)
      st_co8(make_rsrc(p.x_next), (uint32_t)(((size_t)t * H + h) * 2), xv);
    else
      *reinterpret_cast<u32x2_t *>(p.x_next + (size_t)t * H + h) = xv;
  }
  if constexpr (kSignal) signal_step(d, kCtrBound);
  __syncthreads();
}

// ---------------------------------------------------------------- the kernel

// The parameters, read through a pointer to the kernel-argument segment that
// each phase (and each task of a loop) obtains afresh: the compiler cannot
// merge the loads of a field across phases, so no field stays live in a
// register from the first phase to the last.  (Kept live, the fields overflow
// the scalar registers into vector registers and scratch memory, and the
// scratch lines are written back to HBM at the end of every launch.)
__device__ __forceinline__ const BlockParams &kparams() {
  const __attribute__((address_space(4))) BlockParams *pp =
      (const __attribute__((address_space(4))) BlockParams *)(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(pp));
  return *(const BlockParams *)pp;
}

// kQ: the W4A4 variant (MXFP4 activations into the experts), a kernel of its
// own so that each keeps its own code layout and registers.
// kQKV: the next layer's QKV projection follows the boundary in the launch.
// kMR: the many-rows paths (the fp64-MFMA router tiles, the wide
// projections' 64-row block tasks) are compiled in; the plain kernel has a
// many-rows instance of its own for them, the others take both.
template <bool kQ, bool kQKV = false, bool kMR = kQ || kQKV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void block_kernel(BlockParams p_arg) {
  // Plain staging of the expert units' activations: the many-rows instance.
  constexpr bool kPS = kMR && !kQ && !kQKV;
  extern __shared__ __align__(16) unsigned char lds[];
  (void)p_arg;  // read through kparams()
  stamps_begin(kparams());
  stamp(kparams(), 0);
  // Requested now, first needed at a counter.
  // (A workgroup that starts with a router task requests it there.)
  unsigned gen = blockIdx.x < (unsigned)kparams().n_router ? kGenPending : load_generation(kparams().sync);
  const int G = gridDim.x;
  {
    // The grouping's per-expert row bitmaps start empty.
    const BlockParams &p = kparams();
    if (p.needs_routing && !p.route_given) {
      const RouteLds R = route_lds(p, lds);
      for (int i = tid(); i < p.E * ((p.b + 63) / 64); i += kThreads) R.bits[i] = 0ull;
    }
    __syncthreads();
  }

  // 1. Workgroup tasks before routing: router tasks 0 .. nR - 1, then route,
  // pool and pre-norm tasks, numbered on; the workgroup takes tasks
  // blockIdx, blockIdx + G, ..  Each kind has a loop of its own, so that no
  // kind's hoisted constants (the routing's fp64 exp) stay live through
  // another's.
  {
    // The first of this workgroup's task numbers at or after lo.
    auto first_from = [&](int lo) {
      const int b = (int)blockIdx.x;
      return lo <= b ? b : b + G * ((lo - b + G - 1) / G);
    };
    {
      bool first = true;
      for (int j = blockIdx.x; j < kparams().n_router; j += G) {
        const BlockParams &p = kparams();
        if (first) stamp(p, 1);
        first = false;
        if (kMR && p.router_mma) router_mma_task(p, gen, j, lds + p.lds_route_bytes);
        else if (p.router_multi) router_task_multi(p, gen, j, lds + p.lds_route_bytes);
        else router_task(p, gen, j, lds + p.lds_route_bytes);
      }
    }
    {
      bool first = true;
      const int lo = kparams().n_router;
      for (int j = first_from(lo); j < lo + kparams().n_route; j += G) {
        const BlockParams &p = kparams();
        if (first) stamp(p, 2);
        first = false;
        route_task(p, Deps{p.sync, gen}, j - lo);
      }
    }
    {
      bool first = true;
      const int lo = kparams().n_router + kparams().n_route;
      for (int j = first_from(lo); j < lo + kparams().n_pool; j += G) {
        const BlockParams &p = kparams();
        const Deps d{p.sync, gen};
        unsigned char *scratch = lds + p.lds_route_bytes;
        if (first) stamp(p, 3);
        first = false;
        // Pooler: wide tiles, the splits added by the last to finish.  h
        // goes out as tagged words (the up units and the pre-norm poll them),
        // and in bf16 when asked for (the pre-norm writes that then).
        uint16_t *hp = (p.h_plain && !p.pre_norm_w) ? p.h : nullptr;
        uint32_t *ht = p.h_t;
        // Plain staging without a pre-norm: h only in bf16, each finished
        // tile (64-row block) signalled.
        const bool h_signal = kPS && p.plain_stage && !p.pre_norm_w;
        const uint16_t *pw = p.pool_wp ? p.pool_wp : p.pool_w;
        const bool pwk = p.pool_wp != nullptr;
        if (h_signal) {
          hp = p.h;
          ht = nullptr;
        }
        if (kMR && p.row_blocks > 1) {
          // Many rows: one 64-row block per task.
          int gq, rb;
          row_block_task(j - lo, p.row_blocks, gq, rb);
          if (gq < p.n_pool_tiles * p.pool_ks) {
            const int gi = gq / p.pool_ks, q = gq % p.pool_ks, t0 = rb * 64, t1 = t0 + 64;
            proj_wide<false, true>(make_rsrc(p.x), pw, pwk, p.b, p.P, p.H, gi, q, p.pool_ks, p.pool_part, hp, ht,
                                   d.tag(), scratch, []() {}, t0, t1, true);
            unsigned *cnt = &p.pool_cnt[gi * kMaxRowBlocks + rb];
            if (p.pool_ks == 1) {
              if (h_signal) signal_step(d, kCtrPool);
            } else if (last_arrival(cnt, (unsigned)p.pool_ks, proj_flag(scratch))) {
              proj_wide_sum(p.pool_part, hp, ht, d.tag(), p.b, p.P, gi, p.pool_ks, t0, t1);
              if (tid() == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if (h_signal) signal_step(d, kCtrPool);
            }
          }
        } else {
          const int i = j - lo, gi = i / p.pool_ks, q = i % p.pool_ks;
          proj_wide<false>(make_rsrc(p.x), pw, pwk, p.b, p.P, p.H, gi, q, p.pool_ks, p.pool_part, hp, ht, d.tag(),
                           scratch, []() {});
          unsigned *cnt = &p.pool_cnt[gi * kMaxRowBlocks];
          if (p.pool_ks == 1) {
            if (h_signal) signal_step(d, kCtrPool);
          } else if (last_arrival(cnt, (unsigned)p.pool_ks, proj_flag(scratch))) {
            proj_wide_sum(p.pool_part, hp, ht, d.tag(), p.b, p.P, gi, p.pool_ks);
            if (tid() == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (h_signal) signal_step(d, kCtrPool);
          }
        }
        __syncthreads();  // (the workgroup's next task reuses the LDS)
        stamp(p, 7);
      }
    }
    {
      bool first = true;
      const int lo = kparams().n_router + kparams().n_route + kparams().n_pool;
      for (int j = first_from(lo); j < lo + kparams().n_prenorm; j += G) {
        const BlockParams &p = kparams();
        if (first) stamp(p, 4);
        first = false;
        prenorm_task(p, Deps{p.sync, gen}, j - lo, lds + p.lds_route_bytes);
        if (kPS && p.plain_stage) signal_step(Deps{p.sync, gen}, kCtrPrenorm);  // (its h row in bf16)
      }
    }
  }

  // The launch's generation, kept in LDS from here on: a register holding it
  // through the later phases would be spilled, and a reload from scratch
  // memory waits behind every load the wave has in flight.
  unsigned *const gen_slot = reinterpret_cast<unsigned *>(route_lds(kparams(), lds).nact + 1);
  if (tid() == 0) *gen_slot = gen;
  __syncthreads();
  auto launch_gen = [&]() { return (unsigned)uniform((int)*gen_slot); };

  // 2. Routing state (workgroup 0 also writes the routing outputs).
  {
  const BlockParams &p = kparams();
  const Deps d{p.sync, launch_gen()};
  const RouteLds R = route_lds(p, lds);
  if (p.needs_routing && (p.has_up || (p.routing_out && blockIdx.x == 0))) {
    prepare_routing(p, d, R, kPS);
    stamp(p, 5);
  }
  }

  // 3. Expert units, one wave each.
  if (kparams().has_up) {
    const BlockParams &p = kparams();
    const Deps d{p.sync, launch_gen()};
    const RouteLds R = route_lds(p, lds);
    unsigned char *scratch = lds + p.lds_route_bytes;
    stamp(p, 6);
    const int GW = G * kWaves;
    unsigned char *stage = scratch;
    // (Many rows: units per pass of an expert's rows, build_passes.)
    const int nact = kPS ? uniform(R.nact[2]) : uniform(*R.nact);
    const int nU = nact * (p.I / 16), nD = nact * (p.P / 32);
    // Up units and down units are dealt separately, so a wave's down units
    // belong to the experts of its own up units (with as many tiles per
    // expert): they wait on waves that started with them.  (Waves that
    // reach the memory system later -- the later workgroups on a CU -- finish
    // their up units later.)  Unit counts are multiples of four (I / 16 and
    // P / 32 tiles per expert) and so is the wave count, so the four waves of
    // a workgroup always have units, of one expert, in the same rounds: the
    // units' workgroup barriers and signals rely on it.
    //
    // The last resident slot's workgroups on the first quarter of the CUs
    // take the last unit slots (the rest of that slot moving up): when the
    // units leave workgroups idle (704 of 768 busy at the decode step), the
    // idle ones sit on those CUs, whose workgroups measured the slowest to
    // stream their units -- with the experts dealt in either order, so it is
    // the CUs, not the data (c1 49.3 -> 48.7 us; reversing the whole last
    // slot instead gained 0.1 us).
    const int bx = (int)blockIdx.x, last = (G / p.cus - 1) * p.cus, quarter = p.cus / 4;
    const int wslot = bx >= last ? last + (bx - last + p.cus - quarter) % p.cus : bx;
    const int gw = wslot * kWaves + uniform(tid() / MB_WAVE);
    // (The expert layout and the activation format are template arguments:
    // each has its own registers.)
    // Plain staging: h complete before the workgroup's first up unit.
    if (kPS && p.plain_stage && (int)blockIdx.x * kWaves < nU)
      wait_step(d, p.pre_norm_w ? kCtrPrenorm : kCtrPool, p.n_h_ready);
    if constexpr (kPS) {
      // Many rows: units cost more or less with their expert's rows, so
      // after a first round dealt by workgroup index each workgroup claims
      // its next round of four units (one expert's) from a counter -- every
      // up round before any down round, so a down unit only ever waits for
      // up units that running workgroups hold.
      int *slot = R.red;
      auto next = [&](int ctr) {
        if (tid() == 0) *slot = (int)atomic_inc(d.ctr(ctr));
        __syncthreads();
        const int q = G + uniform(*slot);
        __syncthreads();
        return q;
      };
      const int w = uniform(tid() / MB_WAVE);
      if (p.xp) {
        for (int q = blockIdx.x; kWaves * q < nU; q = next(kCtrUpQueue))
          up_unit<true, false, kPS>(p, d, R, kWaves * q + w, stage);
        stamp(p, 20);
        for (int q = blockIdx.x; kWaves * q < nD; q = next(kCtrDownQueue))
          down_unit<true, false, kPS>(p, d, R, kWaves * q + w, stage);
      } else {
        for (int q = blockIdx.x; kWaves * q < nU; q = next(kCtrUpQueue))
          up_unit<false, false, kPS>(p, d, R, kWaves * q + w, stage);
        stamp(p, 20);
        for (int q = blockIdx.x; kWaves * q < nD; q = next(kCtrDownQueue))
          down_unit<false, false, kPS>(p, d, R, kWaves * q + w, stage);
      }
    } else if constexpr (kQ) {
      for (int u = gw; u < nU; u += GW) up_unit<true, true>(p, d, R, u, stage);
      stamp(p, 20);
      for (int u = gw; u < nD; u += GW) down_unit<true, true>(p, d, R, u, stage);
    } else if (p.xp) {
      for (int u = gw; u < nU; u += GW) up_unit<true, false>(p, d, R, u, stage);
      stamp(p, 20);
      for (int u = gw; u < nD; u += GW) down_unit<true, false>(p, d, R, u, stage);
    } else {
      for (int u = gw; u < nU; u += GW) up_unit<false, false>(p, d, R, u, stage);
      stamp(p, 20);
      for (int u = gw; u < nD; u += GW) down_unit<false, false>(p, d, R, u, stage);
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    stamp(p, 11);
  }

  // 4. Workgroup tasks after the experts.
  {
    int last = -1;
    for (int j = blockIdx.x;; j += G) {
      const BlockParams &p = kparams();
      const Deps d{p.sync, launch_gen()};
      const RouteLds R = route_lds(p, lds);
      unsigned char *scratch = lds + p.lds_route_bytes;
      const int nF = p.n_fin, nN = p.n_unpool, nB = p.n_boundary, nQ = kQKV ? p.n_qkv : 0;
      if (j >= nF + nN + nB + nQ) break;
      int step, i = j;
      if (i < nF) {
        step = 8;
      } else if ((i -= nF) < nN) {
        step = 9;
      } else if ((i -= nN) < nB) {
        step = 10;
      } else {
        i -= nB;
        step = 24;
      }
      if (step != last) {
        stamp(p, step);
        last = step;
      }
      if (step == 8) {
        fin_task<kPS>(p, d, R, i, scratch);
      } else if (step == 9) {
        const uint16_t *mo =
            (p.n_fin > 0 && !p.unpool_wide) ? p.moe_rep + (size_t)(blockIdx.x % kMoeReplicas) * p.b * p.P : p.moe_out;
        if (p.unpool_wide) {
          // Many rows: wide tiles, so each workgroup reads the MoE output once
          // per 64 features (one 64-row block of it beyond 64 rows).
          const uint16_t *uw = p.unpool_wp ? p.unpool_wp : p.unpool_w;
          const bool uwk = p.unpool_wp != nullptr;
          if (kMR && p.row_blocks > 1) {
            int gq, rb;
            row_block_task(i, p.row_blocks, gq, rb);
            if (gq < ((p.H + 63) / 64) * p.unpool_ks)
              proj_wide<true, true>(make_rsrc(mo), uw, uwk, p.b, p.H, p.P, gq / p.unpool_ks, gq % p.unpool_ks,
                                    p.unpool_ks, p.unpool_part, p.u, nullptr, 0u, scratch,
                                    [&]() { wait_step(d, kCtrFin, p.n_fin); }, rb * 64, rb * 64 + 64, true);
          } else {
            proj_wide<true>(make_rsrc(mo), uw, uwk, p.b, p.H, p.P, i / p.unpool_ks, i % p.unpool_ks, p.unpool_ks,
                            p.unpool_part, p.u, nullptr, 0u, scratch, [&]() { wait_step(d, kCtrFin, p.n_fin); });
          }
        } else {
          unpool_task(p, d, mo, i, scratch);
        }
        signal_step(d, kCtrUnpool);
        stamp(p, 16);
      } else if (step == 10) {
        if (p.H <= 4096) boundary_task<4, kQKV>(p, d, i, scratch);
        else boundary_task<kBoundGroups, kQKV>(p, d, i, scratch);
        stamp(p, 18);
      } else if constexpr (kQKV) {
        // The next layer's QKV projection of x_next: wide tiles, the splits
        // added by the last to finish.
        const int gi = i / p.qkv_ks, q = i % p.qkv_ks;
        proj_wide<true>(make_rsrc(p.x_next), p.qkv_w, false, p.b, p.qkv_rows, p.H, gi, q, p.qkv_ks, p.qkv_part,
                        p.qkvg, nullptr, 0u, scratch, [&]() { wait_step(d, kCtrBound, p.n_boundary); });
        if (p.qkv_ks > 1 && last_arrival(&p.qkv_cnt[gi], (unsigned)p.qkv_ks, proj_flag(scratch))) {
          proj_wide_sum(p.qkv_part, p.qkvg, nullptr, 0u, p.b, p.qkv_rows, gi, p.qkv_ks);
          if (tid() == 0) __hip_atomic_store(&p.qkv_cnt[gi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        stamp(p, 25);
      }
    }
  }
  prepare_next_launch(kparams().sync, launch_gen());
  stamp(kparams(), 15);
  stamps_end(kparams());
}

}  // namespace

// Workgroups of kernel f, with lds bytes of dynamic LDS, that a CU holds at
// once.  The occupancy query counts LDS in finer steps than gfx950 allocates
// it: measured with workgroups that only stamp their start and spin, a CU
// holds 5 of 32000 bytes (dynamic and static) but 4 of 32001, and 3 of 53760
// but 2 of 53761, where the query answers 5 and 3 -- allocation in 1280-byte
// steps of the CU's 160 KB.  The persistent kernel needs its whole grid
// resident at once, so the query's answer is capped by that allocation.
static int resident_groups(const void *f, size_t lds) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kThreads, lds) != hipSuccess) return 0;
  hipFuncAttributes a{};
  if (hipFuncGetAttributes(&a, f) != hipSuccess) return 0;
  constexpr size_t kLdsPerCu = 160 * 1024, kLdsStep = 1280;
  const size_t step = (lds + a.sharedSizeBytes + kLdsStep - 1) / kLdsStep * kLdsStep;
  const int by_lds = (int)(kLdsPerCu / step);
  return n < by_lds ? n : by_lds;
}

// An ordinary launch: the host sizes the grid to what the device holds at
// once.  Should some workgroups not be resident together with the others
// (another kernel holding compute units), the resident ones may wait on them
// until a wait runs out of polls: the launch then drains with its results
// not to be trusted, and the workspace reports it (mb_workspace_status).
// The W4A4 kernel, the kernel with the fused next-QKV projection and the
// kernel with both are built from this file in translation units of their own
// (block_w4a4.hip, block_qkv.hip, block_w4a4_qkv.hip), and so is the plain
// kernel's many-rows instance (block_many.hip): sharing one code object moved
// the bf16 kernel's code and cost it ~0.6 us per launch.
#if defined(MB_BLOCK_MANY)
hipError_t launch_block_many(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((block_kernel<false, false, true>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

int block_max_groups_per_cu_many(size_t lds) {
  return resident_groups(reinterpret_cast<const void *>(block_kernel<false, false, true>), lds);
}
#elif !defined(MB_BLOCK_W4A4) && !defined(MB_BLOCK_QKV)
hipError_t launch_block(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  if (p.w4a4) return launch_block_w4a4(p, grid, lds, s);
  if (p.n_qkv > 0) return launch_block_qkv(p, grid, lds, s);
  if (p.router_mma || p.row_blocks > 1) return launch_block_many(p, grid, lds, s);
  hipLaunchKernelGGL(block_kernel<false>, dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

int block_max_groups_per_cu(size_t lds, bool w4a4, bool qkv, bool many) {
  if (w4a4) return block_max_groups_per_cu_w4a4(lds, qkv);
  if (qkv) return block_max_groups_per_cu_qkv(lds);
  if (many) return block_max_groups_per_cu_many(lds);
  return resident_groups(reinterpret_cast<const void *>(block_kernel<false>), lds);
}
#elif defined(MB_BLOCK_W4A4) && !defined(MB_BLOCK_QKV)
hipError_t launch_block_w4a4(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  if (p.n_qkv > 0) return launch_block_w4a4_qkv(p, grid, lds, s);
  hipLaunchKernelGGL(block_kernel<true>, dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

int block_max_groups_per_cu_w4a4(size_t lds, bool qkv) {
  if (qkv) return block_max_groups_per_cu_w4a4_qkv(lds);
  return resident_groups(reinterpret_cast<const void *>(block_kernel<true>), lds);
}
#elif defined(MB_BLOCK_QKV) && !defined(MB_BLOCK_W4A4)
hipError_t launch_block_qkv(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((block_kernel<false, true>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

int block_max_groups_per_cu_qkv(size_t lds) {
  return resident_groups(reinterpret_cast<const void *>(block_kernel<false, true>), lds);
}
#else
hipError_t launch_block_w4a4_qkv(const BlockParams &p, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((block_kernel<true, true>), dim3(grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

int block_max_groups_per_cu_w4a4_qkv(size_t lds) {
  return resident_groups(reinterpret_cast<const void *>(block_kernel<true, true>), lds);
}
#endif

}  // namespace mb
