// Parameters and LDS layout of the persistent block kernel (block.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mb_internal.h"

namespace mb {

constexpr int kBlockWaves = 4;      // waves per workgroup
constexpr int kRouterRowBlock = 4;   // rows per router task
constexpr int kRouterExperts = 4;    // experts per router task when there are many rows

// Cross-workgroup state, at the workspace start, in 128-byte lines of kLine
// words so that no two counters share a line:
//   line 0      word 1: the abort record (the tag of the last launch a wait
//               of which ran out of polls; 0 after a zero-fill or reset)
//   kGenLines lines   the generation words, one per workgroup index
//   two counter sets of kSetLines lines each, a set being
//     kNumCtr x kReplicas lines   step counters (kCtr*), each spread over
//                 stripes(i) x replicas(i) lines
//     2 kBlockMaxExperts lines   up units done per expert, then down units
//     kSyncMaxRows / 4 lines     router tasks done per block of 4 rows
// Between launches every generation word holds the same value g (0 in a
// zero-filled workspace).  A launch uses counter set g % 2, which is zero
// when it starts; its workgroups clear set (g + 1) % 2, which the previous
// launch used, and each workgroup b writes g + 1 into the generation words
// b, b + G, b + 2G, .. (G = the grid), so that every word advances by one
// whatever the grid.  No workgroup has to find out that it is the last.
// Increments of one address are serialized, and polls of an address delay
// the increments to it.  So a step counter is held in replicas(i) copies,
// each split into stripes(i) lines: a producer adds one to its stripe (chosen
// by its workgroup index) of every copy, after its coherent stores completed
// (one atomic per lane of one instruction); a consumer sums the stripes of
// the copy its workgroup or wave index selects.  Many consumers call for
// copies, many producers for stripes.
constexpr int kLine = 32;
constexpr int kReplicas = 16;
constexpr int kMaxGrid = 1024;  // workgroups of the persistent launch, at most
constexpr int kBlockMaxExperts = 256;  // larger expert counts use the per-step kernels
constexpr int kSyncMaxRows = 1024;     // rows the counter sets provide for
enum : int {
  kCtrRoute = 0,     // route tasks done
  kCtrPool = 1,      // pooler tiles complete
  kCtrPrenorm = 2,   // pre-norm rows done
  kCtrFin = 3,       // finalize tasks done
  kCtrUnpool = 4,    // unpooler tasks done
  kCtrBound = 5,     // boundary rows done (awaited by the fused next-QKV tiles)
  kCtrUpQueue = 6,   // up-unit rounds claimed past the first (many-rows instance)
  kCtrDownQueue = 7, // down-unit rounds claimed past the first (many-rows instance)
  kNumCtr = 8,
};
// Copies and stripes of step counter i (replicas x stripes <= kReplicas).
// The route and pre-norm counters have few producers and are awaited by
// every workgroup or wave; the pooler's has 128 producers (H / 16 tiles) and
// every wave as consumer; the finalize counter has b * P / 512 producers and
// the unpooler tasks as consumers; the unpooler's has H / 16 (times its
// split) producers and only the b boundary tasks as consumers.
__host__ __device__ constexpr int replicas(int i) {
  return (i == kCtrRoute || i == kCtrPrenorm || i == kCtrBound) ? kReplicas : (i == kCtrPool || i == kCtrFin) ? 4 : 1;
}
__host__ __device__ constexpr int stripes(int i) {
  return (i == kCtrPool || i == kCtrFin) ? 4 : i == kCtrUnpool ? kReplicas : 1;
}
constexpr bool counters_fit() {
  for (int i = 0; i < kNumCtr; ++i)
    if (replicas(i) * stripes(i) > kReplicas) return false;
  return true;
}
static_assert(counters_fit(), "a step counter needs more lines than it has");
constexpr int kGenLines = kMaxGrid / kLine;
// Lines within a counter set.
__host__ __device__ constexpr size_t sync_line_ctr(int i, int rep) { return (size_t)i * kReplicas + rep; }
__host__ __device__ constexpr size_t sync_line_up(int e) { return sync_line_ctr(kNumCtr, 0) + e; }
__host__ __device__ constexpr size_t sync_line_down(int e) { return sync_line_up(kBlockMaxExperts) + e; }
__host__ __device__ constexpr size_t sync_line_logits(int rb) { return sync_line_down(kBlockMaxExperts) + rb; }
constexpr size_t kSetLines = sync_line_logits((kSyncMaxRows + kRouterRowBlock - 1) / kRouterRowBlock);
// Line of counter set `set`'s first line, from the start of the state.
__host__ __device__ constexpr size_t sync_line_set(int set) { return 1 + kGenLines + (size_t)set * kSetLines; }
constexpr size_t kSyncWords = sync_line_set(2) * kLine;

constexpr int kRouteReps = 8;  // copies of the tagged routes (each workgroup polls one)
// The few-row unpooler's tasks: kUnpoolTiles 16-feature tiles over a
// contraction split of at most 4 kUnpoolChunks 32-element chunks.
constexpr int kUnpoolTiles = 2;
constexpr int kUnpoolChunks = 12;
constexpr int kFinChunk = 1024;  // features per finalize task (4 per thread: the most one task covers)
constexpr int kMaxPoolSplit = 32;  // contraction splits of the pooler
constexpr int kMaxRowBlocks = 16;  // 64-row blocks of the wide projections' tasks (kMaxRows / 64)
constexpr int kMoeReplicas = 8;  // copies of the MoE output for the unpooler tasks
constexpr int kTimelineSlots = 32;
constexpr int kBlockGroupsPerCu = 3;  // resident workgroups per CU (one wave per SIMD each)

constexpr int kBoundGroups = 8;      // 4-element groups per thread of a boundary row (H <= 8192)


// Streaming layout of the MXFP4 experts (mb_pack_experts).  Per expert, in
// this order:
//   up codes     [I/16 units][P/128 chunks][2 tiles][64 lanes][16 B]
//   up scales    [I/16 units][ceil(P/512) groups][2 tiles][64 lanes][4 B]
//   down codes   [P/32 units][I/128 chunks][2 tiles][64 lanes][16 B]
//   down scales  [P/32 units][ceil(I/512) groups][2 tiles][64 lanes][4 B]
// Up unit u has tiles w13 rows 16u.. (gate) and I + 16u.. (up); down unit u
// has w2 rows 32u.. and 32u + 16..  Lane l's 16 code bytes of chunk c are
// bytes 64 c + 16 (l / 16) of tile row l % 16 (its 32-element MX block of the
// chunk); its 4 scale bytes of group q are the scales of that block in chunks
// 4q .. 4q + 3 (scale bytes 4 (4q + j) + l / 16 of the row), padded with 127
// (2^0) past the row's end.
struct PackedExperts {
  size_t up_s, down, down_s, stride;  // byte offsets within an expert; expert stride
};
__host__ __device__ inline PackedExperts packed_experts(int P, int I) {
  const size_t up = (size_t)I * P;  // (I/16) * (P/128) * 2048
  const size_t up_s = (size_t)(I / 16) * ((P / 128 + 3) / 4) * 512;
  const size_t down = (size_t)P * I / 2;
  const size_t down_s = (size_t)(P / 32) * ((I / 128 + 3) / 4) * 512;
  return PackedExperts{up, up + up_s, up + up_s + down, up + up_s + down + down_s};
}

// The pooler's and unpooler's bf16 weights in the streaming layout
// (mb_pack_projections): a matrix [n_out][kdim] in tiles of 16 rows (rows
// past n_out zero) and chunks of 32 elements, each (tile t, chunk c) the
// kilobyte one wave loads as its MFMA A operand -- lane l's 16 bytes (at
// 16 l) being elements 32 c + 8 (l / 16) .. + 7 of row 16 t + l % 16 -- at
// (t * kdim / 32 + c) * 1024.  The pooler's [P][H] first, then the
// unpooler's [H][P] at `unpool`.
struct PackedProjections {
  size_t unpool, bytes;
};
__host__ __device__ inline size_t packed_matrix_bytes(int n_out, int kdim) {
  return (size_t)((n_out + 15) / 16) * 16 * kdim * 2;
}
__host__ __device__ inline PackedProjections packed_projections(int P, int H) {
  const size_t pool = (packed_matrix_bytes(P, H) + 255) / 256 * 256;
  return PackedProjections{pool, pool + packed_matrix_bytes(H, P)};
}
// Offset of lane `lane`'s 16 bytes of chunk 0 of 16-row tile t of a packed
// matrix with kdim-element rows, from contraction element k0 (a multiple of
// 32); chunk c + 1 follows chunk c at 1024 bytes.
__host__ __device__ inline size_t packed_offset(int t, int kdim, int k0, int lane) {
  return (((size_t)t * (kdim / 32) + k0 / 32) * 64 + lane) * 16;
}

struct BlockParams {
  int b, H, P, I, E, k, scoring;
  float mult, div_eps, route_scale, norm_eps;
  // task counts (0 = step absent) and step switches
  int n_logit_producers;           // router tasks to wait for (0: logits given)
  int n_router, n_route, n_pool, n_prenorm, n_fin, n_unpool, n_boundary;
  int pool_ks, unpool_ks, n_pool_tiles;
  int has_up, needs_routing, routing_out, route_given, logits_in;
  int unpool_wide;  // unpooler in 64-feature tiles (many rows)
  int row_blocks;   // 64-row blocks of the pooler's and wide unpooler's tasks (1 up to 64 rows)
  int router_multi; // router tasks of kRouterExperts experts (many rows)
  int router_mma;   // router tiles of 16 rows x 16 experts on fp64 MFMA (many rows)
  int router_ks;    // their contraction splits (partials added by the last split)
  double *rtr_part; // [router_ks][tiles][16][16] fp64 partials
  unsigned *rtr_cnt;  // [tiles] splits done (left at zero)
  int cus;          // compute units (the grid holds grid / cus workgroups per CU)
  int lds_route_bytes;
  // inputs
  const uint16_t *x;
  const float *router_w, *bias;
  const uint16_t *pool_w, *pre_norm_w;
  const uint8_t *w13, *w13s, *w2, *w2s;
  // the experts in the streaming layout (or NULL), and its byte offsets
  const uint8_t *xp;
  size_t xp_stride, xp_up_s, xp_down, xp_down_s;
  const uint16_t *post_norm_w, *unpool_w, *ffn_norm_w, *gate, *next_norm_w;
  // The pooler's and unpooler's weights in the streaming layout
  // (PackedProjections), or NULL: pool_w / unpool_w as the caller laid them out.
  const uint16_t *pool_wp, *unpool_wp;
  // in/out
  float *stream;
  uint16_t *x_next;
  float *logits;  // given (logits_in) or written when not NULL
  int32_t *ids, *count, *offset, *route_list, *active, *n_active;
  float *wts;
  uint16_t *h, *moe_out, *u;
  // workspace
  float *logits_f;  // the router's fp32 logits
  float *pool_part, *unpool_part, *y, *ssq;
  uint16_t *act, *moe_rep;  // moe_rep: kMoeReplicas copies of [b, P]
  unsigned *pool_cnt, *sync;
  int64_t *timeline;  // optional [grid][kTimelineSlots]
  // MXFP4 activations into the experts (streaming layout).  Last, so that the
  // other fields keep their kernel-argument offsets.
  int w4a4;
  // The next layer's QKV projection fused after the boundary (n_qkv tasks:
  // 64-feature tiles x qkv_ks contraction splits), or n_qkv = 0.
  const uint16_t *qkv_w;
  uint16_t *qkvg;
  float *qkv_part;
  unsigned *qkv_cnt;
  int qkv_rows, n_qkv, qkv_ks;
  // Tagged hand-off words (8 bytes: payload, then the writing launch's tag):
  // the router's fp32 logits [b][E]; the routes, kRouteReps copies of
  // [2 b k] (ids, then weights).
  uint32_t *logits_t, *routes_t;
  // The pooler's h [b][P/2], the pre-norm's normed h (same shape), and act
  // [R][I/2], as tagged words of two bf16.  h_tagged: the up units read h
  // from h_t / hn_t (the launch's pooler made it), else from h (the
  // caller's).  h_plain: also write h in bf16 (an output).  act_tap: also
  // write act in bf16 there (or NULL).
  uint32_t *h_t, *hn_t, *act_t;
  uint16_t *act_tap;
  int h_tagged, h_plain;
  // Plain staging (the many-rows instance only): the expert units stage h
  // and act as plain bf16 (h, act) behind counters instead of polling tagged
  // words -- h once every pooler tile (or pre-norm row) signalled its step
  // counter (n_h_ready signals), act once the expert's up units signalled
  // its up counter.
  int plain_stage, n_h_ready;
};
constexpr int kMaxQkvGroups = 1024;  // 64-feature tiles of the fused projection (qkv_rows <= 65536)

// Routing state each workgroup keeps in LDS.
struct RouteLds {
  uint8_t *ids;  // [b*k] (experts < 256)
  float *w;      // [b*k]
  uint16_t *rl;  // [b*k] route list (b*k < 65536)
  int *off;    // [E+1]
  int *act;    // [E]
  int *nact;   // [1]; nact[1] holds the launch's generation, nact[2] the entries of vact
  int *red;    // [8] scan scratch
  unsigned long long *bits;  // [E * ceil(b/64)]
  // Many-rows instance: the active experts' passes of up to 32 rows, each
  // with units of its own (expert | pass << 8), in the order of act.  Written
  // once the grouping has read the bitmaps, over them: at most E + b k / 32
  // entries of 2 bytes, within the bitmaps' 8 E ceil(b / 64) bytes for any b
  // (k <= E).
  uint16_t *vact;
};

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ inline size_t route_lds_bytes(int b, int k, int E) {
  const size_t R = (size_t)b * k, W = (size_t)(b + 63) / 64;
  return align16(R) + align16(R * 4) + align16(R * 2) + align16((E + 1) * 4) + align16(E * 4) + 16 + 32 +
         align16(E * W * 8);
}

__device__ inline RouteLds route_lds(const BlockParams &p, unsigned char *base) {
  const size_t R = (size_t)p.b * p.k, W = (size_t)(p.b + 63) / 64;
  RouteLds r;
  size_t o = 0;
  r.ids = base + o;
  o += align16(R);
  r.w = reinterpret_cast<float *>(base + o);
  o += align16(R * 4);
  r.rl = reinterpret_cast<uint16_t *>(base + o);
  o += align16(R * 2);
  r.off = reinterpret_cast<int *>(base + o);
  o += align16((p.E + 1) * 4);
  r.act = reinterpret_cast<int *>(base + o);
  o += align16(p.E * 4);
  r.nact = reinterpret_cast<int *>(base + o);
  o += 16;
  r.red = reinterpret_cast<int *>(base + o);
  o += 32;
  r.bits = reinterpret_cast<unsigned long long *>(base + o);
  r.vact = reinterpret_cast<uint16_t *>(r.bits);
  (void)W;
  return r;
}

// Activation staging of the expert units, per workgroup: pr rows (8, 16 or
// 32) of up to kStageChunkRows / pr chunks of 128 bf16, with 16 bytes of
// padding after each row (spreading the rows over the LDS banks); each thread
// loads kSegLoads 16-byte pieces of a segment.
constexpr int kStageChunkRows = 128;  // rows x chunks of one segment
constexpr int kSegLoads = kStageChunkRows * 16 / 256;
constexpr size_t kStageBytes = 64 * (256 * 2 + 16);  // also the projections' 64 rows x 256 elements
constexpr size_t kProjScratchBytes = 4 * 4 * 64 * 16 + 64;
constexpr size_t kBlockScratchBytes = kProjScratchBytes > kStageBytes ? kProjScratchBytes : kStageBytes;

hipError_t launch_block(const BlockParams &p, int grid, size_t lds, hipStream_t s);
int block_max_groups_per_cu(size_t lds, bool w4a4, bool qkv, bool many);
hipError_t launch_block_many(const BlockParams &p, int grid, size_t lds, hipStream_t s);
int block_max_groups_per_cu_many(size_t lds);
hipError_t launch_block_w4a4(const BlockParams &p, int grid, size_t lds, hipStream_t s);
int block_max_groups_per_cu_w4a4(size_t lds, bool qkv);
hipError_t launch_block_qkv(const BlockParams &p, int grid, size_t lds, hipStream_t s);
hipError_t launch_block_w4a4_qkv(const BlockParams &p, int grid, size_t lds, hipStream_t s);
int block_max_groups_per_cu_w4a4_qkv(size_t lds);
int block_max_groups_per_cu_qkv(size_t lds);

}  // namespace mb
