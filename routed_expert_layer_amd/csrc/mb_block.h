// Parameters and LDS layout of the persistent block kernel (block.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mb_internal.h"

namespace mb {

// Per-launch dependency counters (mb_sync.h region at the workspace start):
// words [0] epoch, [1] abort; then two counter sets of kCtrUp + 2E counters,
// kCtrStride words apart.
constexpr int kCtrStride = 16;
constexpr int kSyncHeader = 64;
enum : int {
  kCtrLogits = 0,    // router tasks done
  kCtrRoute = 1,     // route tasks done
  kCtrPool = 2,      // pooler tiles complete
  kCtrPrenorm = 3,   // pre-norm rows done
  kCtrFin = 4,       // finalize tasks done
  kCtrUnpool = 5,    // unpooler tiles complete
  kCtrFinished = 6,  // workgroups finished
  kCtrUp = 8,        // [E] up tasks done per expert, then [E] down tasks done
};
constexpr int kFinChunk = 512;  // features per finalize task
constexpr int kBlockMaxExperts = 256;  // larger expert counts use the per-step kernels
constexpr int kTimelineSlots = 16;

// Router hidden slice width (a multiple of 256, at most H) so that a router
// task does about 16K fp64 multiply-adds, and the slice count.
inline int router_slice(int b, int H) {
  int sw = 16384 / b;
  sw = (sw / 256) * 256;
  if (sw < 256) sw = 256;
  return sw > H ? H : sw;
}
inline int router_slices(int b, int H) { return (H + router_slice(b, H) - 1) / router_slice(b, H); }

inline size_t sync_words(int E) { return kSyncHeader + 2 * (size_t)(kCtrUp + 2 * E) * kCtrStride; }

struct BlockParams {
  int b, H, P, I, E, k, scoring;
  float mult, div_eps, route_scale, norm_eps;
  // task counts (0 = step absent) and step switches
  int rslices, rslice;             // router hidden slices
  int n_router, n_route, n_pool, n_prenorm, n_fin, n_unpool, n_boundary;
  int pool_ks, unpool_ks, n_pool_tiles, n_unpool_tiles, h_producers;
  int has_up, needs_routing, routing_out, route_given, logits_in;
  int lds_route_bytes;
  // inputs
  const uint16_t *x;
  const float *router_w, *bias;
  const uint16_t *pool_w, *pre_norm_w;
  const uint8_t *w13, *w13s, *w2, *w2s;
  const uint16_t *post_norm_w, *unpool_w, *ffn_norm_w, *gate, *next_norm_w;
  // in/out
  float *stream;
  uint16_t *x_next;
  float *logits;  // given (logits_in) or written when not NULL
  int32_t *ids, *count, *offset, *route_list, *active, *n_active;
  float *wts;
  uint16_t *h, *moe_out, *u;
  // workspace
  double *logit_part;
  float *pool_part, *unpool_part, *y, *ssq;
  uint16_t *act;
  unsigned *pool_cnt, *unpool_cnt, *sync;
  int64_t *timeline;  // optional [grid][kTimelineSlots]
};

// Routing state each workgroup keeps in LDS.
struct RouteLds {
  int *ids;    // [b*k]
  float *w;    // [b*k]
  int *rl;     // [b*k] route list
  int *off;    // [E+1]
  int *act;    // [E]
  int *nact;   // [1]
  int *red;    // [8] scan scratch
  unsigned long long *bits;  // [E * ceil(b/64)]
};

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ inline size_t route_lds_bytes(int b, int k, int E) {
  const size_t R = (size_t)b * k, W = (size_t)(b + 63) / 64;
  return align16(R * 4) * 3 + align16((E + 1) * 4) + align16(E * 4) + 16 + 32 + align16(E * W * 8);
}

__device__ inline RouteLds route_lds(const BlockParams &p, unsigned char *base) {
  const size_t R = (size_t)p.b * p.k, W = (size_t)(p.b + 63) / 64;
  RouteLds r;
  size_t o = 0;
  r.ids = reinterpret_cast<int *>(base + o);
  o += align16(R * 4);
  r.w = reinterpret_cast<float *>(base + o);
  o += align16(R * 4);
  r.rl = reinterpret_cast<int *>(base + o);
  o += align16(R * 4);
  r.off = reinterpret_cast<int *>(base + o);
  o += align16((p.E + 1) * 4);
  r.act = reinterpret_cast<int *>(base + o);
  o += align16(p.E * 4);
  r.nact = reinterpret_cast<int *>(base + o);
  o += 16;
  r.red = reinterpret_cast<int *>(base + o);
  o += 32;
  r.bits = reinterpret_cast<unsigned long long *>(base + o);
  (void)W;
  return r;
}

// Scratch LDS the phases need beyond the routing state.
constexpr size_t kBlockScratchBytes = 4 * 4 * 64 * 16 + 64;

hipError_t launch_block(const BlockParams &p, int grid, size_t lds, hipStream_t s);
int block_max_groups_per_cu(size_t lds);

}  // namespace mb
