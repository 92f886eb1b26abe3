// Host-side internals of libmb.so: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mb.h"

namespace mb {

constexpr int kMaxRows = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxBitmapWords = 4096;  // experts * ceil(rows / 64)
constexpr int kMaxSplitK = 8;          // split-K factor of the bf16 projections

// Byte offsets of the workspace regions (each 256-byte aligned).  The
// regions of plain data grow from the start of the workspace; the regions of
// tagged hand-off words (t_*, offsets from the tagged region's start) sit at
// its end, in its last `tagged` bytes, so that plain data a call with other
// sizes leaves behind never lands where a call polls tagged words (given a
// workspace sized for the largest sizes it serves).
struct Layout {
  size_t sync, logits, ids, wts, count, offset, route_list, active, n_active;
  size_t h, act, y, ssq, moe_out, moe_rep, u, partial;
  size_t pool_part, unpool_part, pool_cnt, qkv_cnt, qkv_part;
  size_t t_logits, t_routes, t_h, t_hn, t_act, tagged;
  size_t rtr_part, rtr_cnt;
  size_t total;
};

Layout layout_of(const mb_dims &d);

// Start of the tagged region in a workspace of ws_bytes (>= L.total) bytes.
inline size_t tagged_base(const Layout &L, size_t ws_bytes) { return (ws_bytes - L.tagged) & ~(size_t)255; }

template <typename T>
inline T *at(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// Routing: logits (unless given), scores + top-k + weights, grouping.
hipError_t launch_router_logits(const mb_dims &d, const uint16_t *x, const float *router_w,
                                float *logits, hipStream_t s);
hipError_t launch_route_select(const mb_dims &d, const float *logits, const float *bias,
                               int32_t *ids, float *wts, hipStream_t s);
hipError_t launch_route_group(const mb_dims &d, const int32_t *ids, int32_t *count,
                              int32_t *offset, int32_t *route_list, int32_t *active,
                              int32_t *n_active, hipStream_t s);

// out[t, n] = bf16(sum_k a[t, k] * w[n, k]) for t < rows, n < n_out; a bf16
// [rows, kdim], w bf16 [n_out, kdim].  Split-K partials and per-tile counters
// come from the workspace.
// out = bf16(a @ w^T), split along kdim into at most ks_cap (<= kMaxSplitK)
// parts whose fp32 partials [ks][rows][n_out] go to `partial`.
hipError_t launch_gemm_bf16(const uint16_t *a, const uint16_t *w, uint16_t *out, int rows,
                            int n_out, int kdim, float *partial, uint32_t *counters,
                            hipStream_t s, int ks_cap = kMaxSplitK);

// In-place h[t] = bf16(RMSNorm(h[t]) * w) over `width` elements.
hipError_t launch_rownorm_bf16(uint16_t *h, const uint16_t *w, int rows, int width, float eps,
                               hipStream_t s);

// Experts: w13 + gated activation into act (route-sorted rows); w2 into y
// (route order) with per-tile sums of squares; the per-route norm, weights
// and sum over routes into moe_out.
hipError_t launch_experts_up(const mb_dims &d, const uint16_t *h, const int32_t *offset,
                             const int32_t *route_list, const int32_t *active,
                             const int32_t *n_active, const uint8_t *w13,
                             const uint8_t *w13_scale, uint16_t *act, hipStream_t s);
hipError_t launch_experts_down(const mb_dims &d, const uint16_t *act, const int32_t *offset,
                               const int32_t *route_list, const int32_t *active,
                               const int32_t *n_active, const uint8_t *w2,
                               const uint8_t *w2_scale, float *y, float *ssq, hipStream_t s);
hipError_t launch_experts_finalize(const mb_dims &d, const float *y, const float *ssq,
                                   const float *wts, const uint16_t *post_norm_w,
                                   uint16_t *moe_out, hipStream_t s);

// The pooler's and unpooler's weights in the streaming layout (PackedProjections).
hipError_t launch_pack_projections(const mb_dims &d, const uint16_t *pool_w, const uint16_t *unpool_w,
                                   uint8_t *packed, hipStream_t s);

// The experts' codes and scales in the streaming layout (PackedExperts).
hipError_t launch_pack_experts(const mb_dims &d, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                               const uint8_t *w2s, uint8_t *packed, hipStream_t s);

// The workspace's abort record: read into *status (MB_OK / MB_ERR_ABORTED),
// or cleared when status is NULL.
hipError_t launch_abort_word(void *workspace, int32_t *status, hipStream_t s);

// Effective norm multiplier: out = bf16(weight + add).
hipError_t launch_norm_weight(const float *weight, int n, float add, uint16_t *out, hipStream_t s);

// Boundary: RMSNorm of u, gated add into the fp32 stream, next pre-norm.
hipError_t launch_boundary(const mb_dims &d, const uint16_t *u, float *stream,
                           const uint16_t *gate, const uint16_t *ffn_norm_w,
                           const uint16_t *next_norm_w, uint16_t *x_next, hipStream_t s);

}  // namespace mb
