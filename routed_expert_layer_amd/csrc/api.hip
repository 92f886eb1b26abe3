// The C ABI of libmb.so (declared and documented in include/mb.h): argument
// checks, workspace layout and the launch sequence of each entry point.

#include <math.h>

#include "mb_internal.h"

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
  L.u = take(b * H * 2);
  L.partial = take((size_t)kMaxSplitK * b * wide * 4);
  L.counters = take(8 * (wide / 16) * 4);
  L.total = o;
  return L;
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

int check_weights_route(const mb_weights *w, int flags, const uint16_t *x) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->expert_bias}));
  if (!(flags & MB_LOGITS_IN)) MB_TRY(need({x, w->router_w}));
  return MB_OK;
}

int check_weights_experts(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  return need({w->w13, w->w13_scale, w->w2, w->w2_scale, w->post_norm_w});
}

int check_weights_boundary(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->unpool_w, w->gate}));
  return maybe({w->ffn_norm_w, w->next_norm_w});
}

int check_weights_pool(const mb_weights *w) {
  if (!w) return MB_ERR_NULL;
  MB_TRY(need({w->pool_w}));
  return maybe({w->pre_norm_w});
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
  const Layout L = layout_of(d);
  MB_HIP(launch_gemm_bf16(x, w->pool_w, h, d.rows, d.pooled, d.hidden, at<float>(ws, L.partial),
                          at<uint32_t>(ws, L.counters), s));
  if (w->pre_norm_w) MB_HIP(launch_rownorm_bf16(h, w->pre_norm_w, d.rows, d.pooled, d.norm_eps, s));
  return MB_OK;
}

int run_experts(const mb_dims &d, const uint16_t *h, const float *wts, const int32_t *offset,
                const int32_t *route_list, const int32_t *active, const int32_t *n_active,
                const mb_weights *w, uint16_t *moe_out, void *ws, hipStream_t s) {
  const Layout L = layout_of(d);
  uint16_t *act = at<uint16_t>(ws, L.act);
  float *y = at<float>(ws, L.y), *ssq = at<float>(ws, L.ssq);
  MB_HIP(launch_experts_up(d, h, offset, route_list, active, n_active, w->w13, w->w13_scale, act, s));
  MB_HIP(launch_experts_down(d, act, offset, route_list, active, n_active, w->w2, w->w2_scale, y,
                             ssq, s));
  MB_HIP(launch_experts_finalize(d, y, ssq, wts, w->post_norm_w, moe_out, s));
  return MB_OK;
}

int run_unpool_boundary(const mb_dims &d, const uint16_t *moe_out, const mb_weights *w,
                        float *stream, uint16_t *x_next, uint16_t *u, void *ws, hipStream_t s) {
  const Layout L = layout_of(d);
  MB_HIP(launch_gemm_bf16(moe_out, w->unpool_w, u, d.rows, d.hidden, d.pooled,
                          at<float>(ws, L.partial), at<uint32_t>(ws, L.counters), s));
  MB_HIP(launch_boundary(d, u, stream, w->gate, w->ffn_norm_w, w->next_norm_w, x_next, s));
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
  return run_unpool_boundary(*dims, moe_out, w, stream, x_next, u, workspace,
                             (hipStream_t)stream_handle);
}

int mb_moe_block(const mb_dims *dims, const uint16_t *x, const mb_weights *w, float *stream,
                 uint16_t *x_next, const mb_block_taps *taps, void *workspace,
                 size_t workspace_bytes, void *stream_handle) {
  MB_TRY(check_dims(dims));
  MB_TRY(check_weights_route(w, 0, x));
  MB_TRY(check_weights_pool(w));
  MB_TRY(check_weights_experts(w));
  MB_TRY(check_weights_boundary(w));
  MB_TRY(need({stream, x_next}));
  mb_block_taps tp{};
  if (taps) {
    tp = *taps;
    MB_TRY(maybe({tp.logits, tp.topk_ids, tp.topk_w, tp.count, tp.offset, tp.route_list,
                  tp.active, tp.n_active, tp.h, tp.moe_out, tp.u}));
  }
  MB_TRY(check_ws(dims, workspace, workspace_bytes));
  const mb_dims &d = *dims;
  const Layout L = layout_of(d);
  void *ws = workspace;
  const hipStream_t s = (hipStream_t)stream_handle;
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
  MB_TRY(run_route(d, x, w, logits, 0, ids, wts, count, offset, route_list, active, n_active, s));
  MB_TRY(run_pool(d, x, w, h, ws, s));
  MB_TRY(run_experts(d, h, wts, offset, route_list, active, n_active, w, moe_out, ws, s));
  return run_unpool_boundary(d, moe_out, w, stream, x_next, u, ws, s);
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
    case MB_ERR_WORKSPACE: return "workspace missing or smaller than mb_workspace_bytes";
    case MB_ERR_HIP: return "a kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
