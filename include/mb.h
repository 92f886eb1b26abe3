/*
 * mb.h - C ABI of the MI355X (gfx950) routed-MoE block library libmb.so.
 *
 * The library computes one decode/verify step of a MuseSpark1x-style routed
 * mixture-of-experts block on one GPU:
 *
 *   router (fp32) -> sigmoid/softmax scores -> top-k with a selection-only
 *   expert bias -> normalised, scaled route weights -> route grouping
 *   -> bf16 pooler H->P -> per-route MXFP4 experts (w13, gated activation, w2)
 *   -> per-route RMSNorm over P -> weighted sum over routes -> bf16 unpooler
 *   P->H -> boundary (RMSNorm, gated add into the fp32 residual stream, next
 *   pre-norm).
 *
 * Sources, by page title and section:
 *   [muse_moe_runner] vllm.models.muse_spark.amd.muse_moe_runner
 *   [mono.decoder]    vllm.models.muse_spark.amd.mono.decoder
 *   [providers]       vllm.models.muse_spark.nvidia.specialized_decode.runtime.providers
 *
 * Conventions (all entry points):
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Every tensor pointer is DEVICE memory, row-major and contiguous, and
 *     must be 16-byte aligned (MB_ERR_ALIGN otherwise).  Sizes are in
 *     elements unless stated.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates, frees or synchronises; weights are read in place, never
 *     copied ([mono.decoder] collect_layer_weights: views, no copy;
 *     [providers] Provider: run allocates nothing).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream) ([providers]: every provider launches on the current
 *     stream).  Argument checks happen on the host before any launch; a
 *     nonzero status means nothing was enqueued, except MB_ERR_HIP, which
 *     reports a failed launch.  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - The workspace must be zero-filled once before its first use.  Every
 *     call leaves it ready for the next (the persistent launch keeps two
 *     counter sets there and a generation count that picks one; each launch
 *     clears the set the next one uses), so one workspace serves any number
 *     of calls, also replays of a captured graph.  Calls that share a
 *     workspace must not overlap.
 *   - Limits (MB_ERR_UNSUPPORTED beyond them): rows <= 1024, experts <= 1024,
 *     top_k <= 16, experts * ceil(rows / 64) <= 4096, hidden % 32 == 0,
 *     pooled % 128 == 0, inter % 128 == 0.
 */
#ifndef MB_H
#define MB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MB_OK = 0,
  MB_ERR_NULL = 1,        /* a required pointer is NULL */
  MB_ERR_DIMS = 2,        /* non-positive size, top_k > experts, bad scoring */
  MB_ERR_UNSUPPORTED = 3, /* outside the limits above */
  MB_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  MB_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than mb_workspace_bytes */
  MB_ERR_HIP = 6,         /* a kernel launch failed */
  MB_ERR_ABORTED = 7,     /* (mb_workspace_status) a launch on the workspace
                             gave up a wait: its results are not to be trusted */
  MB_ERR_SCRATCH = 8      /* (mb_moe_block_noalloc) the sizes need more than its
                             static scratch */
};

/* The static scratch of mb_moe_block_noalloc, per GPU: its size, and the
 * part at its end that holds the block kernel's hand-off words. */
#define MB_NOALLOC_SCRATCH_BYTES (64u << 20)
#define MB_NOALLOC_TAGGED_BYTES (8u << 20)

/* Scoring functions ([muse_moe_runner] MuseSpark1xRouter: the score
 * normalisation is "sigmoid" or "softmax"; anything else is a ValueError). */
enum { MB_SCORING_SIGMOID = 0, MB_SCORING_SOFTMAX = 1 };

/* mb_route flags. */
enum {
  MB_LOGITS_OUT = 1, /* also write the fp32 router logits [rows, experts] */
  MB_LOGITS_IN = 2   /* skip the projection; route from the caller's logits */
};

/* Block sizes and routing scalars.
 *   rows     b, the tokens (decode/verify rows) of the step
 *   hidden   H, model width            pooled  P, expert input width
 *   inter    I, expert intermediate    experts E, top_k k
 * route_scale, router_multiplier and division_eps follow [muse_moe_runner]
 * MuseSpark1xRouter: an absent multiplier is 1.0f and an absent eps is 0.0f
 * (both leave the fp32 result unchanged).  norm_eps is the epsilon of every
 * RMSNorm in the block.
 * act_quant 0: the experts multiply bf16 activations (h, act) by the
 * dequantized MXFP4 weights.  act_quant 1 (the W4A4 variant, [providers]
 * MoEProvider: the FP4 x FP4 expert recipe): h and act are each quantized to
 * MXFP4 along the contraction, per block of 32 consecutive elements, by the
 * OCP Microscaling v1.0 conversion (shared scale 2^(floor(log2 amax) - 2) as
 * an E8M0 byte, clamped to [2^-127, 2^127], 1 for an all-zero block;
 * elements scaled and rounded to the nearest E2M1 value, ties to the even
 * code, magnitudes above 6 saturating to 6), and each contraction runs on
 * fp4 x fp4 products.  act_quant 1 runs in the block kernel only: it needs
 * w->experts_packed and sizes the block kernel takes (experts <= 256,
 * hidden <= 8192, route tables within its LDS), else MB_ERR_UNSUPPORTED.
 * qkv_rows 0: mb_moe_block ends at the boundary.  qkv_rows > 0 (a multiple
 * of 16, at most 65536): mb_moe_block also runs the next layer's QKV
 * projection of x_next (as mb_next_qkv, with w->next_qkv_w bf16
 * [qkv_rows, H]) in the same launch, into taps->qkvg (both required). */
typedef struct {
  int32_t rows, hidden, pooled, inter, experts, top_k;
  int32_t scoring;
  float route_scale;
  float router_multiplier;
  float division_eps;
  float norm_eps;
  int32_t act_quant;
  int32_t qkv_rows;
} mb_dims;

/* The block's weights, all device pointers, in the layouts the pages fix:
 *   router_w    fp32 [E, H]   ([mono.decoder] layer_refusals: router fp32 (E, H))
 *   expert_bias fp32 [E]      selection-only bias
 *   pool_w      bf16 [P, H]   pooler   ([mono.decoder] layer_refusals)
 *   pre_norm_w  bf16 [P] or NULL: optional RMSNorm of the pooler output
 *               ([providers] MoEProvider: pre_expert_norm)
 *   w13         u8 [E, 2I, P/2]  MXFP4 codes, rows [0, I) gate, [I, 2I) up
 *   w13_scale   u8 [E, 2I, P/32] E8M0 scales
 *   w2          u8 [E, P, I/2]   w2_scale u8 [E, P, I/32]
 *               ([mono.decoder] MonoDims.expert_shapes; two E2M1 codes per
 *               byte, the even element in the low nibble; one E8M0 scale per
 *               32 elements along the contraction dimension)
 *   post_norm_w bf16 [P]      per-route norm weight
 *   unpool_w    bf16 [H, P]   unpooler ([mono.decoder] layer_refusals)
 *   ffn_norm_w  bf16 [H] or NULL (= 1): boundary post-FFN norm weight
 *   gate        bf16 [H]      boundary gate g
 *   next_norm_w bf16 [H] or NULL (= 1): next layer's pre-norm weight
 *   experts_packed  NULL, or the output of mb_pack_experts for these
 *               w13 / w2: the experts in the layout the block kernel
 *               streams.  When set, w13, w13_scale, w2 and w2_scale may be
 *               NULL; the per-step kernels (sizes the block kernel does not
 *               take) need them and return MB_ERR_UNSUPPORTED without them.
 *   proj_packed NULL, or the output of mb_pack_projections for these pool_w /
 *               unpool_w: both in the layout the block kernel streams.  When
 *               set, pool_w and unpool_w may be NULL (the per-step kernels
 *               then return MB_ERR_UNSUPPORTED, as for experts_packed).
 * Norm weights are the effective bf16 multipliers ([mono.decoder]
 * effective_norm_weight), applied after normalising. */
typedef struct {
  const float *router_w;
  const float *expert_bias;
  const uint16_t *pool_w;
  const uint16_t *pre_norm_w;
  const uint8_t *w13;
  const uint8_t *w13_scale;
  const uint8_t *w2;
  const uint8_t *w2_scale;
  const uint16_t *post_norm_w;
  const uint16_t *unpool_w;
  const uint16_t *ffn_norm_w;
  const uint16_t *gate;
  const uint16_t *next_norm_w;
  const uint8_t *experts_packed;
  const uint16_t *next_qkv_w;  /* bf16 [dims->qkv_rows, H] or NULL (qkv_rows 0) */
  const uint8_t *proj_packed;
} mb_weights;

/* Optional intermediate outputs of mb_moe_block.  A NULL member is kept in
 * the workspace instead.  Shapes as in mb_route / mb_pool / mb_experts /
 * mb_unpool_boundary. */
typedef struct {
  float *logits;       /* fp32 [b, E] */
  int32_t *topk_ids;   /* int32 [b, k] */
  float *topk_w;       /* fp32 [b, k] */
  int32_t *count;      /* int32 [E] */
  int32_t *offset;     /* int32 [E + 1] */
  int32_t *route_list; /* int32 [b * k] */
  int32_t *active;     /* int32 [E] */
  int32_t *n_active;   /* int32 [1] */
  uint16_t *h;         /* bf16 [b, P] */
  uint16_t *moe_out;   /* bf16 [b, P] */
  uint16_t *u;         /* bf16 [b, H] */
  int64_t *timeline;   /* tracing: int64 [1024][32]; workgroup w keeps the
                          100 MHz real-time counter at its phase boundaries
                          and writes them into row w at its end (0 = slot
                          not reached; the per-step path leaves it untouched) */
  uint16_t *act;       /* bf16 [b * k, I]: the experts' gated activations
                          act = bf16(silu(gu[0:I]) * gu[I:2I]) (mb_experts),
                          row i for route route_list[i] (grouped by expert) */
  uint16_t *qkvg;      /* bf16 [b, qkv_rows]: the fused next-QKV projection
                          of x_next (required when dims->qkv_rows > 0) */
} mb_block_taps;

/* Bytes of workspace every entry point needs for these dims (the same size
 * serves all of them).  Returns MB_OK, MB_ERR_NULL, MB_ERR_DIMS or
 * MB_ERR_UNSUPPORTED. */
int mb_workspace_bytes(const mb_dims *dims, size_t *bytes);

/* Router and routing ([muse_moe_runner] MuseSpark1xRouter and its
 * _compute_routing_native recipe; [providers] RoutedTopk).
 *   logits = x @ router_w^T (fp32 [b, E]; x bf16 [b, H]); optional output
 *   multiplier; sigmoid or softmax; selection key = score + expert_bias
 *   (selection only); top-k by key descending, lowest expert id first among
 *   equal keys, slot j = rank j; weights = gathered UNBIASED scores divided by
 *   (their sum + division_eps), times route_scale, in fp32.
 * Outputs: topk_ids int32 [b, k], topk_w fp32 [b, k], and the route grouping
 * the experts consume: count int32 [E] routes per expert; offset int32 [E+1]
 * exclusive prefix sum (offset[E] = b*k); route_list int32 [b*k], the routes
 * r = t*k + j sorted by (expert, r); active int32 [E], the experts with
 * count > 0 ascending, n_active int32 [1] of them (the rest of `active` is
 * left unwritten).
 * flags: MB_LOGITS_OUT writes the logits to `logits` (may then not be NULL);
 * MB_LOGITS_IN reads them from `logits` and ignores x and router_w. */
int mb_route(const mb_dims *dims, const uint16_t *x, const mb_weights *w,
             float *logits, int flags, int32_t *topk_ids, float *topk_w,
             int32_t *count, int32_t *offset, int32_t *route_list,
             int32_t *active, int32_t *n_active, void *workspace,
             size_t workspace_bytes, void *stream);

/* Pooler: h = bf16(x @ pool_w^T), bf16 [b, P]; then, if w->pre_norm_w is not
 * NULL, h = bf16(RMSNorm_P(h) * pre_norm_w) ([providers] MoEProvider:
 * pooler GEMM + pre_expert_norm; [mono.decoder] _K5Bucket: h bf16 [rows, P]).
 * Independent of routing ([providers] RoutedMoE.run runs it beside the
 * routing). */
int mb_pool(const mb_dims *dims, const uint16_t *x, const mb_weights *w,
            uint16_t *h, void *workspace, size_t workspace_bytes,
            void *stream);

/* Routed experts and tail ([muse_moe_runner] MuseSparkAiterExperts.apply:
 * one unweighted output per route; MuseSparkTopKWeightAndReduce.apply:
 * per-route norm, then route weight, then sum over routes, then cast).
 * For each route (t, j) with e = topk_ids[t, j]:
 *   gu  = dec(w13[e]) @ h[t]                 (fp32, 2I values)
 *   act = bf16(silu(gu[0:I]) * gu[I:2I])
 *   y   = dec(w2[e]) @ act                   (fp32, P values)
 *   yn  = y / sqrt(mean(y^2) + norm_eps) * post_norm_w
 * moe_out[t] = bf16(sum_j topk_w[t, j] * yn(t, j)), bf16 [b, P].
 * The grouping arrays are mb_route's outputs for the same topk_ids. */
int mb_experts(const mb_dims *dims, const uint16_t *h, const int32_t *topk_ids,
               const float *topk_w, const int32_t *count,
               const int32_t *offset, const int32_t *route_list,
               const int32_t *active, const int32_t *n_active,
               const mb_weights *w, uint16_t *moe_out, void *workspace,
               size_t workspace_bytes, void *stream);

/* Unpooler and boundary ([providers] BoundaryProvider: post_ffn_norm, the
 * gated add into the fp32 stream in place, the next pre-norm into bf16 out;
 * [providers] MoEProvider: the unpooler GEMM):
 *   u      = bf16(moe_out @ unpool_w^T)                     bf16 [b, H]
 *   v      = RMSNorm_H(u) * ffn_norm_w
 *   stream = fp32(stream + gate * v)                        in place, fp32 [b, H]
 *   x_next = bf16(RMSNorm_H(stream) * next_norm_w)          bf16 [b, H]
 * u_out may be NULL (u then stays in the workspace). */
int mb_unpool_boundary(const mb_dims *dims, const uint16_t *moe_out,
                       const mb_weights *w, float *stream, uint16_t *x_next,
                       uint16_t *u_out, void *workspace,
                       size_t workspace_bytes, void *stream_handle);

/* The whole block: mb_route + mb_pool, mb_experts, mb_unpool_boundary in one
 * call ([providers] MoEProvider followed by BoundaryProvider; [mono.decoder]
 * _K3Bucket runs the layer as a single launch at small row counts).  x bf16
 * [b, H] in; stream fp32 [b, H] updated in place; x_next bf16 [b, H] out.
 * taps may be NULL. */
int mb_moe_block(const mb_dims *dims, const uint16_t *x, const mb_weights *w,
                 float *stream, uint16_t *x_next, const mb_block_taps *taps,
                 void *workspace, size_t workspace_bytes, void *stream_handle);

/* mb_moe_block for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results, with the workspace replaced by a static
 * device array of MB_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds
 * on every GPU it runs on, until the process ends.  Nothing is allocated
 * or freed, by the library or any library it calls.
 *   - Sizes: the workspace layout's buffers must fit in the first 56 MiB and
 *     its hand-off words in the last MB_NOALLOC_TAGGED_BYTES (8 MiB), else
 *     MB_ERR_SCRATCH before anything is enqueued.  Up to 91 rows fit at
 *     H 4096, P 2048, I 1024, E 64, top_k 4 and up to 53 rows at H 7168,
 *     P 3072, I 1536, E 128, top_k 8; mb_moe_block with a workspace serves
 *     larger sizes.
 *   - The first call on a GPU (with that GPU current) looks up the array's
 *     address there and enqueues its zero-fill on `stream_handle`.
 *   - Every call on a GPU shares that GPU's array, which keeps the last
 *     call's state: calls on one GPU must not overlap (one stream, or
 *     ordered by events); calls that overlap race and their results are
 *     undefined.  mb_workspace_status / mb_workspace_reset do not reach it.
 *   - Other arguments, outputs and errors as mb_moe_block. */
int mb_moe_block_noalloc(const mb_dims *dims, const uint16_t *x, const mb_weights *w,
                         float *stream, uint16_t *x_next, const mb_block_taps *taps,
                         void *stream_handle);

/* Bytes of the streaming layout of all E experts (for mb_pack_experts). */
int mb_packed_experts_bytes(const mb_dims *dims, size_t *bytes);

/* Copy the MXFP4 experts (w13, w13_scale, w2, w2_scale of `w`, all required)
 * into `packed` (device memory, at least mb_packed_experts_bytes, 16-byte
 * aligned) in the layout the block kernel streams: per expert and unit (16
 * gate + 16 up rows of w13, then 32 rows of w2), per 128-element chunk, the
 * 1 KB that one wave loads for each of the unit's two 16-row tiles, lane l
 * getting bytes 64 c + 16 (l / 16) of row l % 16; then the unit's E8M0
 * scales, per 4 chunks and tile 256 bytes, lane l's 4 bytes (at 4 l) being the
 * scales of its blocks of the 4 chunks, padded with 127 (= 2^0).  The values
 * are unchanged, so results are bit-identical to the caller's layout.  Meant
 * for load time, like the weight preparation of [muse_moe_runner]
 * MuseSparkAiterExperts; the caller owns `packed` and keeps it with the
 * weights.  Asynchronous on `stream`.  MB_ERR_WORKSPACE if packed_bytes is
 * too small. */
int mb_pack_experts(const mb_dims *dims, const mb_weights *w, uint8_t *packed, size_t packed_bytes,
                    void *stream);

/* Bytes of the streaming layout of the pooler's and unpooler's weights (for
 * mb_pack_projections). */
int mb_packed_projections_bytes(const mb_dims *dims, size_t *bytes);

/* Copy the bf16 pooler and unpooler weights (pool_w [P, H] and unpool_w
 * [H, P] of `w`, both required) into `packed` (device memory, at least
 * mb_packed_projections_bytes, 16-byte aligned) in the layout the block
 * kernel streams: per matrix of n_out rows of kdim elements, per 16-row tile t
 * (rows past n_out zero) and 32-element chunk c, the kilobyte one wave loads,
 * lane l's 16 bytes at 16 l holding elements 32 c + 8 (l / 16) .. + 7 of row
 * 16 t + l % 16, at byte (t * kdim / 32 + c) * 1024; pool_w's matrix first,
 * unpool_w's from byte ceil(ceil(P / 16) * 16 * H * 2 / 256) * 256.  (Sixteen
 * rows' 64-byte pieces per wave load, as the caller's row-major layout gives,
 * come at a fraction of the rate of contiguous loads.)  The values are
 * unchanged, so results are bit-identical to the caller's layout.  Load-time
 * preparation, as for mb_pack_experts ([muse_moe_runner] MuseSparkAiterExperts
 * takes its weights prepared at load time); the caller owns `packed`.
 * Asynchronous on `stream`.  MB_ERR_WORKSPACE if packed_bytes is too small. */
int mb_pack_projections(const mb_dims *dims, const mb_weights *w, uint8_t *packed, size_t packed_bytes,
                        void *stream);

/* The attention boundary, the step before the block ([providers]
 * AttentionBoundaryProvider: post_attn_norm, the gated add into the fp32
 * stream in place, pre_ffn_norm into bf16 out).  The provider first
 * all-reduces the attention's row-parallel o_proj partial across ranks; on
 * one GPU `partial` is that sum already.
 *   v      = RMSNorm_H(partial) * post_attn_norm_w
 *   stream = fp32(stream + gate * v)                        in place, fp32 [b, H]
 *   out    = bf16(RMSNorm_H(stream) * pre_ffn_norm_w)       bf16 [b, H] (the block's x)
 * partial bf16 [b, H]; gate bf16 [H] (the attention add's gate); the norm
 * weights bf16 [H] or NULL (= 1), effective multipliers as in mb_weights;
 * epsilon dims->norm_eps.  Device pointers, 16-byte aligned; `out` must not
 * overlap `partial`.  Asynchronous on `stream_handle`; no workspace. */
int mb_attn_boundary(const mb_dims *dims, const uint16_t *partial, const uint16_t *post_attn_norm_w,
                     const uint16_t *gate, const uint16_t *pre_ffn_norm_w, float *stream, uint16_t *out,
                     void *stream_handle);

/* The next layer's QKV projection, the step after the block ([mono.decoder]
 * LayerWeights: w_qkvg, the next layer's qkv_proj weight, which the HB launch
 * applies to x_next after the FFN boundary; its rows are
 * MonoDims.qkvg_rows = 2 * q_rows + 2 * kv_rows: q, k, v and the o-gate):
 *   qkvg = bf16(x_next @ w_qkvg^T)                          bf16 [b, n_out]
 * x_next bf16 [b, H]; w_qkvg bf16 [n_out, H] row-major; n_out > 0 and a
 * multiple of 16 (else MB_ERR_DIMS / MB_ERR_UNSUPPORTED).  fp32 accumulation
 * split along H, the splits added in a fixed order; the split partials go to
 * the workspace.  With a workspace of mb_workspace_bytes for these dims with
 * qkv_rows = n_out (and act_quant 0), the projection runs as the block
 * kernel's projection step (the one mb_moe_block fuses after the boundary);
 * with one of mb_workspace_bytes(dims) only, as a split-K GEMM whose split is
 * capped so that its partials fit.  The QK norm, RoPE and KV insert of the
 * attention's QKV front are not part of this call. */
int mb_next_qkv(const mb_dims *dims, const uint16_t *x_next, const uint16_t *w_qkvg, int32_t n_out,
                uint16_t *qkvg, void *workspace, size_t workspace_bytes, void *stream);

/* The bf16 norm multiplier of a norm with a zero-centred gamma ([mono.decoder]
 * effective_norm_weight: the multiplier a norm applies is its weight, plus its
 * gain centre when the gamma is zero-centred):
 *   out[i] = bf16(fp32(weight[i] + gain_center))   (zero_centered != 0)
 *   out[i] = bf16(weight[i])                          (zero_centered == 0)
 * weight fp32 [n] (the norm's parameter, widened), out bf16 [n]; device
 * pointers.  Load-time preparation of the norm weights every entry point
 * takes (mb_weights' *_norm_w, the attention boundary's).  Asynchronous on
 * `stream`.  MB_ERR_DIMS if n <= 0 or gain_center is not finite. */
int mb_effective_norm_weight(const float *weight, int32_t n, float gain_center, int32_t zero_centered,
                             uint16_t *out, void *stream);

/* Whether a launch on this workspace gave up a wait since the workspace was
 * zero-filled or last reset.  The block kernel's workgroups hand work to one
 * another inside the launch, and every wait of one on another is bounded; a
 * wait that runs out (some workgroups never became resident together with the
 * others, say, because another kernel held compute units) makes the launch
 * drain without its results, and records it in the workspace.  Later
 * launches on the workspace compute as usual; the record stays until
 * mb_workspace_reset.  Enqueues on `stream` the write of MB_OK or
 * MB_ERR_ABORTED to *status (int32, device memory), readable once the stream
 * has reached it; allocates nothing, does not synchronise.  Returns MB_OK
 * (enqueued), MB_ERR_NULL, MB_ERR_ALIGN, MB_ERR_WORKSPACE (smaller than the
 * launch state every workspace starts with) or MB_ERR_HIP. */
int mb_workspace_status(const void *workspace, size_t workspace_bytes, int32_t *status, void *stream);

/* Clears the record mb_workspace_status reads (and nothing else: the
 * workspace stays ready for the next call).  Enqueued on `stream`; the same
 * returns as mb_workspace_status (no status argument). */
int mb_workspace_reset(void *workspace, size_t workspace_bytes, void *stream);

/* A static, human-readable reason for a status code. */
const char *mb_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MB_H */
