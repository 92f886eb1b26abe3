"""The routed-MoE block, step by step, on the CPU in numpy (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  The steps follow the order of the MoE block as the providers page
lists it ([providers] MoEProvider: router, routing, pooler, routed experts,
tail, unpooler) followed by the boundary ([providers] BoundaryProvider).

Readings where the pages leave a step open (each restated where it is used):

* top-k order: selection key descending, lowest expert id first among equal
  keys; a NaN key ranks below every number.
* the route-weight sum runs over the slots in slot order, in fp32.
* the router output multiplier scales the fp32 logits after the projection
  (as the native routing recipe does), not folded into the weights.
* scores are the correctly rounded fp32 value of the fp64 sigmoid / softmax.
* gated activation: silu(gate) * up with gate = w13 rows [0, I) and
  up = rows [I, 2I); its result is rounded to bf16 (MoE activations in bf16).
* expert outputs y and their norm stay in high precision; the MoE output is
  rounded to bf16 once, after the weighted sum over routes.
* every RMSNorm is x / sqrt(mean(x^2) + eps) * weight, the weight applied after
  normalising; an absent weight is 1.
* boundary: v = RMSNorm_H(u) * w_pff; stream <- fp32(stream + g * v);
  x_next = bf16(RMSNorm_H(stream) * w_in).
* MXFP4: E2M1 codes, two per byte, the even element in the low nibble; one
  E8M0 scale per 32 elements along the contraction dimension (OCP Microscaling
  Formats v1.0, sections 5.3.3 and 5.4.1).
* MXFP4 activations (the W4A4 variant; the pages leave the quantizer to their
  AITER backend): OCP Microscaling Formats v1.0, section 6.3 -- per block of 32
  along the contraction dimension, shared exponent floor(log2(amax)) - 2 (2 =
  E2M1's largest exponent) kept within E8M0's [-127, 127], each element divided
  by 2**shared_exp and rounded to the nearest E2M1 value, ties to the even
  mantissa, magnitudes above 6 saturating to 6; an all-zero block gets the
  smallest scale.  h and the gated activation are quantized from their bf16
  values (the same intermediates as the bf16 path).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F64 = np.float64
F32 = np.float32


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(F64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round values to the nearest bf16 (ties to even); uint16 bit patterns.

    bf16 has 8 significant bits and fp32's exponent range.  The value is
    written as m * 2**e with 0.5 <= |m| < 1, m is rounded to a multiple of
    2**-8 (numpy's rint rounds halves to even), and below the normal range the
    quantum is fixed at the subnormal step 2**-133.
    """
    v = np.asarray(v, dtype=F64)
    m, e = np.frexp(v)
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    tiny = np.abs(v) < 2.0 ** -126
    q = np.where(tiny, np.ldexp(np.rint(np.ldexp(v, 133)), -133), q)
    q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, v), q)
    bits = (q.astype(F32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), bits).astype(np.uint16)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """E2M1 nibble -> value (OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent bits with
    bias 1, 1 mantissa bit; exponent field 0 is subnormal, 0.5 * mantissa).
    Two codes per byte ([providers] ExpertsInput)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    ex = (c >> 1) & 3
    man = c & 1
    mag = np.where(ex == 0, 0.5 * man, np.ldexp(1.0 + 0.5 * man, ex - 1))
    return sign * mag


def decode_e8m0(s: np.ndarray) -> np.ndarray:
    """E8M0 scale byte -> 2**(s - 127); 0xFF is NaN (OCP MX v1.0, E8M0)."""
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[N, K/2] packed E2M1 + [N, K/32] E8M0 -> fp64 [N, K].

    Shapes follow [mono.decoder] MonoDims.expert_shapes: w13 is
    (E, 2I, P/2) with scales (E, 2I, P/32) and w2 is (E, P, I/2) with scales
    (E, P, I/32), i.e. row n of an expert matrix holds output feature n, and
    its contraction index runs along the packed bytes; one scale per 32."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, kh = codes.shape
    table = decode_e2m1(np.arange(16))  # the 16 code values, looked up per nibble
    vals = np.empty((n, 2 * kh), dtype=F64)
    vals[:, 0::2] = table[codes & 0x0F]
    vals[:, 1::2] = table[codes >> 4]
    return vals * np.repeat(decode_e8m0(scales), 32, axis=1)


E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def quantize_mxfp4(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp64 [..., K] (K a multiple of 32) -> E2M1 codes [..., K] (one per
    element, sign in bit 3) and E8M0 scale bytes [..., K/32], by the conversion
    of OCP Microscaling Formats v1.0, section 6.3 (see the module notes)."""
    v = np.asarray(v, dtype=F64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    _, e = np.frexp(amax)  # amax = m * 2**e, m in [0.5, 1): floor(log2(amax)) = e - 1
    shared = np.where(amax > 0, e - 1 - 2, -127)
    shared = np.clip(shared, -127, 127)
    x = blocks / np.ldexp(1.0, shared)[..., None]
    a = np.abs(x)
    # Nearest E2M1 magnitude, ties to the even mantissa (even index), saturating.
    idx = np.searchsorted(E2M1_MAGS, a, side="right") - 1  # largest magnitude <= a
    idx = np.clip(idx, 0, 7)
    lo = E2M1_MAGS[idx]
    hi = E2M1_MAGS[np.minimum(idx + 1, 7)]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & (idx % 2 == 1))
    q = np.where((idx < 7) & up, idx + 1, idx)
    codes = (q | np.where(x < 0, 8, 0)).astype(np.uint8)
    return codes.reshape(v.shape), (shared + 127).astype(np.uint8)


def fake_quant_mxfp4(v: np.ndarray) -> np.ndarray:
    """The values an MXFP4 quantization of v (along the last axis) stands for."""
    codes, scales = quantize_mxfp4(v)
    k = codes.shape[-1]
    return decode_e2m1(codes) * np.repeat(decode_e8m0(scales), 32, axis=-1).reshape(codes.shape[:-1] + (k,))


def rms_norm(v: np.ndarray, weight: Optional[np.ndarray], eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight over the last axis, in fp64.
    The weight is the effective bf16 multiplier ([mono.decoder]
    effective_norm_weight), applied after normalising; None means 1."""
    v = np.asarray(v, dtype=F64)
    out = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    if weight is not None:
        out = out * bf16_to_f64(weight)
    return out


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """fp32 router projection [b, H] x [E, H]^T -> [b, E] ([providers]
    MoEProvider: fp32 GateLinear; [mono.decoder] layer_refusals: router fp32
    [E, H]; the router reads the bf16 MoE input, [providers] RoutedMoE.build).
    The dot product is exact to fp64 and rounded once to fp32."""
    l = bf16_to_f64(x) @ np.asarray(router_w, dtype=F32).astype(F64).T
    return l.astype(F32)


def score(logits: np.ndarray, scoring: str, multiplier: Optional[float]) -> np.ndarray:
    """Optional output multiplier, then sigmoid or softmax over experts
    ([muse_moe_runner] MuseSpark1xRouter._compute_routing_native).  The
    multiplier is an fp32 product on the fp32 logits; the score is the fp32
    rounding of the fp64 function value."""
    g = np.asarray(logits, dtype=F32)
    if multiplier is not None:
        g = (g * F32(multiplier)).astype(F32)
    z = g.astype(F64)
    if scoring == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-z))
    elif scoring == "softmax":
        ez = np.exp(z - np.max(z, axis=-1, keepdims=True))
        s = ez / np.sum(ez, axis=-1, keepdims=True)
    else:
        raise ValueError(f"Invalid router_score_normalization: {scoring}")
    return s.astype(F32)


def select_topk(scores: np.ndarray, bias: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Selection key = fp32(score + bias), used for selection only
    ([muse_moe_runner] MuseSpark1xRouter: the bias is added for SELECTION and
    the UNBIASED scores are gathered).  Top-k by key descending, lowest id
    first among equal keys, NaN below all numbers; slot j holds rank j.
    Returns (ids int32 [b, k], keys fp32 [b, E])."""
    keys = (np.asarray(scores, dtype=F32) + np.asarray(bias, dtype=F32)).astype(F32)
    b, n = keys.shape
    ids = np.empty((b, k), dtype=np.int32)
    for t in range(b):
        row = keys[t]
        order = sorted(range(n), key=lambda e: (bool(np.isnan(row[e])),
                                                0.0 if np.isnan(row[e]) else -float(row[e]), e))
        ids[t] = order[:k]
    return ids, keys


def route_weights(scores: np.ndarray, ids: np.ndarray, route_scale: float,
                  division_eps: Optional[float]) -> np.ndarray:
    """Gather the unbiased scores of the chosen experts, divide by their sum
    (+ division eps) and scale by route_scale, all in fp32
    ([muse_moe_runner] MuseSpark1xRouter._compute_routing_native; the weights
    are fp32, [providers] RoutedTopk).  The sum runs over slots in slot order;
    the quotient is formed before the scaling."""
    b, k = ids.shape
    w = np.empty((b, k), dtype=F32)
    for t in range(b):
        g = [F32(scores[t, e]) for e in ids[t]]
        s = g[0]
        for j in range(1, k):
            s = F32(s + g[j])
        d = s if division_eps is None else F32(s + F32(division_eps))
        for j in range(k):
            w[t, j] = F32(F32(g[j] / d) * F32(route_scale))
    return w


def group_routes(ids: np.ndarray, experts: int) -> dict:
    """Route-sorted grouping of the routes r = t*k + j by expert.

    count[e] routes per expert; offset = exclusive prefix sum of count with
    offset[E] = b*k; route_list = the routes sorted by (expert, r); active =
    the experts with count > 0 in ascending order; n_active.  This is the
    per-expert row grouping the expert GEMMs consume ([muse_moe_runner]
    MuseSparkAiterExperts.apply hands the routes to the fused experts, which
    sort them by expert; [providers] RoutedMoE.run: the routing writes the
    experts' routing metadata)."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    count = np.zeros(experts, dtype=np.int32)
    for e in flat:
        count[e] += 1
    offset = np.zeros(experts + 1, dtype=np.int32)
    for e in range(experts):
        offset[e + 1] = offset[e] + count[e]
    route_list = np.array(sorted(range(flat.size), key=lambda r: (flat[r], r)), dtype=np.int32)
    active = np.array([e for e in range(experts) if count[e] > 0], dtype=np.int32)
    return {"count": count, "offset": offset, "route_list": route_list,
            "active": active, "n_active": np.int32(active.size)}


@dataclasses.dataclass
class Routing:
    logits: np.ndarray  # f32 [b, E] (before the multiplier)
    scores: np.ndarray  # f32 [b, E]
    keys: np.ndarray  # f32 [b, E]
    ids: np.ndarray  # i32 [b, k]
    weights: np.ndarray  # f32 [b, k]
    count: np.ndarray
    offset: np.ndarray
    route_list: np.ndarray
    active: np.ndarray
    n_active: int

    def margins(self) -> np.ndarray:
        """Per row: k-th largest key minus (k+1)-th largest key (inf if k = E)."""
        k = self.ids.shape[1]
        srt = -np.sort(-self.keys.astype(F64), axis=1)
        if k >= self.keys.shape[1]:
            return np.full(self.keys.shape[0], np.inf)
        return srt[:, k - 1] - srt[:, k]


def route_from_logits(logits, bias, k, scoring, multiplier, division_eps, route_scale) -> Routing:
    """Routing from given fp32 logits ([muse_moe_runner]
    MuseSpark1xRouter._compute_routing_native, plus the grouping)."""
    logits = np.asarray(logits, dtype=F32)
    s = score(logits, scoring, multiplier)
    ids, keys = select_topk(s, bias, k)
    w = route_weights(s, ids, route_scale, division_eps)
    g = group_routes(ids, logits.shape[1])
    return Routing(logits, s, keys, ids, w, g["count"], g["offset"], g["route_list"],
                   g["active"], int(g["n_active"]))


def route(inp) -> Routing:
    """Router projection then routing, on a synth.BlockInputs."""
    d = inp.dims
    l = router_logits(inp.x, inp.router_w)
    return route_from_logits(l, inp.expert_bias, d.top_k, d.scoring, d.multiplier,
                             d.division_eps, d.route_scale)


# --------------------------------------------------------------------------
# Pooler, experts, tail, unpooler, boundary
# --------------------------------------------------------------------------

def pool(x: np.ndarray, pool_w: np.ndarray, pre_norm_w: Optional[np.ndarray] = None,
         norm_eps: float = 1e-6) -> np.ndarray:
    """h = bf16(x @ Wp^T), Wp bf16 [P, H] ([mono.decoder] layer_refusals: pooler
    bf16 (P, H); [mono.decoder] _K5Bucket: h bf16 [rows, P]).  With a
    pre-expert norm weight, h = bf16(RMSNorm_P(h) * w) on the bf16 h
    ([providers] MoEProvider: pooler GEMM + pre_expert_norm)."""
    h = round_bf16(bf16_to_f64(x) @ bf16_to_f64(pool_w).T)
    if pre_norm_w is not None:
        h = round_bf16(rms_norm(bf16_to_f64(h), pre_norm_w, norm_eps))
    return h


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def experts(h: np.ndarray, ids: np.ndarray, weights: np.ndarray, w13, w13_scale, w2, w2_scale,
            post_norm_w: np.ndarray, norm_eps: float, want_routes: bool = False, act_quant: bool = False):
    """Per-route MXFP4 experts, per-route RMSNorm over P, weighted sum over routes.

    For route (t, j) with e = ids[t, j]:
      gu  = dec(w13[e]) @ h[t]                       (2I values)
      act = bf16(silu(gu[:I]) * gu[I:])              (I values)
      y   = dec(w2[e]) @ act                         (P values)
      yn  = RMSNorm_P(y) * w_post
    moe_out[t] = bf16(sum_j weights[t, j] * yn(t, j)), the sum in slot order.

    The experts return one unweighted output per route and the route weights
    are applied after the per-route norm ([muse_moe_runner]
    MuseSparkAiterExperts.apply and MuseSparkTopKWeightAndReduce.apply:
    norm, then multiply by the route weight, then sum over k, then cast).
    With act_quant (the W4A4 variant) the expert GEMMs take h and act as their
    MXFP4 quantizations (quantize_mxfp4, blocks of 32 along P and I).
    Returns moe_out (bf16 bits [b, P]) and, with want_routes, the per-route
    act [b, k, I] (bf16 bits) and y [b, k, P] (fp64)."""
    b, k = ids.shape
    hf = bf16_to_f64(h)
    if act_quant:
        hf = fake_quant_mxfp4(hf)
    I = w2.shape[2] * 2
    act = np.zeros((b, k, I), dtype=np.uint16)
    for e in sorted(set(int(v) for v in np.asarray(ids).reshape(-1))):
        sel = np.argwhere(np.asarray(ids) == e)  # (t, j) pairs
        W13 = dequant_mxfp4(w13[e], w13_scale[e])  # [2I, P]
        gu = hf[sel[:, 0]] @ W13.T  # [n, 2I]
        act[sel[:, 0], sel[:, 1]] = round_bf16(silu(gu[:, :I]) * gu[:, I:])
    moe_out, y = experts_down(act, ids, weights, w2, w2_scale, post_norm_w, norm_eps, act_quant)
    if want_routes:
        return moe_out, act, y
    return moe_out


def experts_down(act: np.ndarray, ids: np.ndarray, weights: np.ndarray, w2, w2_scale,
                 post_norm_w: np.ndarray, norm_eps: float, act_quant: bool = False):
    """The second half of `experts`, from the per-route act (bf16 bits
    [b, k, I]): y = dec(w2[e]) @ act (act as its MXFP4 quantization with
    act_quant), the per-route RMSNorm over P, the route weight, the sum over
    the k slots in slot order and the bf16 cast ([muse_moe_runner]
    MuseSparkAiterExperts.apply, MuseSparkTopKWeightAndReduce.apply).
    Returns (moe_out bf16 bits [b, P], y fp64 [b, k, P])."""
    b, k = ids.shape
    P = w2.shape[1]
    y = np.zeros((b, k, P), dtype=F64)
    for e in sorted(set(int(v) for v in np.asarray(ids).reshape(-1))):
        sel = np.argwhere(np.asarray(ids) == e)
        W2 = dequant_mxfp4(w2[e], w2_scale[e])  # [P, I]
        af = bf16_to_f64(act[sel[:, 0], sel[:, 1]])
        y[sel[:, 0], sel[:, 1]] = (fake_quant_mxfp4(af) if act_quant else af) @ W2.T
    yn = rms_norm(y, post_norm_w, norm_eps)
    acc = np.zeros((b, P), dtype=F64)
    for j in range(k):
        acc = acc + np.asarray(weights, dtype=F32).astype(F64)[:, j:j + 1] * yn[:, j]
    return round_bf16(acc), y


def unpool(moe_out: np.ndarray, unpool_w: np.ndarray) -> np.ndarray:
    """u = bf16(moe_out @ Wu^T), Wu bf16 [H, P] ([mono.decoder] layer_refusals:
    unpooler bf16 (H, P); [providers] MoEProvider: the unpooler GEMM, whose
    bf16 column block feeds the next boundary)."""
    return round_bf16(bf16_to_f64(moe_out) @ bf16_to_f64(unpool_w).T)


def boundary(u: np.ndarray, stream: np.ndarray, gate: np.ndarray, ffn_norm_w, next_norm_w,
             norm_eps: float):
    """The FFN boundary ([providers] BoundaryProvider: post_ffn_norm, the gated
    add into the fp32 stream in place, the next pre-norm into bf16 out).
    Returns (stream_new fp32 [b, H], x_next bf16 bits [b, H])."""
    v = rms_norm(bf16_to_f64(u), ffn_norm_w, norm_eps)
    s_new = (np.asarray(stream, dtype=F32).astype(F64) + bf16_to_f64(gate) * v).astype(F32)
    x_next = round_bf16(rms_norm(s_new.astype(F64), next_norm_w, norm_eps))
    return s_new, x_next


def attn_boundary(partial: np.ndarray, stream: np.ndarray, gate: np.ndarray, post_attn_norm_w,
                  pre_ffn_norm_w, norm_eps: float):
    """The attention boundary, the step before the block ([providers]
    AttentionBoundaryProvider: post_attn_norm of the attention's (all-reduced)
    o_proj partial, the gated add into the fp32 stream in place, pre_ffn_norm
    into the bf16 out, the block's x).  The same three operations as the FFN
    boundary, with the attention side's weights:
      v = RMSNorm_H(partial) * w_post_attn;  stream' = fp32(stream + g * v);
      out = bf16(RMSNorm_H(stream') * w_pre_ffn).
    Returns (stream' fp32 [b, H], out bf16 bits [b, H])."""
    v = rms_norm(bf16_to_f64(partial), post_attn_norm_w, norm_eps)
    s_new = (np.asarray(stream, dtype=F32).astype(F64) + bf16_to_f64(gate) * v).astype(F32)
    out = round_bf16(rms_norm(s_new.astype(F64), pre_ffn_norm_w, norm_eps))
    return s_new, out


def effective_norm_weight(weight: np.ndarray, gain_center: float, zero_centered: bool) -> np.ndarray:
    """The bf16 multiplier a norm applies ([mono.decoder] effective_norm_weight):
    the weight widened to fp32, plus the gain centre when the gamma is
    zero-centred (an fp32 addition), rounded to bf16.  Returns bf16 bits."""
    w = np.asarray(weight, dtype=F32)
    if zero_centered:
        w = (w + F32(gain_center)).astype(F32)
    return round_bf16(w.astype(F64))


def next_qkv(x_next: np.ndarray, w_qkvg: np.ndarray) -> np.ndarray:
    """The next layer's QKV (+ o-gate) projection on the block's x_next
    ([mono.decoder] LayerWeights: w_qkvg, the next layer's qkv_proj weight, bf16
    [qkvg_rows, H] with qkvg_rows = 2 q_rows + 2 kv_rows, applied after the FFN
    boundary): bf16(x_next @ w_qkvg^T), bf16 bits [b, qkvg_rows]."""
    return round_bf16(bf16_to_f64(x_next) @ bf16_to_f64(w_qkvg).T)


@dataclasses.dataclass
class BlockResult:
    routing: Routing
    h: np.ndarray  # bf16 bits [b, P]
    moe_out: np.ndarray  # bf16 bits [b, P]
    u: np.ndarray  # bf16 bits [b, H]
    stream: np.ndarray  # f32 [b, H] (updated)
    x_next: np.ndarray  # bf16 bits [b, H]
    act: Optional[np.ndarray] = None
    y: Optional[np.ndarray] = None


def block(inp, want_routes: bool = False, act_quant: bool = False) -> BlockResult:
    """The whole block on a synth.BlockInputs: routing and pooler (independent,
    [providers] RoutedMoE.run), experts and tail, unpooler, boundary
    (act_quant: the W4A4 experts)."""
    d = inp.dims
    r = route(inp)
    h = pool(inp.x, inp.pool_w, inp.pre_norm_w, d.norm_eps)
    ex = experts(h, r.ids, r.weights, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale,
                 inp.post_norm_w, d.norm_eps, want_routes=want_routes, act_quant=act_quant)
    moe_out, act, y = ex if want_routes else (ex, None, None)
    u = unpool(moe_out, inp.unpool_w)
    s_new, x_next = boundary(u, inp.stream, inp.gate, inp.ffn_norm_w, inp.next_norm_w, d.norm_eps)
    return BlockResult(r, h, moe_out, u, s_new, x_next, act, y)
