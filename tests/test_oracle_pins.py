"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests retypes an oracle formula: each checks a printed value, a
closed form worked out by hand on a constructed input, an invariant of the
method, or a brute-force answer on a tiny input.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import steps
from conftest import read_golden

F32 = np.float32


def bf16(v):
    return oracle.round_bf16(np.asarray(v, dtype=np.float64))


def f(bits):
    return oracle.bf16_to_f64(bits)


# ---------------------------------------------------------------- formats

def test_e2m1_table_matches_spec():
    rows = read_golden("e2m1_values.txt")
    codes = np.array([int(c, 16) for c, _ in rows])
    want = np.array([float(v) for _, v in rows])
    got = oracle.decode_e2m1(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # 0x8 is -0


def test_e8m0_values_match_spec():
    for byte, val in read_golden("e8m0_values.txt"):
        got = float(oracle.decode_e8m0(np.array([int(byte)]))[0])
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)


def test_mxfp4_nibble_order_and_block_scale():
    # Byte 0x21: low nibble 0x1 (0.5) is element 0, high nibble 0x2 (1.0) element 1.
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 16] = 0xF7  # elements 32, 33 in the second block: 6.0, -6.0
    scales = np.array([[127, 123]], dtype=np.uint8)  # block 0 x1, block 1 x2**-4
    v = oracle.dequant_mxfp4(codes, scales)
    assert v.shape == (1, 64)
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0
    assert v[0, 32] == 6.0 / 16 and v[0, 33] == -6.0 / 16
    assert np.count_nonzero(v) == 4


def test_mxfp4_all_codes_all_scales():
    for sbyte in (119, 120, 121, 122, 123, 127):
        codes = np.zeros((1, 16), dtype=np.uint8)
        for m in range(16):
            codes[0, m] = (m & 0xF) | (((15 - m) & 0xF) << 4)
        v = oracle.dequant_mxfp4(codes, np.array([[sbyte]], dtype=np.uint8))[0]
        table = {int(c, 16): float(x) for c, x in read_golden("e2m1_values.txt")}
        for m in range(16):
            assert v[2 * m] == table[m] * 2.0 ** (sbyte - 127)
            assert v[2 * m + 1] == table[15 - m] * 2.0 ** (sbyte - 127)
    nan = oracle.dequant_mxfp4(np.full((1, 16), 0x22, np.uint8), np.array([[255]], np.uint8))
    assert np.isnan(nan).all()


def test_bf16_rounding_hand_cases():
    for expr, bits in read_golden("bf16_rounding.txt"):
        v = eval(expr, {"__builtins__": {}})  # plain arithmetic on literals
        assert int(bf16(np.array([v]))[0]) == int(bits, 16), expr


def test_bf16_rounding_agrees_with_bit_trick_on_fp32():
    # synth's fp32 -> bf16 uses the integer round-half-even trick on the bit
    # pattern; the oracle rounds the real value.  They must agree on fp32 inputs.
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(F32)
    assert np.array_equal(bf16(a.astype(np.float64)), synth.f32_to_bf16_bits(a))


def test_bf16_of_bf16_is_identity():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(bf16(f(bits)), bits)
    assert np.array_equal(bf16(-f(bits)), bits | 0x8000)


def test_rmsnorm_constant_row_closed_form():
    c, eps = 0.75, 1e-6
    got = oracle.rms_norm(np.full((1, 8), c), None, eps)
    assert np.allclose(got, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    w = bf16(np.linspace(0.5, 1.5, 8))
    got = oracle.rms_norm(np.full((1, 8), c), w, eps)
    assert np.allclose(got, c / math.sqrt(c * c + eps) * f(w), rtol=1e-15, atol=0)


# ---------------------------------------------------------------- routing

def test_router_one_hot_gives_weight_column():
    rng = np.random.default_rng(1)
    E, H = 8, 64
    w = (rng.standard_normal((E, H)) * 0.02).astype(F32)
    for h in (0, 17, 63):
        x = np.zeros((1, H), np.uint16)
        x[0, h] = 0x3F80  # 1.0
        assert np.array_equal(oracle.router_logits(x, w)[0], w[:, h])
    x = np.zeros((1, H), np.uint16)
    x[0, 3] = 0xC000  # -2.0
    assert np.array_equal(oracle.router_logits(x, w)[0], -2 * w[:, 3])


def test_sigmoid_and_softmax_values():
    l = np.array([[0.0, 2.0, -1.0, 30.0, -30.0]], dtype=F32)
    s = oracle.score(l, "sigmoid", None)[0]
    assert s[0] == F32(0.5)
    assert s[1] == F32(1 / (1 + math.exp(-2.0)))
    assert s[3] == F32(1.0)  # saturated
    sm = oracle.score(l, "softmax", None)[0]
    den = sum(math.exp(v - 30.0) for v in l[0].astype(float))
    for i in range(5):
        assert sm[i] == F32(math.exp(float(l[0, i]) - 30.0) / den)
    # The multiplier scales the logits before scoring.
    m = oracle.score(l, "sigmoid", 1.5)[0]
    assert m[1] == F32(1 / (1 + math.exp(-3.0)))
    with pytest.raises(ValueError):
        oracle.score(l, "relu", None)


def _brute_topk(keys, k):
    """Expert e is chosen iff fewer than k experts beat it (key greater, or equal
    key with a lower id); slot order is the order of beating counts."""
    n = len(keys)
    beats = [sum(1 for o in range(n) if keys[o] > keys[e] or (keys[o] == keys[e] and o < e))
             for e in range(n)]
    return [e for r in range(k) for e in range(n) if beats[e] == r]


def test_topk_brute_force_exhaustive_small():
    # E = 8, k = 2, keys over all 3**8 patterns of three levels (many ties).
    import itertools
    levels = np.array([0.25, 0.5, 0.75], dtype=F32)
    pats = np.array(list(itertools.product(range(3), repeat=8)))
    scores = levels[pats]
    ids, keys = oracle.select_topk(scores, np.zeros(8, F32), 2)
    for t in range(0, len(pats), 1):
        assert list(ids[t]) == _brute_topk(list(keys[t]), 2)


def test_topk_brute_force_random_with_bias():
    rng = np.random.default_rng(2)
    for E, k in ((16, 4), (64, 8), (128, 8), (8, 8)):
        s = rng.integers(0, 6, size=(20, E)).astype(F32) / F32(8)
        bias = (rng.integers(-2, 3, size=E) / 16).astype(F32)
        ids, keys = oracle.select_topk(s, bias, k)
        for t in range(20):
            assert list(ids[t]) == _brute_topk(list(keys[t]), k)


def test_topk_nan_ranks_last():
    s = np.array([[np.nan, 0.1, np.nan, 0.2]], dtype=F32)
    ids, _ = oracle.select_topk(s, np.zeros(4, F32), 3)
    assert list(ids[0]) == [3, 1, 0]


def test_warm_up_pattern():
    rows = read_golden("warm_up_routing.txt")
    b, E, k = 2, 16, 4
    stride = E // (b * k)
    logits = np.full((b, E), -30.0, dtype=F32)
    for t in range(b):
        for j in range(k):
            logits[t, (t * k + j) * stride] = 30.0
    r = oracle.route_from_logits(logits, np.zeros(E, F32), k, "sigmoid", None, None, 2.5)
    for t, ids, ws in rows:
        t = int(t)
        assert list(r.ids[t]) == [int(v) for v in ids.split(",")]
        assert list(r.weights[t]) == [F32(v) for v in ws.split(",")]
    # With a division eps, each weight is fp32(fp32(1 / fp32(k + eps)) * scale).
    r = oracle.route_from_logits(logits, np.zeros(E, F32), k, "sigmoid", None, 1e-6, 2.5)
    d = F32(F32(4.0) + F32(1e-6))
    assert d > F32(4.0)
    assert (r.weights == F32(F32(F32(1.0) / d) * F32(2.5))).all()


def test_weight_sum_invariant():
    for name in ("c0",):
        inp = synth.make_block(name)
        r = oracle.route(inp)
        d = inp.dims
        S = np.array([sum(float(r.scores[t, e]) for e in r.ids[t]) for t in range(d.rows)])
        want = d.route_scale * S / (S + (d.division_eps or 0.0))
        assert np.allclose(r.weights.sum(1), want, rtol=8 * 2.0 ** -24, atol=0)
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 128)).astype(F32)
    r = oracle.route_from_logits(logits, np.zeros(128, F32), 8, "softmax", 1.5, 1e-6, 2.5)
    S = np.array([sum(float(r.scores[t, e]) for e in r.ids[t]) for t in range(50)])
    assert np.allclose(r.weights.sum(1), 2.5 * S / (S + 1e-6), rtol=8 * 2.0 ** -24, atol=0)


def test_softmax_all_experts_weights_are_scaled_scores():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((10, 8)).astype(F32)
    r = oracle.route_from_logits(logits, np.zeros(8, F32), 8, "softmax", None, 1e-6, 2.5)
    z = logits.astype(np.float64)
    sm = np.exp(z - z.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    got = np.take_along_axis(r.weights, np.argsort(r.ids, axis=1), axis=1)
    assert np.allclose(got, sm * 2.5 / (1 + 1e-6), rtol=1e-6, atol=0)


def test_bias_affects_selection_only():
    inp = synth.make_block("c0")
    r0 = oracle.route(inp)
    chosen = set(int(e) for e in r0.ids.reshape(-1))
    # Lowering the bias of experts nobody chose changes nothing.
    b1 = inp.expert_bias.copy()
    for e in range(inp.dims.experts):
        if e not in chosen:
            b1[e] -= F32(0.5)
    r1 = oracle.route_from_logits(r0.logits, b1, inp.dims.top_k, inp.dims.scoring,
                                  inp.dims.multiplier, inp.dims.division_eps, inp.dims.route_scale)
    assert np.array_equal(r1.ids, r0.ids) and np.array_equal(r1.weights, r0.weights)
    # A bias that reorders the choice changes ids, but every weight is still
    # computed from unbiased scores: same ids -> bitwise same weights.
    b2 = np.zeros_like(inp.expert_bias)
    b2[0] = 10.0  # expert 0 is now chosen first in every row
    r2 = oracle.route_from_logits(r0.logits, b2, inp.dims.top_k, inp.dims.scoring,
                                  inp.dims.multiplier, inp.dims.division_eps, inp.dims.route_scale)
    assert (r2.ids[:, 0] == 0).all()
    s = r0.scores
    for t in range(inp.dims.rows):
        g = [F32(s[t, e]) for e in r2.ids[t]]
        tot = g[0]
        for v in g[1:]:
            tot = F32(tot + v)
        tot = F32(tot + F32(inp.dims.division_eps))
        assert list(r2.weights[t]) == [F32(F32(v / tot) * F32(2.5)) for v in g]


def test_multiplier_is_applied_to_logits():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((12, 32)).astype(F32)
    bias = rng.uniform(-0.01, 0.01, 32).astype(F32)
    a = oracle.route_from_logits(l, bias, 4, "softmax", 1.5, 1e-6, 2.5)
    b = oracle.route_from_logits((l * F32(1.5)).astype(F32), bias, 4, "softmax", None, 1e-6, 2.5)
    assert np.array_equal(a.ids, b.ids) and np.array_equal(a.weights, b.weights)


def test_grouping_properties():
    rng = np.random.default_rng(7)
    for b, E, k in ((4, 8, 2), (16, 64, 4), (33, 128, 8), (1, 4, 4)):
        ids = np.array([rng.permutation(E)[:k] for _ in range(b)], dtype=np.int32)
        g = oracle.group_routes(ids, E)
        flat = ids.reshape(-1)
        assert g["offset"][0] == 0 and g["offset"][E] == b * k
        assert np.array_equal(np.diff(g["offset"]), g["count"])
        assert sorted(g["route_list"].tolist()) == list(range(b * k))
        for e in range(E):
            seg = g["route_list"][g["offset"][e]:g["offset"][e + 1]]
            assert (flat[seg] == e).all()
            assert list(seg) == sorted(seg)
        assert list(g["active"]) == sorted(set(flat.tolist()))
        assert g["n_active"] == len(set(flat.tolist()))


# ---------------------------------------------------------------- projections

def test_pool_and_unpool_one_hot():
    rng = np.random.default_rng(8)
    P, H = 32, 64
    wp = bf16(rng.standard_normal((P, H)) * 0.02)
    wu = bf16(rng.standard_normal((H, P)) * 0.02)
    x = np.zeros((2, H), np.uint16)
    x[0, 5] = 0x3F80
    x[1, 60] = 0x4000  # 2.0
    h = oracle.pool(x, wp)
    assert np.array_equal(h[0], wp[:, 5])
    assert np.array_equal(f(h[1]), 2 * f(wp[:, 60]))
    m = np.zeros((1, P), np.uint16)
    m[0, 31] = 0x3F80
    assert np.array_equal(oracle.unpool(m, wu)[0], wu[:, 31])


def test_pre_expert_norm_closed_form():
    H, P = 8, 4
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80
    wp = np.zeros((P, H), np.uint16)
    wp[:, 0] = bf16(np.array([0.5, -0.5, 0.5, -0.5]))  # h = +-0.5, mean square 0.25
    w = bf16(np.array([1.0, 2.0, 1.0, 0.5]))
    h = oracle.pool(x, wp, w, 1e-6)
    want = bf16(np.array([0.5, -1.0, 0.5, -0.25]) / math.sqrt(0.25 + 1e-6))
    assert np.array_equal(h[0], want)


# ---------------------------------------------------------------- experts

def _one_hot_experts():
    """Two experts whose every weight row has a single nonzero code, so each
    expert output element is a known function of one or two h elements."""
    P, I, E = 64, 32, 2
    w13 = np.zeros((E, 2 * I, P // 2), np.uint8)
    s13 = np.full((E, 2 * I, P // 32), 127, np.uint8)
    w2 = np.zeros((E, P, I // 2), np.uint8)
    s2 = np.full((E, P, I // 32), 127, np.uint8)
    col13 = lambda e, n: (5 * n + 3 * e) % P  # noqa: E731
    col2 = lambda e, p: (3 * p + e) % I  # noqa: E731
    for e in range(E):
        for n in range(2 * I):
            c = col13(e, n)
            w13[e, n, c // 2] |= (0x2 << (4 * (c % 2)))  # +1.0
            s13[e, n, c // 32] = 127 + (n % 2)  # x1 or x2
        for p in range(P):
            c = col2(e, p)
            w2[e, p, c // 2] |= (0x5 << (4 * (c % 2)))  # +3.0
            s2[e, p, c // 32] = 126 + (p % 3)  # x0.5, x1, x2
    return P, I, E, w13, s13, w2, s2, col13, col2


def _check_experts_closed_form():
    P, I, E, w13, s13, w2, s2, col13, col2 = _one_hot_experts()
    b = 3
    hv = np.array([[((p * 7 + t * 3) % 16 - 8) / 8.0 for p in range(P)] for t in range(b)])
    h = bf16(hv)
    ids = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    w = np.array([[0.75, 1.75], [2.0, 0.5], [1.25, 1.25]], dtype=F32)
    post = bf16(np.array([1.0 + 0.01 * (p % 5) for p in range(P)]))
    eps = 1e-6
    got = oracle.experts(h, ids, w, w13, s13, w2, s2, post, eps)
    want = np.zeros((b, P))
    for t in range(b):
        acc = [0.0] * P
        for j in range(2):
            e = int(ids[t, j])
            gu = [f(h[t, col13(e, n)]) * (2.0 ** (n % 2)) for n in range(2 * I)]
            act = []
            for i in range(I):
                g_, u_ = float(gu[i]), float(gu[I + i])
                act.append(float(f(bf16(np.array([g_ / (1 + math.exp(-g_)) * u_])))[0]))
            y = [3.0 * 2.0 ** (p % 3 - 1) * act[col2(e, p)] for p in range(P)]
            ms = sum(v * v for v in y) / P
            for p in range(P):
                acc[p] += float(w[t, j]) * (y[p] / math.sqrt(ms + eps) * float(f(post[p])))
        want[t] = acc
    assert np.array_equal(got, bf16(want))


def test_experts_closed_form_one_hot_weights():
    _check_experts_closed_form()


def test_planted_mistake_fails_the_closed_form(monkeypatch):
    # A dropped sigmoid in the gated activation must not pass the pin.
    monkeypatch.setattr(steps, "silu", lambda z: z)
    with pytest.raises(AssertionError):
        _check_experts_closed_form()


def test_planted_dropped_norm_weight_fails(monkeypatch):
    real = steps.rms_norm
    monkeypatch.setattr(steps, "rms_norm", lambda v, w, eps: real(v, None, eps))
    with pytest.raises(AssertionError):
        _check_experts_closed_form()


def _c0_moe(inp, **over):
    # norm eps 0: doubling y then leaves the per-route norm exactly unchanged
    # (power-of-two scaling commutes with rounding, mean and square root).
    r = oracle.route(inp)
    h = oracle.pool(inp.x, inp.pool_w)
    args = dict(w13=inp.w13, w13_scale=inp.w13_scale, w2=inp.w2, w2_scale=inp.w2_scale)
    args.update(over)
    return oracle.experts(h, r.ids, r.weights, post_norm_w=inp.post_norm_w,
                          norm_eps=0.0, **args)


def _ulps(a, b):
    return np.abs(a.astype(np.int64) - b.astype(np.int64))


def test_norm_after_w2_scale_invariance():
    inp = synth.make_block("c0")
    base = _c0_moe(inp)
    # Doubling every w2 (E8M0 + 1) doubles y; the per-route norm removes it.
    assert np.array_equal(_c0_moe(inp, w2_scale=inp.w2_scale + 1), base)
    # Doubling the up half of w13 doubles act exactly, hence y: no change.
    I = inp.dims.inter
    s = inp.w13_scale.copy()
    s[:, I:, :] += 1
    assert np.array_equal(_c0_moe(inp, w13_scale=s), base)
    # Doubling the gate half goes through silu: the output must change.
    s = inp.w13_scale.copy()
    s[:, :I, :] += 1
    assert (_c0_moe(inp, w13_scale=s) != base).mean() > 0.5


def test_identical_experts_routing_invariance():
    inp = synth.make_block("c0")
    E = inp.dims.experts
    same = dict(w13=np.repeat(inp.w13[:1], E, 0), w13_scale=np.repeat(inp.w13_scale[:1], E, 0),
                w2=np.repeat(inp.w2[:1], E, 0), w2_scale=np.repeat(inp.w2_scale[:1], E, 0))
    h = oracle.pool(inp.x, inp.pool_w)
    r = oracle.route(inp)
    a = oracle.experts(h, r.ids, r.weights, post_norm_w=inp.post_norm_w, norm_eps=1e-6, **same)
    # Every route of a row now gives the same yn: the weighted sum equals one
    # route carrying the summed weight, whichever expert ids were chosen.
    wsum = r.weights.astype(np.float64).sum(1, keepdims=True).astype(F32)
    other = np.full((inp.dims.rows, 1), E - 1, np.int32)
    b = oracle.experts(h, other, wsum, post_norm_w=inp.post_norm_w, norm_eps=1e-6, **same)
    assert _ulps(a, b).max() <= 1


def test_top1_is_weighted_normed_route():
    inp = synth.make_block("c0")
    h = oracle.pool(inp.x, inp.pool_w)
    ids = np.array([[3], [3], [5], [0]], np.int32)
    one = np.ones((4, 1), F32)
    half = np.full((4, 1), 0.5, F32)
    a = oracle.experts(h, ids, one, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, inp.post_norm_w, 1e-6)
    b = oracle.experts(h, ids, half, inp.w13, inp.w13_scale, inp.w2, inp.w2_scale, inp.post_norm_w, 1e-6)
    assert np.array_equal(f(b), f(a) / 2)  # halving a bf16 value is exact


# ---------------------------------------------------------------- boundary

def test_boundary_zero_gate_leaves_stream():
    rng = np.random.default_rng(9)
    u = bf16(rng.standard_normal((3, 16)))
    s = rng.standard_normal((3, 16)).astype(F32)
    s_new, _ = oracle.boundary(u, s, np.zeros(16, np.uint16), None, None, 1e-6)
    assert np.array_equal(s_new, s)


def test_boundary_constant_rows_closed_form():
    H, eps = 8, 1e-6
    c = 0.75
    u = bf16(np.full((1, H), c))
    s = np.array([[0.5, -1.0, 2.0, 0.0, 1.5, -0.25, 3.0, -2.0]], dtype=F32)
    g = bf16(np.array([0.5, 0.25, 1.0, 0.5, 0.125, 2.0, 0.5, 0.75]))
    s_new, xn = oracle.boundary(u, s, g, None, None, eps)
    v = c / math.sqrt(c * c + eps)
    want_s = [F32(float(s[0, i]) + float(f(g[i])) * v) for i in range(H)]
    assert list(s_new[0]) == want_s
    ms = sum(float(x) ** 2 for x in want_s) / H
    want_x = bf16(np.array([float(x) / math.sqrt(ms + eps) for x in want_s]))
    assert np.array_equal(xn[0], want_x)


# ------------------------------------------- steps either side of the block

def test_attn_boundary_closed_forms():
    """A zero gate leaves the stream unchanged; a constant partial row normalises
    to 1 (times the post-attention norm weight) and adds g * w there; the out
    row is the stream row over its root mean square, times the pre-FFN weight."""
    H, eps = 8, 1e-6
    rng = np.random.default_rng(21)
    s = rng.standard_normal((2, H)).astype(F32)
    part = bf16(rng.standard_normal((2, H)))
    s0, _ = oracle.attn_boundary(part, s, np.zeros(H, np.uint16), None, None, eps)
    assert np.array_equal(s0, s)
    c = -1.5
    part = bf16(np.full((1, H), c))
    g = bf16(np.array([0.5, 0.25, 1.0, 0.5, 0.125, 2.0, 0.5, 0.75]))
    wa = bf16(np.array([1.0, 2.0, 0.5, 1.0, 1.0, 0.25, 1.0, 4.0]))
    wf = bf16(np.array([2.0, 1.0, 1.0, 0.5, 1.0, 1.0, 0.25, 1.0]))
    s1 = s[:1]
    s_new, out = oracle.attn_boundary(part, s1, g, wa, wf, eps)
    v = c / math.sqrt(c * c + eps)
    want_s = [F32(float(s1[0, i]) + float(f(g[i])) * v * float(f(wa[i]))) for i in range(H)]
    assert list(s_new[0]) == want_s
    ms = sum(float(x) ** 2 for x in want_s) / H
    want_o = bf16(np.array([float(x) / math.sqrt(ms + eps) * float(f(wf[i])) for i, x in enumerate(want_s)]))
    assert np.array_equal(out[0], want_o)


def test_effective_norm_weight_hand_cases():
    w = np.array([0.0, -1.0, 0.25, 2.0 ** -9, 2.0 ** -8, 3 * 2.0 ** -8, 0.5], np.float32)
    got = oracle.effective_norm_weight(w, 1.0, True)
    # 1, 0, 1.25, 1 + 2^-9 -> 1.0 (below half an ulp), 1 + 2^-8 -> 1.0 (tie, even),
    # 1 + 3 * 2^-8 -> 1 + 2^-6 (tie, even), 1.5
    assert got.tolist() == [0x3F80, 0x0000, 0x3FA0, 0x3F80, 0x3F80, 0x3F82, 0x3FC0]
    assert oracle.effective_norm_weight(w[[2, 6]], 1.0, False).tolist() == [0x3E80, 0x3F00]
    # The gain centre is added in fp32 before the bf16 rounding.
    assert oracle.effective_norm_weight(np.array([1e-8], np.float32), 1.0, True).tolist() == [0x3F80]


def test_next_qkv_one_hot_and_linearity():
    rng = np.random.default_rng(22)
    H, N = 64, 48
    w = bf16(rng.standard_normal((N, H)) * 0.02)
    x = np.zeros((2, H), np.uint16)
    x[0, 7] = 0x3F80  # 1.0: the projection is column 7 of w exactly
    x[1, 7] = 0x3F80
    x[1, 40] = 0xBF80  # -1.0
    q = oracle.next_qkv(x, w)
    assert q.shape == (2, N)
    assert np.array_equal(q[0], w[:, 7])
    assert np.array_equal(q[1], bf16(f(w[:, 7]) - f(w[:, 40])))


# ---------------------------------------------------------------- whole block

def test_rows_are_independent():
    inp = synth.make_block("c0")
    full = oracle.block(inp)
    part = oracle.block(inp.rows(2))
    for name in ("h", "moe_out", "u", "stream", "x_next"):
        assert np.array_equal(getattr(part, name), getattr(full, name)[:2]), name
    assert np.array_equal(part.routing.ids, full.routing.ids[:2])
    assert np.array_equal(part.routing.weights, full.routing.weights[:2])


def test_c0_block_shapes_and_finite():
    inp = synth.make_block("c0", norm_weights=True)
    r = oracle.block(inp)
    d = inp.dims
    assert r.routing.ids.shape == (d.rows, d.top_k)
    assert r.h.shape == (d.rows, d.pooled) and r.moe_out.shape == (d.rows, d.pooled)
    assert r.u.shape == (d.rows, d.hidden) and r.x_next.shape == (d.rows, d.hidden)
    assert np.isfinite(r.stream).all() and np.isfinite(f(r.x_next)).all()
