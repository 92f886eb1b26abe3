"""Pins of the oracle's MXFP4 activation quantizer (the W4A4 variant).

The conversion follows OCP Microscaling Formats v1.0, section 6.3: per block of
32, shared exponent floor(log2(amax)) - 2, elements rounded to the nearest E2M1
value with ties to the even mantissa, saturating at 6.  These tests check the
oracle against hand-worked blocks, against a brute-force nearest-value search
written independently of it, and against properties the rule fixes."""

import itertools

import numpy as np
import pytest

from oracle import steps as o

# E2M1 values by code (sign bit 3), written out from the format: 1 sign bit, 2
# exponent bits (bias 1), 1 mantissa bit, exponent 0 subnormal.
E2M1 = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def block(*vals):
    v = np.zeros(32)
    v[: len(vals)] = vals
    return v


def test_hand_worked_block_ties_and_saturation():
    # amax 7 -> floor(log2 7) = 2 -> shared exponent 0, scale byte 127.
    v = block(0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, 7, -0.25, -0.3, 0.26, 2.49, -5.01)
    codes, scales = o.quantize_mxfp4(v)
    assert scales.tolist() == [127]
    #            0  .25 .75 1.25 1.75 2.5 3.5 5  6  7  -.25 -.3 .26 2.49 -5.01
    assert codes[:15].tolist() == [0, 0, 2, 2, 4, 4, 6, 6, 7, 7, 8, 9, 1, 4, 15]


def test_scale_is_floor_log2_amax_minus_two():
    for amax, want in [(1.0, 125), (1.99, 125), (2.0, 126), (0.75, 124), (6.0, 127), (8.0, 128),
                       (2.0 ** -100, 127 - 102), (3 * 2.0 ** 60, 127 + 59)]:
        _, s = o.quantize_mxfp4(block(amax, -amax / 3))
        assert int(s[0]) == want, amax


def test_scale_clamps_to_e8m0_range_and_zero_block():
    _, s = o.quantize_mxfp4(block(2.0 ** -130))
    assert int(s[0]) == 0
    codes, s = o.quantize_mxfp4(np.zeros(32))
    assert int(s[0]) == 0 and not codes.any()


def brute(v):
    """Nearest E2M1 value times the block scale, ties to the even mantissa,
    found by trying every code (independent of the oracle's search)."""
    v = np.asarray(v, float)
    amax = np.max(np.abs(v))
    if amax == 0:
        return np.zeros_like(v)
    e = int(np.floor(np.log2(amax)))
    while 2.0 ** e > amax:
        e -= 1
    while 2.0 ** (e + 1) <= amax:
        e += 1
    x = 2.0 ** max(-127, min(127, e - 2))
    out = []
    for val in v:
        best = None
        for code, mag in E2M1.items():
            for sign in (1, -1):
                cand = sign * mag * x
                key = (abs(val - cand), code % 2)  # nearer first, then even mantissa
                if best is None or key < best[0]:
                    best = (key, cand)
        out.append(best[1])
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_matches_brute_force_nearest(seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((8, 64)) * np.exp2(rng.integers(-20, 20, (8, 1)))
    # Put exact midpoints and saturating values into some blocks.
    v[0, :8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9]) * 2.0 ** 3
    got = o.fake_quant_mxfp4(v)
    want = np.stack([np.concatenate([brute(r[:32]), brute(r[32:])]) for r in v])
    assert np.array_equal(np.abs(got), np.abs(want))
    assert np.array_equal(np.sign(got)[want != 0], np.sign(want)[want != 0])


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(3)
    mags = np.array(list(E2M1.values()))
    for s in (-20, 0, 7):
        v = rng.choice(mags, 32) * rng.choice([-1, 1], 32) * 2.0 ** s
        v[0] = 6.0 * 2.0 ** s  # amax 6 * 2**s keeps the shared exponent s
        assert np.array_equal(o.fake_quant_mxfp4(v), v)


def test_error_within_half_a_step():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((16, 32))
    q = o.fake_quant_mxfp4(v)
    for row, qr in zip(v, q):
        amax = np.max(np.abs(row))
        x = 2.0 ** (np.floor(np.log2(amax)) - 2)
        # Below 6x the step is at most 2x (between 4 and 6); saturation aside.
        sat = np.abs(row) > 6 * x
        assert np.all(np.abs(row - qr)[~sat] <= 1.0 * x + 1e-300)
        assert np.all(np.abs(qr[sat]) == 6 * x)


def test_w4a4_experts_match_a_direct_loop():
    """Tiny W4A4 experts against a loop over (route, output) with the brute-force
    quantizer: h and act quantized per 32 along the contraction."""
    rng = np.random.default_rng(5)
    E, P, I, b, k = 3, 64, 64, 2, 2
    w13 = rng.integers(0, 256, (E, 2 * I, P // 2), dtype=np.uint8)
    w13s = rng.integers(122, 130, (E, 2 * I, P // 32), dtype=np.uint8)
    w2 = rng.integers(0, 256, (E, P, I // 2), dtype=np.uint8)
    w2s = rng.integers(122, 130, (E, P, I // 32), dtype=np.uint8)
    h = o.round_bf16(rng.standard_normal((b, P)))
    ids = np.array([[0, 2], [2, 1]])
    wts = np.array([[0.7, 0.3], [0.5, 0.5]], np.float32)
    post = o.round_bf16(np.ones(P))
    got = o.experts(h, ids, wts, w13, w13s, w2, w2s, post, 1e-6, act_quant=True)
    hf = o.bf16_to_f64(h)
    want = np.zeros((b, P))
    for t in range(b):
        hq = np.concatenate([brute(hf[t, i:i + 32]) for i in range(0, P, 32)])
        for j in range(k):
            e = ids[t, j]
            W13 = o.dequant_mxfp4(w13[e], w13s[e])
            gu = W13 @ hq
            a = o.bf16_to_f64(o.round_bf16(gu[:I] / (1 + np.exp(-gu[:I])) * gu[I:]))
            aq = np.concatenate([brute(a[i:i + 32]) for i in range(0, I, 32)])
            y = o.dequant_mxfp4(w2[e], w2s[e]) @ aq
            yn = y / np.sqrt(np.mean(y * y) + 1e-6)
            want[t] += float(wts[t, j]) * yn
    assert np.array_equal(got, o.round_bf16(want))
