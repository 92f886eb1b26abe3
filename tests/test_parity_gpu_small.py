"""GPU parity of the HIP path against the oracle: small workloads and edge cases.

Every test calls the library through its C ABI (the ctypes binding) and
compares element by element with the oracle on the same seeded inputs:
bit-exact routing (ids, grouping) and fp32 logits, route weights within 1e-5
relative, bf16 outputs and the fp32 stream within 1e-2 absolute + 2e-2
relative."""

import dataclasses

import numpy as np
import pytest

import oracle
import synth
from parity import GpuBlock, assert_block, assert_close, assert_routing, say
from conftest import read_golden

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def small(rows=4, hidden=256, pooled=128, inter=256, experts=8, top_k=2, scoring="sigmoid",
          multiplier=None, eps=1e-20, route_scale=2.5):
    return synth.Dims(rows, hidden, pooled, inter, experts, top_k, scoring, route_scale,
                      multiplier, eps)


def run_and_check(blk, name):
    say(f"[gpu] block {name} dims={blk.dims}")
    g = GpuBlock(blk)
    got = g.run_block()
    ref = oracle.block(blk)
    return assert_block(got, ref, name, blk)


def test_c0_block():
    run_and_check(synth.make_block("c0"), "c0")


def test_c0_block_with_all_norm_weights():
    run_and_check(synth.make_block("c0", norm_weights=True), "c0+norms")


def test_c0_stages_teacher_forced():
    blk = synth.make_block("c0", norm_weights=True)
    g = GpuBlock(blk)
    ref = oracle.block(blk)
    say("[gpu] c0 stages: route")
    assert_routing(g.run_route(), ref.routing, "c0 route")
    say("[gpu] c0 stages: route from logits")
    assert_routing(g.run_route(logits_in=ref.routing.logits), ref.routing, "c0 route(logits)")
    say("[gpu] c0 stages: pool")
    assert_close(g.run_pool(), ref.h, "c0 pool")
    say("[gpu] c0 stages: experts")
    assert_close(g.run_experts(ref.h, ref.routing), ref.moe_out, "c0 experts")
    say("[gpu] c0 stages: unpool+boundary")
    got = g.run_unpool_boundary(ref.moe_out)
    assert_close(got["u"], ref.u, "c0 u")
    assert_close(got["stream"], ref.stream, "c0 stream", is_bf16=False)
    assert_close(got["x_next"], ref.x_next, "c0 x_next")


@pytest.mark.parametrize("rows", [1, 2, 5, 13, 16, 17, 33, 100, 256])
def test_ragged_rows(rows):
    run_and_check(synth.make_block("c0", seed=100 + rows, dims=small(rows=rows)), f"rows={rows}")


@pytest.mark.parametrize("case", [
    dict(top_k=8, scoring="softmax", multiplier=1.5, eps=1e-6),  # k = E
    dict(top_k=1),
    dict(experts=100, top_k=7, scoring="softmax"),  # E not a multiple of the wave
    dict(experts=1, top_k=1),
    dict(experts=1024, top_k=16, rows=4, inter=128),  # largest expert count and top-k
    dict(rows=1024, inter=128),  # largest row count
    dict(hidden=96, pooled=384, inter=384, rows=21),  # odd multiples of the tile sizes
    dict(hidden=4096, pooled=2048, inter=1024, experts=64, top_k=4, rows=3),
    # fp64-MFMA router tiles: contraction split 8 ways; and one split (more
    # tiles than half the grid), rows and experts past whole tiles.
    dict(rows=64, experts=64, hidden=512, top_k=4),
    dict(rows=500, experts=136, top_k=2, inter=128),
])
def test_shape_edges(case):
    d = small(**case)
    run_and_check(synth.make_block("c0", seed=7, dims=d), f"edge {case}")


@pytest.mark.parametrize("case", [dict(rows=65), dict(rows=256),
                                  dict(rows=64, experts=64, hidden=512, top_k=4)])
def test_many_rows_with_norm_weights(case):
    """The block kernel's many-rows instance (beyond 64 rows, or the fp64-MFMA
    router from 64), where the expert units stage plain h and act behind
    counters; with every norm weight, so the pre-norm rows make h."""
    d = small(**case)
    run_and_check(synth.make_block("c0", seed=80 + case["rows"], dims=d, norm_weights=True), f"many rows+norms {case}")


def test_many_rows_experts_in_passes():
    """mb_experts from the oracle's h and routing at 200 rows over 8 experts:
    the many-rows instance with the caller's routing, where every expert's
    rows go to units in passes of 32 (several per expert here)."""
    d = small(rows=200, experts=8, top_k=2)
    blk = synth.make_block("c0", seed=90, dims=d)
    ref = oracle.block(blk)
    assert ref.routing.count.max() > 64
    g = GpuBlock(blk)
    say("[gpu] many-rows experts in passes")
    assert_close(g.run_experts(ref.h, ref.routing), ref.moe_out, "many-rows experts")


@pytest.mark.parametrize("rows", [13, 70])
def test_per_step_kernels_with_norm_weights(rows):
    """More experts than the block kernel takes (300 > 256): mb_moe_block runs
    the per-step kernels (router and routing, pooler and its row norm,
    experts, unpooler and boundary), here with every norm weight."""
    d = small(rows=rows, experts=300, top_k=6, inter=384, scoring="softmax", multiplier=1.5, eps=1e-6)
    run_and_check(synth.make_block("c0", seed=60 + rows, dims=d, norm_weights=True), f"per-step E=300 rows={rows}")


def test_per_step_kernels_wider():
    """The per-step kernels at a wider shape than the test above: 320 experts
    (more than the block kernel takes), H 2048, P 512, I 256, top-8 of
    sigmoid scores, 24 rows, with every norm weight, so that the pooler's
    row norm, the expert kernels and the boundary run over many tiles."""
    d = small(rows=24, hidden=2048, pooled=512, inter=256, experts=320, top_k=8, eps=1e-6)
    run_and_check(synth.make_block("c0", seed=71, dims=d, norm_weights=True), "per-step E=320 H=2048")


def test_warm_up_saturated_logits():
    rows = read_golden("warm_up_routing.txt")
    d = small(rows=2, experts=16, top_k=4, eps=None)
    blk = synth.make_block("c0", seed=3, dims=d)
    blk.expert_bias = np.zeros(16, np.float32)
    logits = np.full((2, 16), -30.0, np.float32)
    for t in range(2):
        for j in range(4):
            logits[t, (t * 4 + j) * 2] = 30.0
    g = GpuBlock(blk)
    say("[gpu] warm-up pattern via MB_LOGITS_IN")
    got = g.run_route(logits_in=logits)
    for t, ids, ws in rows:
        t = int(t)
        assert list(got["topk_ids"][t]) == [int(v) for v in ids.split(",")]
        assert list(got["topk_w"][t]) == [np.float32(v) for v in ws.split(",")]


def test_exact_ties_go_to_lowest_id():
    d = small(rows=6, experts=16, top_k=3)
    blk = synth.make_block("c0", seed=5, dims=d)
    w = blk.router_w
    w[9] = w[2]
    w[12] = w[2]
    w[7] = w[4]
    blk.expert_bias = np.zeros(16, np.float32)
    blk.expert_bias[[2, 9, 12]] = 2.0  # the three copies always win, in id order
    g = GpuBlock(blk)
    say("[gpu] exact ties")
    got = g.run_route()
    ref = oracle.route(blk)
    assert (ref.ids == np.array([2, 9, 12])).all()
    assert_routing(got, ref, "ties")


@pytest.mark.parametrize("experts", [16, 128])
def test_block_exact_ties_go_to_lowest_id(experts):
    """The fused block's own routing (one wave per row: 32-bit order values,
    the lowest id among equal ones) on exact ties: copies of one router row,
    biased to win, go out in id order.  With 128 experts a lane holds experts
    e and e + 64, and the copies sit in both halves."""
    d = small(rows=6, experts=experts, top_k=3)
    blk = synth.make_block("c0", seed=5, dims=d)
    a, b, c = (2, 9, 12) if experts == 16 else (66, 2, 73)
    w = blk.router_w
    w[b] = w[a]
    w[c] = w[a]
    blk.expert_bias = np.zeros(experts, np.float32)
    blk.expert_bias[[a, b, c]] = 2.0
    ref = oracle.block(blk)
    assert (ref.routing.ids == np.array(sorted([a, b, c]))).all()
    g = GpuBlock(blk)
    say(f"[gpu] block exact ties E={experts}")
    got = g.run_block()
    assert_block(got, ref, f"block ties E={experts}", blk)


def test_block_is_deterministic():
    blk = synth.make_block("c0", seed=11, dims=small(rows=37, experts=16, top_k=4))
    g = GpuBlock(blk)
    say("[gpu] determinism")
    a = g.run_block()
    b = g.run_block()
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), n


def test_binding_raises_on_unsupported_dims():
    import routed_expert_layer_amd as rel
    blk = synth.make_block("c0")
    g = GpuBlock(blk)
    bad = dataclasses.replace(blk.dims, pooled=96)
    from synth.device import dims_kwargs
    d = rel.make_dims(**dims_kwargs(bad))
    h = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rel.MbError) as ei:
        rel.mb_pool(d, g.x, g.weights, h, g.ws)
    assert ei.value.status == rel.MB_ERR_UNSUPPORTED


# ---------------------------------------------------------------- streaming layout

def packed_reference(blk) -> np.ndarray:
    """The streaming layout that mb_pack_experts documents, built on the host
    from the caller-layout weights (test code: index arithmetic only)."""
    d = blk.dims
    P, I, E = d.pooled, d.inter, d.experts

    def codes(w, units, nch, unit_rows, t1_row):
        u, c, t, l = np.meshgrid(np.arange(units), np.arange(nch), np.arange(2), np.arange(64), indexing="ij")
        row = unit_rows * u + t * t1_row + (l & 15)
        col = 64 * c + 16 * (l >> 4)
        idx = col[..., None] + np.arange(16)
        return w[:, row[..., None], idx].reshape(E, -1)

    def scales(s, units, ngr, unit_rows, t1_row):
        rb = s.shape[2]
        pad = np.full((E, s.shape[1], ngr * 16), 127, np.uint8)
        pad[:, :, :rb] = s
        u, g, t, l = np.meshgrid(np.arange(units), np.arange(ngr), np.arange(2), np.arange(64), indexing="ij")
        row = unit_rows * u + t * t1_row + (l & 15)
        idx = 4 * (4 * g[..., None] + np.arange(4)) + (l >> 4)[..., None]
        return pad[:, row[..., None], idx].reshape(E, -1)

    nch_p, nch_i = P // 128, I // 128
    parts = [codes(blk.w13, I // 16, nch_p, 16, I), scales(blk.w13_scale, I // 16, (nch_p + 3) // 4, 16, I),
             codes(blk.w2, P // 32, nch_i, 32, 16), scales(blk.w2_scale, P // 32, (nch_i + 3) // 4, 32, 16)]
    return np.concatenate(parts, axis=1).reshape(-1)


def packed_matrix_reference(m):
    """mb_pack_projections' layout of one bf16 matrix [n_out, kdim] (bit
    patterns), as mb.h documents it: per 16-row tile t (rows past n_out zero)
    and 32-element chunk c, lane l's 8 elements 32 c + 8 (l / 16) .. + 7 of
    row 16 t + l % 16, lanes in order."""
    n_out, kdim = m.shape
    tiles = (n_out + 15) // 16
    pad = np.zeros((tiles * 16, kdim), np.uint16)
    pad[:n_out] = m
    # [t, r, c, g, j] -> [t, c, g, r, j]: lane l = 16 g + r.
    return pad.reshape(tiles, 16, kdim // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1).view(np.uint8)


def packed_projections_reference(blk):
    pool = packed_matrix_reference(blk.pool_w)
    unpool = packed_matrix_reference(blk.unpool_w)
    gap = np.zeros((-len(pool)) % 256, np.uint8)
    return np.concatenate([pool, gap, unpool])


@pytest.mark.parametrize("dims", [dict(), dict(hidden=96, pooled=640, inter=384, experts=5),
                                  dict(pooled=2048, inter=1024, experts=3)])
def test_packed_layout_is_the_documented_one(dims):
    blk = synth.make_block("c0", seed=21, dims=small(**dims))
    g = GpuBlock(blk)
    say(f"[gpu] pack experts and projections {blk.dims}")
    packed = g.use_packed().cpu().numpy()
    want = packed_reference(blk)
    assert packed.shape == want.shape
    assert np.array_equal(packed, want)
    proj = g.proj_packed.cpu().numpy()
    want = packed_projections_reference(blk)
    assert proj.shape == want.shape
    assert np.array_equal(proj, want)


@pytest.mark.parametrize("case", [dict(), dict(rows=17), dict(rows=100, experts=16, top_k=4),
                                  dict(hidden=96, pooled=640, inter=384, rows=21),
                                  dict(hidden=4096, pooled=2048, inter=1024, experts=64, top_k=4, rows=16)])
def test_packed_experts_match_caller_layout(case):
    """Experts and projections in the streaming layouts: same values, same
    arithmetic order, so every output is bit-identical to the caller-layout
    run, and both match the oracle."""
    blk = synth.make_block("c0", seed=31, dims=small(**case))
    g = GpuBlock(blk)
    say(f"[gpu] packed vs caller layout {case}")
    plain = g.run_block()
    g.use_packed()
    packed = g.run_block()
    for n in plain:
        assert np.array_equal(plain[n], packed[n], equal_nan=True), n
    assert_block(packed, oracle.block(blk), f"packed {case}", blk)


def test_packed_only_refused_where_the_block_kernel_declines():
    import routed_expert_layer_amd as rel
    blk = synth.make_block("c0", seed=41, dims=small(rows=3, experts=300, top_k=2, inter=128))
    g = GpuBlock(blk)
    g.use_packed()
    with pytest.raises(rel.MbError) as e:
        g.run_block()
    assert e.value.status == rel.MB_ERR_UNSUPPORTED
