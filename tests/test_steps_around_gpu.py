"""GPU parity of the steps either side of the block: the attention boundary
(mb_attn_boundary) that produces the block's input x, and the next layer's
QKV + o-gate projection (mb_next_qkv) of the block's x_next; then the three
chained as one layer's FFN half (teacher-forced stage by stage).

The QKV shape is synthetic: 32 query heads and 8 KV heads of 128, so
qkvg_rows = 2 * 4096 + 2 * 1024 = 10240 at H = 4096."""

import pytest

import oracle
import routed_expert_layer_amd as rel
import synth
from parity import BF16, GpuBlock, assert_block, assert_close, say
from synth.device import bits, dims_kwargs, to_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

QKVG_C1 = 10240


def _dims(rows, hidden, pooled=2048):
    return rel.make_dims(rows=rows, hidden=hidden, pooled=pooled, inter=1024, experts=64, top_k=4,
                         scoring="sigmoid", route_scale=2.5)


def _dims_q(rows, hidden, n_out):
    return rel.make_dims(rows=rows, hidden=hidden, pooled=2048, inter=1024, experts=64, top_k=4,
                         scoring="sigmoid", route_scale=2.5, qkv_rows=n_out)


def _attn(rows, hidden, seed, norm_weights=True):
    a = synth.make_attn_side(rows, hidden, 16, seed, norm_weights)
    say(f"[gpu] attention boundary rows {rows} H {hidden} norms {norm_weights}")
    d = _dims(rows, hidden)
    stream = to_tensor(a["stream"])
    out = torch.zeros((rows, hidden), dtype=BF16, device="cuda")
    t = {k: (None if a[k] is None else to_tensor(a[k])) for k in ("partial", "gate", "post_attn_norm_w",
                                                                  "pre_ffn_norm_w")}
    rel.mb_attn_boundary(d, t["partial"], t["gate"], stream, out, t["post_attn_norm_w"], t["pre_ffn_norm_w"])
    torch.cuda.synchronize()
    s_ref, o_ref = oracle.attn_boundary(a["partial"], a["stream"], a["gate"], a["post_attn_norm_w"],
                                        a["pre_ffn_norm_w"], 1e-6)
    assert_close(stream.cpu().numpy(), s_ref, "stream", atol=1e-5, rtol=1e-5, is_bf16=False)
    assert_close(bits(out), o_ref, "out")


@pytest.mark.parametrize("rows,hidden,norms", [(16, 4096, True), (37, 4096, False), (1, 7168, True),
                                               (64, 7168, True), (3, 12288, True)])
def test_attn_boundary(rows, hidden, norms):
    _attn(rows, hidden, 50 + rows, norms)


@pytest.mark.parametrize("persistent", [False, True])
@pytest.mark.parametrize("rows,hidden,n_out", [(16, 4096, QKVG_C1), (37, 4096, 1040), (1, 4096, 16),
                                               (64, 7168, 2048)])
def test_next_qkv(rows, hidden, n_out, persistent):
    a = synth.make_attn_side(rows, hidden, n_out, 60 + rows)
    say(f"[gpu] next qkv rows {rows} H {hidden} n_out {n_out} persistent {persistent}")
    d = _dims(rows, hidden)
    # A workspace sized with qkv_rows = n_out selects the block kernel's projection step.
    ws = rel.workspace(_dims_q(rows, hidden, n_out) if persistent else d)
    x = to_tensor(a["partial"])  # any bf16 [rows, H] stands for x_next
    q = torch.zeros((rows, n_out), dtype=BF16, device="cuda")
    rel.mb_next_qkv(d, x, to_tensor(a["w_qkvg"]), q, ws)
    torch.cuda.synchronize()
    assert_close(bits(q), oracle.next_qkv(a["partial"], a["w_qkvg"]), "qkvg")


def test_ffn_half_of_a_layer_chained():
    """attention boundary -> block -> next QKV at c1, each stage checked on the
    GPU's own input to it (the block end to end as in the block tests)."""
    blk = synth.make_block("c1")
    d = blk.dims
    a = synth.make_attn_side(d.rows, d.hidden, QKVG_C1, 70)
    say("[gpu] chained: attention boundary, block, next qkv (c1)")
    g = GpuBlock(blk)
    stream = to_tensor(a["stream"])
    x = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
    t = {k: to_tensor(a[k]) for k in ("partial", "gate", "post_attn_norm_w", "pre_ffn_norm_w")}
    rel.mb_attn_boundary(g.dims, t["partial"], t["gate"], stream, x, t["post_attn_norm_w"], t["pre_ffn_norm_w"])
    torch.cuda.synchronize()
    s1_ref, x_ref = oracle.attn_boundary(a["partial"], a["stream"], a["gate"], a["post_attn_norm_w"],
                                         a["pre_ffn_norm_w"], d.norm_eps)
    s1 = stream.cpu().numpy()
    assert_close(s1, s1_ref, "stream after attention", atol=1e-5, rtol=1e-5, is_bf16=False)
    assert_close(bits(x), x_ref, "x")
    # The block on the GPU's x and stream.
    blk.x, blk.stream = bits(x), s1
    g.x, g.stream0 = x, stream
    got = g.run_block()
    assert_block(got, oracle.block(blk), "c1 after attention boundary", blk)
    q = torch.zeros((d.rows, QKVG_C1), dtype=BF16, device="cuda")
    rel.mb_next_qkv(g.dims, to_tensor(got["x_next"]), to_tensor(a["w_qkvg"]), q, g.ws)
    torch.cuda.synchronize()
    assert_close(bits(q), oracle.next_qkv(got["x_next"], a["w_qkvg"]), "qkvg on GPU x_next")


@pytest.mark.parametrize("zero_centered", [False, True])
def test_effective_norm_weight(zero_centered):
    import numpy as np
    rng = np.random.default_rng(90)
    w = (rng.standard_normal(5000) * 0.1).astype(np.float32)
    w[:4] = [0.0, -1.0, 2.0 ** -8, 3 * 2.0 ** -8]
    say(f"[gpu] effective norm weight zero_centered={zero_centered}")
    out = rel.mb_effective_norm_weight(to_tensor(w), 1.0, zero_centered)
    torch.cuda.synchronize()
    assert (bits(out) == oracle.effective_norm_weight(w, 1.0, zero_centered)).all()


def _block_with_qkv(g, n_out, w_qkvg):
    """mb_moe_block with the next-QKV projection fused (qkv_rows = n_out)."""
    d = g.blk.dims
    dims = rel.make_dims(**dims_kwargs(d), qkv_rows=n_out)
    wt = dict(g.wt, next_qkv_w=to_tensor(w_qkvg))
    ws = rel.workspace(dims)
    stream = g.stream0.clone()
    x_next = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
    qkvg = torch.zeros((d.rows, n_out), dtype=BF16, device="cuda")
    rel.mb_moe_block(dims, g.x, rel.make_weights(**wt), stream, x_next, ws, taps=rel.make_taps(qkvg=qkvg))
    torch.cuda.synchronize()
    assert int(ws[4:8].cpu().view(torch.int32)[0]) == 0, "block kernel aborted a wait"
    return {"stream": stream.cpu().numpy(), "x_next": bits(x_next), "qkvg": bits(qkvg)}, (dims, wt, ws)


@pytest.mark.parametrize("case,n_out", [("c1", QKVG_C1), ("b37", 1040), ("c2", 2048), ("b1", 16), ("b100", 528)])
def test_fused_next_qkv(case, n_out):
    """The block with the projection fused: the block's own outputs bit-identical
    to the block without it, qkvg within the bf16 tolerance of the oracle's
    projection of the GPU's x_next, and a second call on the same workspace
    bit-identical to the first (the tile counters are left at zero)."""
    import numpy as np
    if case == "b37":
        blk = synth.make_block("c0", seed=47, dims=synth.Dims(37, 512, 384, 640, 16, 4, "sigmoid", 2.5, None, 1e-20))
    elif case == "b1":
        blk = synth.make_block("c0", seed=48, dims=synth.Dims(1, 256, 128, 256, 8, 2, "sigmoid", 2.5, None, 1e-20))
    elif case == "b100":
        # Beyond 64 rows: the block's 64-row block tasks and the projection's rows in two passes.
        blk = synth.make_block("c0", seed=49, dims=synth.Dims(100, 256, 256, 1280, 8, 4, "softmax", 1.0, 1.5, 1e-6))
    else:
        blk = synth.make_block(case)
    d = blk.dims
    w_qkvg = synth.make_attn_side(1, d.hidden, n_out, 91)["w_qkvg"]
    say(f"[gpu] fused next qkv: {case} rows {d.rows} H {d.hidden} qkv_rows {n_out}")
    g = GpuBlock(blk)
    plain = g.run_block()
    got, (dims, wt, ws) = _block_with_qkv(g, n_out, w_qkvg)
    assert np.array_equal(got["stream"], plain["stream"])
    assert np.array_equal(got["x_next"], plain["x_next"])
    assert_close(got["qkvg"], oracle.next_qkv(got["x_next"], w_qkvg), f"{case}: fused qkvg")
    again, _ = _block_with_qkv(g, n_out, w_qkvg)
    assert np.array_equal(again["qkvg"], got["qkvg"])


def test_fused_next_qkv_with_w4a4():
    """Both options at once (c1): the W4A4 block's own outputs bit-identical
    with and without the fused projection, qkvg against the oracle on the
    GPU's x_next."""
    import numpy as np
    blk = synth.make_block("c1")
    d = blk.dims
    w_qkvg = synth.make_attn_side(1, d.hidden, 1024, 92)["w_qkvg"]
    say("[gpu] fused next qkv with W4A4 experts (c1, qkv_rows 1024)")
    g = GpuBlock(blk)
    g.use_packed()
    outs = []
    for qkv_rows in (0, 1024):
        dims = rel.make_dims(**dims_kwargs(d), act_quant=1, qkv_rows=qkv_rows)
        wt = dict(g.wt, next_qkv_w=to_tensor(w_qkvg))
        ws = rel.workspace(dims)
        stream = g.stream0.clone()
        x_next = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
        qkvg = torch.zeros((d.rows, 1024), dtype=BF16, device="cuda")
        rel.mb_moe_block(dims, g.x, rel.make_weights(**wt), stream, x_next, ws,
                         taps=rel.make_taps(qkvg=qkvg if qkv_rows else None))
        torch.cuda.synchronize()
        assert int(ws[4:8].cpu().view(torch.int32)[0]) == 0, "block kernel aborted a wait"
        outs.append((stream.cpu().numpy(), bits(x_next), bits(qkvg)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert_close(outs[1][2], oracle.next_qkv(outs[1][1], w_qkvg), "W4A4 fused qkvg")
