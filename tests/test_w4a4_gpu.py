"""GPU parity of the W4A4 variant: the experts' activations (h and act)
quantized to MXFP4 per block of 32 and multiplied on fp4 x fp4 products.

A quantized code is an integer decided by floating point, so both sides must
decide it from the same value: the oracle quantizes the GPU's own bf16 h and
act (the block's taps), and each stage is compared with the oracle's result
on the GPU's input to it.  Quantizing a bf16 value is exact arithmetic on
both sides (an exponent, a scaling by a power of two, a rounding to E2M1), so
equal inputs give equal codes.  The chain checked:
  h        against the oracle's pooler                 (bf16 tolerance)
  act      against the oracle's up half on the GPU's h (bf16 tolerance)
  moe_out  against the oracle's down half on the GPU's act
  u, stream, x_next on the GPU's moe_out and u, as in the bf16 tests.
End to end (no teacher forcing) a bf16 unit of act that straddles an E2M1
rounding boundary moves that element by a whole E2M1 step, so the end-to-end
comparison only reports how many codes the two sides took differently."""

import numpy as np
import pytest

import oracle
import routed_expert_layer_amd as rel
import synth
from parity import BF16, GpuBlock, assert_close, assert_routing, f, say
from synth.device import bits, dims_kwargs, to_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _q(g: GpuBlock) -> GpuBlock:
    g.use_packed()
    g.dims = rel.make_dims(**dims_kwargs(g.blk.dims), act_quant=1)
    return g


def _run(g: GpuBlock) -> dict:
    d = g.blk.dims
    b, k, I = d.rows, d.top_k, d.inter
    act = torch.zeros((b * k, I), dtype=BF16, device="cuda")
    stream = g.stream0.clone()
    x_next = torch.zeros((b, d.hidden), dtype=BF16, device="cuda")
    taps = g._routing_bufs()
    taps.update(h=torch.zeros((b, d.pooled), dtype=BF16, device="cuda"),
                moe_out=torch.zeros((b, d.pooled), dtype=BF16, device="cuda"),
                u=torch.zeros((b, d.hidden), dtype=BF16, device="cuda"), act=act)
    rel.mb_moe_block(g.dims, g.x, g.weights, stream, x_next, g.ws, taps=rel.make_taps(**taps))
    torch.cuda.synchronize()
    g.check_no_abort()
    out = {n: (bits(t) if t.dtype == BF16 else t.cpu().numpy()) for n, t in taps.items()}
    out["stream"] = stream.cpu().numpy()
    out["x_next"] = bits(x_next)
    # act rows are in grouped order: row i is route route_list[i] = t * k + j.
    per_route = np.zeros((b, k, I), np.uint16)
    rl = out["route_list"]
    per_route[rl // k, rl % k] = out["act"]
    out["act_route"] = per_route
    return out


def check_w4a4(blk, name: str) -> dict:
    d = blk.dims
    g = _q(GpuBlock(blk))
    say(f"[gpu] w4a4 {name}: rows {d.rows} H {d.hidden} P {d.pooled} I {d.inter} E {d.experts} k {d.top_k}")
    got = _run(g)
    r = oracle.route(blk)
    assert_routing(got, r, name)
    errs = {"h": assert_close(got["h"], oracle.pool(blk.x, blk.pool_w, blk.pre_norm_w, d.norm_eps), f"{name}: h")}
    _, act_tf, _ = oracle.experts(got["h"], r.ids, r.weights, blk.w13, blk.w13_scale, blk.w2, blk.w2_scale,
                                  blk.post_norm_w, d.norm_eps, want_routes=True, act_quant=True)
    errs["act"] = assert_close(got["act_route"], act_tf, f"{name}: act on GPU h")
    moe_tf, _ = oracle.experts_down(got["act_route"], r.ids, r.weights, blk.w2, blk.w2_scale, blk.post_norm_w,
                                    d.norm_eps, act_quant=True)
    errs["moe_out"] = assert_close(got["moe_out"], moe_tf, f"{name}: moe_out on GPU act")
    u_tf = oracle.unpool(got["moe_out"], blk.unpool_w)
    errs["u"] = assert_close(got["u"], u_tf, f"{name}: u on GPU moe_out")
    s_tf, x_tf = oracle.boundary(got["u"], blk.stream, blk.gate, blk.ffn_norm_w, blk.next_norm_w, d.norm_eps)
    errs["stream"] = assert_close(got["stream"], s_tf, f"{name}: stream on GPU u", atol=1e-5, rtol=1e-5,
                                  is_bf16=False)
    errs["x_next"] = assert_close(got["x_next"], x_tf, f"{name}: x_next on GPU u")
    # How many act codes the two sides decide differently end to end (the
    # GPU's act against the oracle's act on the GPU's h): report only.
    ca, _ = oracle.quantize_mxfp4(f(got["act_route"]))
    cb, _ = oracle.quantize_mxfp4(f(act_tf))
    say(f"[gpu] w4a4 {name}: max errors {errs}; act codes differing {int((ca != cb).sum())} of {ca.size}")
    return got


def test_w4a4_c0():
    check_w4a4(synth.make_block("c0"), "c0")


@pytest.mark.parametrize("dims", [
    # Ragged passes (up to 16 rows), odd chunk counts (3 up chunks, 5 down chunks).
    synth.Dims(37, 512, 384, 640, 16, 4, "sigmoid", 2.5, None, 1e-20),
    # 32-row passes (two 16-row column blocks) and down units of 10 chunks (the ring).
    synth.Dims(100, 256, 256, 1280, 8, 4, "softmax", 1.0, 1.5, 1e-6),
    # One row.
    synth.Dims(1, 256, 128, 256, 8, 2, "sigmoid", 2.5, None, 1e-20),
], ids=["b37_ragged", "b100_pass32", "b1"])
def test_w4a4_shapes(dims):
    check_w4a4(synth.make_block("c0", seed=41, dims=dims), f"b{dims.rows}")


def test_w4a4_c1_decode_step():
    check_w4a4(synth.make_block("c1"), "c1")


def test_w4a4_c2_softmax_block():
    """128 experts, top-8, softmax, H 7168 (the larger block's dims, with its
    hot-expert skew)."""
    check_w4a4(synth.make_block("c2"), "c2")


def test_w4a4_experts_entry_point_matches_block():
    """mb_experts with act_quant on the block's own h and routing gives the
    block's moe_out bit for bit (the same kernel code, deterministic)."""
    blk = synth.make_block("c0", seed=43, dims=synth.Dims(37, 512, 384, 640, 16, 4, "sigmoid", 2.5, None, 1e-20))
    g = _q(GpuBlock(blk))
    got = _run(g)
    say("[gpu] w4a4 mb_experts on the block's h and routing")
    d = blk.dims
    moe = torch.zeros((d.rows, d.pooled), dtype=BF16, device="cuda")
    rel.mb_experts(g.dims, to_tensor(got["h"]), to_tensor(got["topk_ids"]), to_tensor(got["topk_w"]),
                   to_tensor(got["count"]), to_tensor(got["offset"]), to_tensor(got["route_list"]),
                   to_tensor(got["active"]), to_tensor(got["n_active"]), g.weights, moe, g.ws)
    torch.cuda.synchronize()
    g.check_no_abort()
    assert np.array_equal(bits(moe), got["moe_out"])


def test_bf16_path_unchanged_by_the_flag_off():
    """act_quant 0 on the packed layout still matches the bf16 oracle (the
    W4A4 kernels are separate template instances)."""
    blk = synth.make_block("c0", seed=44)
    g = GpuBlock(blk)
    g.use_packed()
    got = g.run_block()
    ref = oracle.block(blk)
    assert_close(got["moe_out"], ref.moe_out, "c0 bf16 moe_out")


def test_w4a4_needs_the_streaming_layout():
    blk = synth.make_block("c0", seed=45)
    g = GpuBlock(blk)
    g.dims = rel.make_dims(**dims_kwargs(blk.dims), act_quant=1)
    with pytest.raises(rel.MbError) as e:
        g.run_block()
    assert e.value.status == rel.MB_ERR_UNSUPPORTED
