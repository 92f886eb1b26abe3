"""GPU: mb_moe_block_noalloc (the block on the library's static per-GPU
scratch) gives mb_moe_block's results bit for bit, call after call: at the
b = 16 decode step, then at fewer rows, then at other dims (E 128, H 7168),
then at 80 rows (the many-rows kernel instance), then at the first size again (the kernels are deterministic, so any state
the scratch carried over wrongly would show as a difference)."""

import numpy as np
import pytest

import synth
from parity import BF16, GpuBlock, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _taps(d):
    import routed_expert_layer_amd as rel
    b, E, k, P, H = d.rows, d.experts, d.top_k, d.pooled, d.hidden
    t = dict(logits=torch.full((b, E), float("nan"), dtype=torch.float32, device="cuda"),
             topk_ids=torch.full((b, k), -1, dtype=torch.int32, device="cuda"),
             topk_w=torch.full((b, k), float("nan"), dtype=torch.float32, device="cuda"),
             h=torch.zeros((b, P), dtype=BF16, device="cuda"),
             moe_out=torch.zeros((b, P), dtype=BF16, device="cuda"),
             u=torch.zeros((b, H), dtype=BF16, device="cuda"))
    return t, rel.make_taps(**t)


def _run(g: GpuBlock, noalloc: bool) -> dict:
    import routed_expert_layer_amd as rel
    d = g.blk.dims
    stream = g.stream0.clone()
    x_next = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
    t, taps = _taps(d)
    if noalloc:
        rel.mb_moe_block_noalloc(g.dims, g.x, g.weights, stream, x_next, taps=taps)
    else:
        rel.mb_moe_block(g.dims, g.x, g.weights, stream, x_next, rel.workspace(g.dims), taps=taps)
    torch.cuda.synchronize()
    out = {n: v.cpu().view(torch.int16 if v.dtype == BF16 else v.dtype).numpy() for n, v in t.items()}
    out["stream"] = stream.cpu().numpy()
    out["x_next"] = x_next.cpu().view(torch.int16).numpy()
    return out


def _same(g: GpuBlock, what: str) -> None:
    say(f"[gpu] no-alloc block: {what}")
    want = _run(g, noalloc=False)
    got = _run(g, noalloc=True)
    for n in want:
        assert np.array_equal(got[n], want[n], equal_nan=True), f"{what}: {n} differs"


def test_noalloc_block_matches_the_workspace_block_call_after_call():
    c1 = GpuBlock(synth.make_block("c1"))
    c1.use_packed()
    _same(c1, "b=16, H 4096, E 64 (packed experts)")
    c1.set_rows(5)
    _same(c1, "b=5 of the same")
    big = GpuBlock(synth.make_c3_block("calibrated").rows(24))
    big.use_packed()
    _same(big, "b=24, H 7168, E 128 (skewed routing)")
    del big
    torch.cuda.empty_cache()
    many = GpuBlock(synth.make_block("c1", seed=5, dims=synth.inputs.C1.with_rows(80)))
    many.use_packed()
    _same(many, "b=80 at the decode dims (the many-rows instance: fp64-MFMA router, 64-row block "
                "tasks, plain staging, claimed unit rounds)")
    del many
    torch.cuda.empty_cache()
    c1 = GpuBlock(synth.make_block("c1"))
    _same(c1, "b=16 again, caller expert layout")
