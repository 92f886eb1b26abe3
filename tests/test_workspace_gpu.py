"""GPU: one workspace serves any sequence of calls, and a captured launch
replays.

The persistent launch keeps its cross-workgroup counters in the workspace:
two counter sets, picked by a generation count that every launch advances,
each launch clearing the set the next one uses.  These tests check that state
carries over correctly -- from call to call at different row counts and
entry points (different task lists, so different counters in use), and from
replay to replay of a captured graph -- by comparing every result bit for bit
with the same call on a fresh workspace (the kernels are deterministic)."""

import numpy as np
import pytest

import oracle
import synth
from parity import GpuBlock, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dims(rows):
    return synth.Dims(rows, 256, 128, 256, 16, 4, "sigmoid", 2.5, None, 1e-20)


def _same(a: dict, b: dict, what: str) -> None:
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), f"{what}: {n}"


def test_one_workspace_many_calls_and_row_counts():
    big = synth.make_block("c0", seed=31, dims=_dims(100))
    shared = GpuBlock(big).ws  # sized for the most rows
    say("[gpu] shared workspace: block calls at rows 100, 4, 37, 1, 100, 64, 17")
    for i, b in enumerate([100, 4, 37, 1, 100, 64, 17]):
        g = GpuBlock(big.rows(b))
        fresh = g.run_block()
        g.ws = shared
        got = g.run_block()
        _same(got, fresh, f"call {i} rows {b}")
        if i == 2:
            # Other entry points on the same workspace in between.
            say("[gpu] shared workspace: route, pool, experts, unpool+boundary")
            r = g.run_route()
            h = g.run_pool()
            ref = oracle.route(g.blk)
            moe = g.run_experts(h, ref)
            g.run_unpool_boundary(moe)
            assert (r["topk_ids"] == ref.ids).all()


def test_captured_block_replays():
    import routed_expert_layer_amd as rel
    from synth.device import bits
    blk = synth.make_block("c0", seed=32, dims=_dims(37))
    g = GpuBlock(blk)
    d = blk.dims
    say("[gpu] graph replay: eager reference")
    want_stream = g.stream0.clone()
    want_next = torch.zeros((d.rows, d.hidden), dtype=torch.bfloat16, device="cuda")
    rel.mb_moe_block(g.dims, g.x, g.weights, want_stream, want_next, rel.workspace(g.dims))
    torch.cuda.synchronize()
    want = {"stream": want_stream.cpu().numpy(), "x_next": bits(want_next)}
    stream = torch.empty_like(g.stream0)
    x_next = torch.zeros_like(want_next)
    ws = rel.workspace(g.dims)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say("[gpu] graph replay: capture")
    with torch.cuda.graph(graph, stream=side, capture_error_mode="thread_local"):
        stream.copy_(g.stream0)
        rel.mb_moe_block(g.dims, g.x, g.weights, stream, x_next, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[gpu] graph replay {rep}")
        x_next.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert int(ws[4:8].cpu().view(torch.int32)[0]) == 0, "block kernel aborted a wait"
        assert np.array_equal(stream.cpu().numpy(), want["stream"]), rep
        assert np.array_equal(bits(x_next), want["x_next"]), rep
        # Eager work on the device between replays.
        g.run_block()


def test_abort_record_reported_and_reset():
    r"""A launch whose waits give up is reported by mb_workspace_status until
    mb_workspace_reset, and does not disturb later launches.  The record is
    pre-set from the host to the next launch's tag (the generation in the
    workspace's generation words, plus one), so that every bounded wait of
    that launch gives up after its first 256 polls and the kernel drains as
    usual: no wait is made to run out for real."""
    import routed_expert_layer_amd as rel
    from synth.device import bits
    blk = synth.make_block("c0", seed=33, dims=_dims(17))
    g = GpuBlock(blk)
    say("[gpu] abort record: a normal launch")
    want = g.run_block()
    st = rel.mb_workspace_status(g.ws)
    torch.cuda.synchronize()
    assert int(st.item()) == rel.MB_OK

    def launch():
        stream = g.stream0.clone()
        x_next = torch.zeros((blk.dims.rows, blk.dims.hidden), dtype=torch.bfloat16, device="cuda")
        rel.mb_moe_block(g.dims, g.x, g.weights, stream, x_next, g.ws)
        torch.cuda.synchronize()
        return stream.cpu().numpy(), bits(x_next)

    gen = int(g.ws[128:132].view(torch.int32).item())  # generation word of workgroup 0 (line 1)
    g.ws[4:8].view(torch.int32).fill_(gen + 1)
    say("[gpu] abort record: a launch whose waits give up")
    launch()
    st = rel.mb_workspace_status(g.ws)
    torch.cuda.synchronize()
    assert int(st.item()) == rel.MB_ERR_ABORTED
    say("[gpu] abort record: the next launch computes as usual, the record stays")
    s1, x1 = launch()
    assert np.array_equal(s1, want["stream"]) and np.array_equal(x1, want["x_next"])
    st = rel.mb_workspace_status(g.ws)
    torch.cuda.synchronize()
    assert int(st.item()) == rel.MB_ERR_ABORTED
    say("[gpu] abort record: reset")
    rel.mb_workspace_reset(g.ws)
    st = rel.mb_workspace_status(g.ws)
    torch.cuda.synchronize()
    assert int(st.item()) == rel.MB_OK
    s2, x2 = launch()
    assert np.array_equal(s2, want["stream"]) and np.array_equal(x2, want["x_next"])
    g.check_no_abort()
