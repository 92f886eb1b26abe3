"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (mb_moe_block): the b=16 decode step, the b=64 softmax block
(both skew readings), the row-bucket sweep at its dims (uniform and both skew
readings) and the 60-layer stack, checked layer by layer on the GPU's own
inputs (teacher-forced).  The oracle computes every output of these sizes, so
the comparison is element by element."""

import numpy as np
import pytest

import oracle
import synth
from parity import GpuBlock, assert_block, assert_close, say, slice_result

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("layout", ["caller", "packed"])
def test_c1_decode_step(layout):
    blk = synth.make_block("c1")
    say(f"[gpu] c1 b=16 block, {layout} expert layout")
    g = GpuBlock(blk)
    if layout == "packed":
        g.use_packed()
    got = g.run_block()
    ref = oracle.block(blk)
    assert_block(got, ref, "c1", blk)


@pytest.mark.parametrize("skew,layout", [("calibrated", "caller"), ("literal", "caller"), ("uniform", "caller"),
                                         ("calibrated", "packed")])
def test_c2_softmax_block(skew, layout):
    blk = synth.make_block("c2", skew=skew)
    say(f"[gpu] c2 b=64 skew={skew}, {layout} expert layout")
    g = GpuBlock(blk)
    if layout == "packed":
        g.use_packed()
    got = g.run_block()
    ref = oracle.block(blk)
    assert_block(got, ref, f"c2 {skew}", blk)
    hot = synth.hot_experts(2, 128)
    share = np.isin(ref.routing.ids, hot).mean()
    say(f"[gpu] c2 {skew}: hot-expert share of routes {share:.3f}, active experts {ref.routing.n_active}")


@pytest.fixture(scope="module")
def c3_gpu():
    blk = synth.make_c3_block(None)
    return GpuBlock(blk), blk


@pytest.mark.parametrize("skew", [None, "calibrated", "literal"])
def test_c3_bucket_sweep(c3_gpu, skew):
    g, blk0 = c3_gpu
    full = synth.make_c3_block(skew) if skew else blk0
    ref = oracle.block(full)
    g.blk = full
    g.set_bias(full.expert_bias)
    base_x, base_s = g.x, g.stream0
    for b in synth.inputs.C3_BUCKETS:
        say(f"[gpu] c3 skew={skew} b={b}")
        g.x, g.stream0, g.blk = base_x, base_s, full
        g.set_rows(b)
        got = g.run_block()
        assert_block(got, slice_result(ref, b, 128), f"c3 {skew} b={b}", g.blk)
    g.x, g.stream0, g.blk = base_x, base_s, full


def test_c4_stack_teacher_forced():
    """Layers 0-2 and 59 of the stack, each checked on the GPU's own input
    (x, stream) from the layer before; the chain starts at the stack input."""
    x, s = synth.make_c4_stream()
    for layer in (0, 1, 2, 59):
        blk = synth.make_c4_layer(layer)
        blk.x, blk.stream = x, s
        say(f"[gpu] c4 layer {layer}")
        g = GpuBlock(blk)
        got = g.run_block()
        ref = oracle.block(blk)
        assert_block(got, ref, f"c4 layer {layer}", blk)
        x, s = got["x_next"], got["stream"]
        del g
        torch.cuda.empty_cache()
