"""Host-side checks of libmb.so that need no GPU: it loads, exports every entry
point include/mb.h declares, and rejects bad arguments before any launch."""

import ctypes
import os
import re

import pytest

import routed_expert_layer_amd as rel
from routed_expert_layer_amd import (MB_ERR_ABORTED, MB_ERR_ALIGN, MB_ERR_DIMS, MB_ERR_NULL, MB_ERR_SCRATCH,
                                     MB_ERR_UNSUPPORTED, MB_ERR_WORKSPACE, MB_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(rel.LIB_PATH),
                                reason="libmb.so not built (python -m routed_expert_layer_amd.build)")


def header_functions():
    with open(os.path.join(ROOT, "include", "mb.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mb_\w+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = header_functions()
    for n in ("mb_route", "mb_pool", "mb_experts", "mb_unpool_boundary", "mb_moe_block",
              "mb_workspace_bytes", "mb_packed_experts_bytes", "mb_pack_experts", "mb_status_string",
              "mb_attn_boundary", "mb_next_qkv", "mb_effective_norm_weight", "mb_workspace_status",
              "mb_workspace_reset", "mb_moe_block_noalloc", "mb_packed_projections_bytes",
              "mb_pack_projections"):
        assert n in names
    assert set(names) == set(rel.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(rel.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), n


def c1_dims(**over):
    kw = dict(rows=16, hidden=4096, pooled=2048, inter=1024, experts=64, top_k=4,
              scoring="sigmoid", route_scale=2.5)
    kw.update(over)
    return rel.make_dims(**kw)


def status_of_ws(d):
    n = ctypes.c_size_t(0)
    return rel.lib().mb_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), n.value


def test_workspace_bytes_ok_and_monotone():
    st, n16 = status_of_ws(c1_dims())
    assert st == MB_OK and n16 > 0 and n16 % 256 == 0
    st, n64 = status_of_ws(c1_dims(rows=64))
    assert st == MB_OK and n64 > n16


@pytest.mark.parametrize("over,code", [
    (dict(rows=0), MB_ERR_DIMS),
    (dict(hidden=-32), MB_ERR_DIMS),
    (dict(top_k=65), MB_ERR_DIMS),
    (dict(scoring="relu"), MB_ERR_DIMS),
    (dict(norm_eps=-1.0), MB_ERR_DIMS),
    (dict(route_scale=float("inf")), MB_ERR_DIMS),
    (dict(rows=1025), MB_ERR_UNSUPPORTED),
    (dict(experts=2048, top_k=4), MB_ERR_UNSUPPORTED),
    (dict(top_k=17), MB_ERR_UNSUPPORTED),
    (dict(pooled=2000), MB_ERR_UNSUPPORTED),
    (dict(inter=1000), MB_ERR_UNSUPPORTED),
    (dict(hidden=4100), MB_ERR_UNSUPPORTED),
    (dict(rows=1024, experts=512), MB_ERR_UNSUPPORTED),
    (dict(act_quant=2), MB_ERR_DIMS),
    (dict(act_quant=-1), MB_ERR_DIMS),
])
def test_bad_dims_rejected(over, code):
    assert status_of_ws(c1_dims(**over))[0] == code


def test_status_strings():
    assert rel.status_string(0) == "ok"
    for st in range(1, MB_ERR_SCRATCH + 1):
        assert len(rel.status_string(st)) > 10
    assert "reset" in rel.status_string(MB_ERR_ABORTED)
    assert rel.status_string(99) == "unknown status"


FAKE = 0x100000  # a 16-byte-aligned address that is never dereferenced


def call_route(d, x=FAKE, wts=None, flags=0, logits=None, ws=FAKE, ws_bytes=1 << 40, out=FAKE):
    w = rel.Weights() if wts is None else wts
    return rel.lib().mb_route(ctypes.byref(d), x, ctypes.byref(w), logits, flags, out, out, out,
                              out, out, out, out, ws, ws_bytes, None)


def full_weights(**over):
    names = dict(router_w=FAKE, expert_bias=FAKE, pool_w=FAKE, w13=FAKE, w13_scale=FAKE, w2=FAKE,
                 w2_scale=FAKE, post_norm_w=FAKE, unpool_w=FAKE, gate=FAKE)
    names.update(over)
    return rel.Weights(*[names.get(n) for n in rel._WEIGHT_FIELDS])


def test_route_argument_checks_before_launch():
    d = c1_dims()
    assert call_route(d, wts=full_weights(router_w=None)) == MB_ERR_NULL
    assert call_route(d, wts=full_weights(expert_bias=None)) == MB_ERR_NULL
    assert call_route(d, wts=full_weights(), x=None) == MB_ERR_NULL
    assert call_route(d, wts=full_weights(), out=None) == MB_ERR_NULL
    assert call_route(d, wts=full_weights(), x=FAKE + 4) == MB_ERR_ALIGN
    assert call_route(d, wts=full_weights(), flags=1) == MB_ERR_NULL  # logits out needs a buffer
    assert call_route(d, wts=full_weights(), flags=3, logits=FAKE) == MB_ERR_DIMS
    assert call_route(d, wts=full_weights(), flags=8, logits=FAKE) == MB_ERR_DIMS
    assert call_route(d, wts=full_weights(), ws=None) == MB_ERR_WORKSPACE
    assert call_route(d, wts=full_weights(), ws_bytes=16) == MB_ERR_WORKSPACE
    assert call_route(d, wts=full_weights(), ws=FAKE + 8) == MB_ERR_ALIGN
    # Routing from given logits needs neither x nor the router weight.
    assert call_route(d, wts=full_weights(router_w=None), x=None, flags=2, logits=None) == MB_ERR_NULL


def test_other_entry_points_check_arguments():
    d = c1_dims()
    L = rel.lib()
    w = full_weights(w2=None)
    assert L.mb_experts(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == MB_ERR_NULL
    w = full_weights(pool_w=FAKE + 2)
    assert L.mb_pool(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == MB_ERR_ALIGN
    w = full_weights(gate=None)
    assert L.mb_unpool_boundary(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE,
                                1 << 40, None) == MB_ERR_NULL
    w = full_weights()
    assert L.mb_unpool_boundary(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, FAKE + 4, FAKE,
                                1 << 40, None) == MB_ERR_ALIGN
    taps = rel.Taps(*([None] * 8 + [FAKE + 2, None, None]))
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(taps),
                          FAKE, 1 << 40, None) == MB_ERR_ALIGN
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), None, FAKE, None, FAKE, 1 << 40,
                          None) == MB_ERR_NULL
    bad = c1_dims(top_k=0)
    assert L.mb_moe_block(ctypes.byref(bad), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE,
                          1 << 40, None) == MB_ERR_DIMS


def test_binding_refuses_host_tensors():
    import torch
    d = c1_dims()
    with pytest.raises(ValueError):
        rel.mb_pool(d, torch.zeros(16, 4096, dtype=torch.bfloat16), rel.Weights(),
                    torch.zeros(1), torch.zeros(8, dtype=torch.uint8))


def test_packed_experts_bytes():
    # c1: per expert, up codes I*P, up scales (I/16) * ceil(P/512) * 512,
    # down codes P*I/2, down scales (P/32) * ceil(I/512) * 512: the caller
    # layout's bytes when P and I are multiples of 512.
    n = ctypes.c_size_t(0)
    assert rel.lib().mb_packed_experts_bytes(ctypes.byref(c1_dims()), ctypes.byref(n)) == 0
    P, I, E = 2048, 1024, 64
    assert n.value == E * (2 * I * P // 2 + 2 * I * P // 32 + P * I // 2 + P * I // 32)
    # Scales padded to groups of four chunks: P = 128 (one chunk), I = 384 (three).
    d = c1_dims(pooled=128, inter=384, experts=3, top_k=2)
    assert rel.lib().mb_packed_experts_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 3 * (384 * 128 + (384 // 16) * 512 + 128 * 384 // 2 + (128 // 32) * 512)
    assert rel.lib().mb_packed_experts_bytes(ctypes.byref(c1_dims(pooled=96)), ctypes.byref(n)) == 3


def test_pack_experts_argument_checks_before_launch():
    d = c1_dims()
    L = rel.lib()
    n = ctypes.c_size_t(0)
    L.mb_packed_experts_bytes(ctypes.byref(d), ctypes.byref(n))
    w = full_weights()
    assert L.mb_pack_experts(ctypes.byref(d), ctypes.byref(w), None, n.value, None) == MB_ERR_NULL
    assert L.mb_pack_experts(ctypes.byref(d), ctypes.byref(w), FAKE, n.value - 1, None) == MB_ERR_WORKSPACE
    assert L.mb_pack_experts(ctypes.byref(d), ctypes.byref(w), FAKE + 8, n.value, None) == MB_ERR_ALIGN
    w = full_weights(w2_scale=None)
    assert L.mb_pack_experts(ctypes.byref(d), ctypes.byref(w), FAKE, n.value, None) == MB_ERR_NULL


def test_packed_experts_stand_in_for_the_caller_layout():
    d = c1_dims()
    L = rel.lib()
    # Packed experts alone satisfy the experts' checks (the call then fails
    # on the missing workspace, before any launch) ...
    w = full_weights(w13=None, w13_scale=None, w2=None, w2_scale=None, experts_packed=FAKE)
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, None, 0,
                          None) == MB_ERR_WORKSPACE
    # ... a misaligned buffer is refused, and without either layout the experts are missing.
    w = full_weights(experts_packed=FAKE + 4)
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                          None) == MB_ERR_ALIGN
    w = full_weights(w13=None)
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                          None) == MB_ERR_NULL


def test_packed_projections_bytes():
    # Both matrices whole (P and H multiples of 16): P*H*2 bytes each, the
    # second from a 256-byte boundary.
    n = ctypes.c_size_t(0)
    assert rel.lib().mb_packed_projections_bytes(ctypes.byref(c1_dims()), ctypes.byref(n)) == MB_OK
    assert n.value == 2 * (2048 * 4096 * 2)
    # H = 96 (six 16-row tiles of the unpooler's matrix), P = 128.
    d = c1_dims(hidden=96, pooled=128, inter=128)
    assert rel.lib().mb_packed_projections_bytes(ctypes.byref(d), ctypes.byref(n)) == MB_OK
    assert n.value == (128 * 96 * 2 + 255) // 256 * 256 + 96 * 128 * 2
    assert rel.lib().mb_packed_projections_bytes(ctypes.byref(c1_dims(pooled=96)), ctypes.byref(n)) == 3
    assert rel.lib().mb_packed_projections_bytes(ctypes.byref(c1_dims()), None) == MB_ERR_NULL


def test_pack_projections_argument_checks_before_launch():
    d = c1_dims()
    L = rel.lib()
    n = ctypes.c_size_t(0)
    L.mb_packed_projections_bytes(ctypes.byref(d), ctypes.byref(n))
    w = full_weights()
    assert L.mb_pack_projections(ctypes.byref(d), ctypes.byref(w), None, n.value, None) == MB_ERR_NULL
    assert L.mb_pack_projections(ctypes.byref(d), ctypes.byref(w), FAKE, n.value - 1, None) == MB_ERR_WORKSPACE
    assert L.mb_pack_projections(ctypes.byref(d), ctypes.byref(w), FAKE + 8, n.value, None) == MB_ERR_ALIGN
    for missing in ("pool_w", "unpool_w"):
        w = full_weights(**{missing: None})
        assert L.mb_pack_projections(ctypes.byref(d), ctypes.byref(w), FAKE, n.value, None) == MB_ERR_NULL


def test_packed_projections_stand_in_for_the_caller_layout():
    d = c1_dims()
    L = rel.lib()
    # The packed projections alone satisfy the pooler's and unpooler's checks
    # (the calls then fail on the missing workspace, before any launch) ...
    w = full_weights(pool_w=None, unpool_w=None, proj_packed=FAKE)
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, None, 0,
                          None) == MB_ERR_WORKSPACE
    assert L.mb_pool(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, None, 0, None) == MB_ERR_WORKSPACE
    assert L.mb_unpool_boundary(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, None, 0,
                                None) == MB_ERR_WORKSPACE
    # ... a misaligned buffer is refused, and without either layout the weights are missing.
    w = full_weights(proj_packed=FAKE + 4)
    assert L.mb_pool(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == MB_ERR_ALIGN
    w = full_weights(pool_w=None)
    assert L.mb_pool(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == MB_ERR_NULL
    w = full_weights(unpool_w=None)
    assert L.mb_unpool_boundary(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                                None) == MB_ERR_NULL


def test_mxfp4_activations_need_the_streaming_layout():
    # act_quant 1 runs only in the block kernel's streaming path: without
    # experts_packed it is refused before any launch.
    d = c1_dims(act_quant=1)
    L = rel.lib()
    w = full_weights()
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                          None) == MB_ERR_UNSUPPORTED
    assert L.mb_experts(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == MB_ERR_UNSUPPORTED


def test_mxfp4_activations_limited_to_the_block_kernel_sizes():
    # With the streaming layout, act_quant 1 takes every size the block
    # kernel takes (up to 256 experts); beyond that it is refused before any
    # launch (the per-step kernels have no MXFP4-activation path).
    L = rel.lib()
    w = full_weights(experts_packed=FAKE)
    for E, want in ((257, MB_ERR_UNSUPPORTED), (512, MB_ERR_UNSUPPORTED)):
        d = c1_dims(act_quant=1, experts=E, top_k=8)
        assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                              None) == want, E
        assert L.mb_experts(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            ctypes.byref(w), FAKE, FAKE, 1 << 40, None) == want, E


def test_steps_around_the_block_check_arguments():
    d = c1_dims()
    L = rel.lib()
    # mb_attn_boundary(dims, partial, post_attn_norm_w, gate, pre_ffn_norm_w, stream, out, s)
    assert L.mb_attn_boundary(ctypes.byref(d), FAKE, None, None, None, FAKE, FAKE, None) == MB_ERR_NULL
    assert L.mb_attn_boundary(ctypes.byref(d), FAKE, FAKE + 2, FAKE, None, FAKE, FAKE, None) == MB_ERR_ALIGN
    assert L.mb_attn_boundary(ctypes.byref(d), FAKE, None, FAKE, None, None, FAKE, None) == MB_ERR_NULL
    # mb_next_qkv(dims, x_next, w_qkvg, n_out, qkvg, ws, ws_bytes, s)
    assert L.mb_next_qkv(ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, 1 << 40, None) == MB_ERR_DIMS
    assert L.mb_next_qkv(ctypes.byref(d), FAKE, FAKE, 24, FAKE, FAKE, 1 << 40, None) == MB_ERR_UNSUPPORTED
    assert L.mb_next_qkv(ctypes.byref(d), FAKE, None, 32, FAKE, FAKE, 1 << 40, None) == MB_ERR_NULL
    assert L.mb_next_qkv(ctypes.byref(d), FAKE, FAKE, 32, FAKE, FAKE, 16, None) == MB_ERR_WORKSPACE


def test_effective_norm_weight_checks_arguments():
    L = rel.lib()
    assert L.mb_effective_norm_weight(FAKE, 0, 1.0, 1, FAKE, None) == MB_ERR_DIMS
    assert L.mb_effective_norm_weight(FAKE, 8, float("nan"), 1, FAKE, None) == MB_ERR_DIMS
    assert L.mb_effective_norm_weight(None, 8, 1.0, 1, FAKE, None) == MB_ERR_NULL


def test_fused_qkv_options_checked_before_launch():
    assert status_of_ws(c1_dims(qkv_rows=-16))[0] == MB_ERR_DIMS
    assert status_of_ws(c1_dims(qkv_rows=24))[0] == MB_ERR_UNSUPPORTED
    assert status_of_ws(c1_dims(qkv_rows=65536 + 16))[0] == MB_ERR_UNSUPPORTED
    st, n0 = status_of_ws(c1_dims())
    st, n1 = status_of_ws(c1_dims(qkv_rows=1024))
    assert st == MB_OK and n1 > n0  # room for the projection's split partials
    L = rel.lib()
    d = c1_dims(qkv_rows=1024)
    w = full_weights()  # no next_qkv_w
    taps = rel.Taps(*([None] * len(rel._TAP_FIELDS)))
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, ctypes.byref(taps), FAKE,
                          1 << 40, None) == MB_ERR_NULL
    w = full_weights(next_qkv_w=FAKE)
    assert L.mb_moe_block(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE, None, FAKE, 1 << 40,
                          None) == MB_ERR_NULL  # qkvg tap missing


def test_workspace_status_and_reset_check_arguments():
    """The abort record's calls check the workspace (and the status pointer)
    before enqueuing anything."""
    lib = rel.lib()
    big = 1 << 30
    assert lib.mb_workspace_status(None, big, FAKE, None) == MB_ERR_NULL
    assert lib.mb_workspace_status(FAKE, big, None, None) == MB_ERR_NULL
    assert lib.mb_workspace_status(FAKE + 4, big, FAKE, None) == MB_ERR_ALIGN
    assert lib.mb_workspace_status(FAKE, big, FAKE + 2, None) == MB_ERR_ALIGN
    assert lib.mb_workspace_status(FAKE, 1024, FAKE, None) == MB_ERR_WORKSPACE
    assert lib.mb_workspace_reset(None, big, None) == MB_ERR_NULL
    assert lib.mb_workspace_reset(FAKE + 8, big, None) == MB_ERR_ALIGN
    assert lib.mb_workspace_reset(FAKE, 1024, None) == MB_ERR_WORKSPACE


def test_noalloc_block_checks_arguments_and_sizes_before_anything():
    """mb_moe_block_noalloc checks its arguments as mb_moe_block does, then
    refuses sizes its static scratch cannot hold, before any GPU call (here,
    without a GPU, anything else would come back as MB_ERR_HIP)."""
    L = rel.lib()
    w = full_weights()
    d = c1_dims()
    assert L.mb_moe_block_noalloc(ctypes.byref(d), FAKE, ctypes.byref(w), None, FAKE, None, None) == MB_ERR_NULL
    assert L.mb_moe_block_noalloc(ctypes.byref(d), FAKE, ctypes.byref(w), FAKE, FAKE + 2, None, None) == MB_ERR_ALIGN
    bad = c1_dims(top_k=0)
    assert L.mb_moe_block_noalloc(ctypes.byref(bad), FAKE, ctypes.byref(w), FAKE, FAKE, None, None) == MB_ERR_DIMS
    big = dict(hidden=7168, pooled=3072, inter=1536, experts=128, top_k=8, scoring="softmax")
    for rows, fits in ((1, True), (16, True), (32, True), (53, True), (54, False), (64, False), (256, False)):
        dd = c1_dims(rows=rows, **big)
        st, n = status_of_ws(dd)
        assert st == MB_OK
        got = L.mb_moe_block_noalloc(ctypes.byref(dd), FAKE, ctypes.byref(w), FAKE, FAKE, None, None)
        if fits:
            assert got != MB_ERR_SCRATCH, rows
        else:
            assert got == MB_ERR_SCRATCH, (rows, n)
    assert "56 MiB" in rel.status_string(MB_ERR_SCRATCH)
