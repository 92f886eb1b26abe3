"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
on seeded inputs and compare it with the oracle on the same inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import routed_expert_layer_amd as rel
from synth.device import bits, dims_kwargs, to_tensor, upload

BF16_ATOL, BF16_RTOL = 1e-2, 2e-2  # bf16 outputs and the fp32 stream
W_RTOL = 1e-5  # fp32 route weights

I32, F32, BF16 = torch.int32, torch.float32, torch.bfloat16


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class GpuBlock:
    """A block's inputs resident on the GPU, with its dims, weights and workspace."""

    def __init__(self, blk):
        self.blk = blk
        self.wt, self.x, self.stream0 = upload(blk)
        self.dims = rel.make_dims(**dims_kwargs(blk.dims))
        self.weights = rel.make_weights(**self.wt)
        self.ws = rel.workspace(self.dims)

    def set_rows(self, b: int) -> None:
        """Use only the first b rows of x and the stream (the weights stay)."""
        self.blk = self.blk.rows(b)
        self.x = self.x[:b].contiguous()
        self.stream0 = self.stream0[:b].contiguous()
        self.dims = rel.make_dims(**dims_kwargs(self.blk.dims))

    def use_packed(self, keep_plain: bool = False) -> torch.Tensor:
        """Stream the experts from mb_pack_experts' layout and the pooler's
        and unpooler's weights from mb_pack_projections' (and, unless
        keep_plain, pass no caller-layout pointers for them at all).  Returns
        the packed experts; the packed projections stay in proj_packed."""
        packed = rel.pack_experts(self.dims, self.weights)
        self.proj_packed = rel.pack_projections(self.dims, self.weights)
        torch.cuda.synchronize()
        self.wt["experts_packed"] = packed
        self.wt["proj_packed"] = self.proj_packed
        if not keep_plain:
            for n in ("w13", "w13_scale", "w2", "w2_scale", "pool_w", "unpool_w"):
                self.wt.pop(n, None)
        self.weights = rel.make_weights(**self.wt)
        return packed

    def set_bias(self, bias: np.ndarray) -> None:
        self.blk.expert_bias = bias
        self.wt["expert_bias"] = to_tensor(bias)
        self.weights = rel.make_weights(**self.wt)

    def check_no_abort(self):
        """No launch on the workspace gave up a wait (mb_workspace_status)."""
        st = rel.mb_workspace_status(self.ws)
        torch.cuda.synchronize()
        assert int(st.item()) == rel.MB_OK, "a block-kernel launch gave up a wait"

    def _routing_bufs(self):
        d = self.blk.dims
        b, E, k = d.rows, d.experts, d.top_k
        dev = "cuda"
        return dict(
            topk_ids=torch.full((b, k), -1, dtype=I32, device=dev),
            topk_w=torch.full((b, k), float("nan"), dtype=F32, device=dev),
            count=torch.full((E,), -1, dtype=I32, device=dev),
            offset=torch.full((E + 1,), -1, dtype=I32, device=dev),
            route_list=torch.full((b * k,), -1, dtype=I32, device=dev),
            active=torch.full((E,), -1, dtype=I32, device=dev),
            n_active=torch.full((1,), -1, dtype=I32, device=dev))

    def run_block(self) -> dict:
        d = self.blk.dims
        b, H, P, E = d.rows, d.hidden, d.pooled, d.experts
        stream = self.stream0.clone()
        x_next = torch.zeros((b, H), dtype=BF16, device="cuda")
        taps = self._routing_bufs()
        taps.update(logits=torch.full((b, E), float("nan"), dtype=F32, device="cuda"),
                    h=torch.zeros((b, P), dtype=BF16, device="cuda"),
                    moe_out=torch.zeros((b, P), dtype=BF16, device="cuda"),
                    u=torch.zeros((b, H), dtype=BF16, device="cuda"))
        rel.mb_moe_block(self.dims, self.x, self.weights, stream, x_next, self.ws,
                         taps=rel.make_taps(**taps))
        torch.cuda.synchronize()
        self.check_no_abort()
        out = {n: (bits(t) if t.dtype == BF16 else t.cpu().numpy()) for n, t in taps.items()}
        out["stream"] = stream.cpu().numpy()
        out["x_next"] = bits(x_next)
        return out

    def run_route(self, logits_in: np.ndarray | None = None) -> dict:
        d = self.blk.dims
        bufs = self._routing_bufs()
        if logits_in is None:
            lg = torch.full((d.rows, d.experts), float("nan"), dtype=F32, device="cuda")
            flags = rel.MB_LOGITS_OUT
        else:
            lg = to_tensor(np.ascontiguousarray(logits_in, dtype=np.float32))
            flags = rel.MB_LOGITS_IN
        rel.mb_route(self.dims, self.x, self.weights, ws=self.ws, logits=lg, flags=flags, **bufs)
        torch.cuda.synchronize()
        self.check_no_abort()
        out = {n: t.cpu().numpy() for n, t in bufs.items()}
        out["logits"] = lg.cpu().numpy()
        return out

    def run_pool(self) -> np.ndarray:
        d = self.blk.dims
        h = torch.zeros((d.rows, d.pooled), dtype=BF16, device="cuda")
        rel.mb_pool(self.dims, self.x, self.weights, h, self.ws)
        torch.cuda.synchronize()
        self.check_no_abort()
        return bits(h)

    def run_experts(self, h_bits: np.ndarray, r: oracle.Routing) -> np.ndarray:
        d = self.blk.dims
        moe = torch.zeros((d.rows, d.pooled), dtype=BF16, device="cuda")
        act = np.zeros(d.experts, np.int32)
        act[: r.n_active] = r.active
        rel.mb_experts(self.dims, to_tensor(h_bits), to_tensor(r.ids), to_tensor(r.weights),
                       to_tensor(r.count), to_tensor(r.offset), to_tensor(r.route_list),
                       to_tensor(act), to_tensor(np.array([r.n_active], np.int32)),
                       self.weights, moe, self.ws)
        torch.cuda.synchronize()
        self.check_no_abort()
        return bits(moe)

    def run_unpool_boundary(self, moe_bits: np.ndarray) -> dict:
        d = self.blk.dims
        stream = self.stream0.clone()
        x_next = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
        u = torch.zeros((d.rows, d.hidden), dtype=BF16, device="cuda")
        rel.mb_unpool_boundary(self.dims, to_tensor(moe_bits), self.weights, stream, x_next,
                               self.ws, u_out=u)
        torch.cuda.synchronize()
        self.check_no_abort()
        return {"u": bits(u), "stream": stream.cpu().numpy(), "x_next": bits(x_next)}


def f(b):
    return oracle.bf16_to_f64(b)


def assert_close(got, ref, name, atol=BF16_ATOL, rtol=BF16_RTOL, is_bf16=True):
    a = f(got) if is_bf16 else np.asarray(got, np.float64)
    b = f(ref) if is_bf16 else np.asarray(ref, np.float64)
    assert a.shape == b.shape, (name, a.shape, b.shape)
    err = np.abs(a - b)
    bad = ~(err <= atol + rtol * np.abs(b))
    if bad.any():
        i = np.unravel_index(np.argmax(err - rtol * np.abs(b)), a.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} of {a.size} outside tolerance; worst at "
                             f"{i}: got {a[i]!r} ref {b[i]!r}")
    return float(err.max()) if err.size else 0.0


def assert_routing(got: dict, r: oracle.Routing, name: str, check_logits=True) -> None:
    if check_logits and "logits" in got:
        diff = got["logits"] != r.logits
        assert not diff.any(), (f"{name}: fp32 logits differ at {np.argwhere(diff)[:5].tolist()} "
                                f"(got {got['logits'][diff][:5]}, ref {r.logits[diff][:5]})")
    rows = np.where((got["topk_ids"] != r.ids).any(1))[0]
    if rows.size:
        m = r.margins()[rows]
        raise AssertionError(f"{name}: topk_ids differ in rows {rows[:8].tolist()} "
                             f"(selection margins {m[:8].tolist()})")
    err = np.abs(got["topk_w"].astype(np.float64) - r.weights)
    bad = ~(err <= W_RTOL * np.abs(r.weights.astype(np.float64)))
    assert not bad.any(), f"{name}: route weights outside 1e-5 relative at {np.argwhere(bad)[:5].tolist()}"
    assert np.array_equal(got["count"], r.count), f"{name}: count"
    assert np.array_equal(got["offset"], r.offset), f"{name}: offset"
    assert np.array_equal(got["route_list"], r.route_list), f"{name}: route_list"
    assert int(got["n_active"][0]) == r.n_active, f"{name}: n_active"
    assert np.array_equal(got["active"][: r.n_active], r.active), f"{name}: active"


def plain_misses(got: dict, ref: oracle.BlockResult) -> dict:
    """Elements of u, stream and x_next outside the plain tolerance
    1e-2 + 2e-2 |ref| against the oracle's end-to-end result."""
    out = {}
    for n, r, is_bf16 in (("u", ref.u, True), ("stream", ref.stream, False), ("x_next", ref.x_next, True)):
        a = f(got[n]) if is_bf16 else np.asarray(got[n], np.float64)
        b = f(r) if is_bf16 else np.asarray(r, np.float64)
        out[n] = int((~(np.abs(a - b) <= BF16_ATOL + BF16_RTOL * np.abs(b))).sum())
    return out


def _ulp_bf16(v: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place of |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    return np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)


def assert_block(got: dict, ref: oracle.BlockResult, name: str, blk=None) -> dict:
    """Routing bit-exact; h, moe_out and u within the plain bf16 tolerance
    1e-2 + 2e-2 |ref| end to end; the stream and x_next within it plus what
    u's tolerance can move them (a bound computed from the oracle's values
    alone, below).

    Each stage after a bf16 rounding is also checked on the GPU's own input
    to it (teacher-forced: u on the GPU's moe_out, the boundary on the GPU's
    u), where only the stage's own arithmetic differs.  End to end, u may
    differ from the oracle's by up to its tolerance (the MoE output, whose
    bf16 rounding either side may take differently, feeds a long
    contraction), and the boundary carries that into the stream: to first
    order, with r = 1/rms(u), a change du of u moves v = RMSNorm_H(u) w_pff
    by at most w_pff,n r (|du_n| + |u_n| r^2 sum_k |u_k du_k| / H), and the
    stream by |g_n| times that; x_next = RMSNorm_H(stream) w_in moves the
    same way with the stream's bound.  Where |u_n| is several times rms(u)
    and the stream near zero, one bf16 unit of u already moves the stream
    by more than the absolute tolerance, so the plain tolerance alone would
    fail for reasons of rounding, not of a wrong kernel.  How many elements
    need the extra bound is logged per case."""
    assert_routing(got, ref.routing, name)
    errs = {}
    errs["h"] = assert_close(got["h"], ref.h, f"{name}: h")
    errs["moe_out"] = assert_close(got["moe_out"], ref.moe_out, f"{name}: moe_out")
    misses = plain_misses(got, ref)
    mo_ulps = np.abs(f(got["moe_out"]) - f(ref.moe_out)) / _ulp_bf16(f(ref.moe_out))
    say(f"[parity] {name}: outside 1e-2 + 2e-2|ref| end to end: " +
        ", ".join(f"{n} {m} of {got[n].size}" for n, m in misses.items()) +
        f"; moe_out bf16 units apart: max {mo_ulps.max():.1f}, over one {int((mo_ulps > 1).sum())}")
    errs.update({f"miss_{n}": m for n, m in misses.items()})
    errs["u"] = assert_close(got["u"], ref.u, f"{name}: u end to end")
    if blk is None:
        errs["stream"] = assert_close(got["stream"], ref.stream, f"{name}: stream", is_bf16=False)
        errs["x_next"] = assert_close(got["x_next"], ref.x_next, f"{name}: x_next")
        return errs
    u_tf = oracle.unpool(got["moe_out"], blk.unpool_w)
    errs["u_tf"] = assert_close(got["u"], u_tf, f"{name}: u on GPU moe_out")
    eps = blk.dims.norm_eps
    s_tf, x_tf = oracle.boundary(got["u"], blk.stream, blk.gate, blk.ffn_norm_w, blk.next_norm_w, eps)
    errs["stream_tf"] = assert_close(got["stream"], s_tf, f"{name}: stream on GPU u", atol=1e-5,
                                     rtol=1e-5, is_bf16=False)
    errs["x_next_tf"] = assert_close(got["x_next"], x_tf, f"{name}: x_next on GPU u")
    # End to end: the plain tolerance plus the first-order effect of u's.
    H = blk.dims.hidden
    uf = f(ref.u)
    du = BF16_ATOL + BF16_RTOL * np.abs(uf)
    wpff = 1.0 if blk.ffn_norm_w is None else np.abs(f(blk.ffn_norm_w))
    win = 1.0 if blk.next_norm_w is None else np.abs(f(blk.next_norm_w))
    ds = np.abs(f(blk.gate)) * _rmsnorm_bound(uf, du, eps, H) * wpff
    sref = ref.stream.astype(np.float64)
    e_s = np.abs(got["stream"].astype(np.float64) - sref)
    s_tol = BF16_ATOL + BF16_RTOL * np.abs(sref)
    bad = e_s > s_tol + ds
    assert not bad.any(), f"{name}: stream end to end outside tolerance at {np.argwhere(bad)[:5].tolist()}"
    xr = f(ref.x_next)
    e_x = np.abs(f(got["x_next"]) - xr)
    dx = win * _rmsnorm_bound(sref, s_tol + ds, eps, H)
    bad = e_x > BF16_ATOL + BF16_RTOL * np.abs(xr) + dx
    assert not bad.any(), f"{name}: x_next end to end outside tolerance at {np.argwhere(bad)[:5].tolist()}"
    errs["stream"], errs["x_next"] = float(e_s.max()), float(e_x.max())
    return errs


def _rmsnorm_bound(a: np.ndarray, da: np.ndarray, eps: float, n: int) -> np.ndarray:
    """First-order bound on how far a / rms(a) moves, per element, when each
    a_k moves by at most da_k (rows of a, rms over the last axis of n)."""
    r = 1.0 / np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + eps)
    return r * (da + np.abs(a) * r * r * np.sum(np.abs(a) * da, axis=-1, keepdims=True) / n)


def slice_result(ref: oracle.BlockResult, b: int, experts: int) -> oracle.BlockResult:
    """The oracle's result on the first b rows (rows are independent; the
    grouping is rebuilt from the first b rows' ids)."""
    r = ref.routing
    g = oracle.group_routes(r.ids[:b], experts)
    rr = oracle.Routing(r.logits[:b], r.scores[:b], r.keys[:b], r.ids[:b], r.weights[:b],
                        g["count"], g["offset"], g["route_list"], g["active"], int(g["n_active"]))
    return oracle.BlockResult(rr, ref.h[:b], ref.moe_out[:b], ref.u[:b], ref.stream[:b],
                              ref.x_next[:b])
