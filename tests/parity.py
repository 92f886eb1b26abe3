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
        """Stream the experts from mb_pack_experts' layout (and, unless
        keep_plain, pass no caller-layout expert pointers at all)."""
        packed = rel.pack_experts(self.dims, self.weights)
        torch.cuda.synchronize()
        self.wt["experts_packed"] = packed
        if not keep_plain:
            for n in ("w13", "w13_scale", "w2", "w2_scale"):
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


def _ulp_bf16(v: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place of |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    return np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)


def assert_block(got: dict, ref: oracle.BlockResult, name: str, blk=None) -> dict:
    """Routing bit-exact; h and moe_out within the bf16 tolerance end to end.

    u follows a bf16 rounding of moe_out, and the boundary one of u, that either
    side may take one unit apart (fp32 vs fp64 accumulation before the same
    rounding).  So u is checked on the GPU's own moe_out, and the boundary
    twice: on the GPU's own u (oracle boundary of that u:
    the fp32 stream within 1e-5, x_next within the bf16 tolerance), and end to
    end within the bf16 tolerance plus what one bf16 unit of u moves it."""
    assert_routing(got, ref.routing, name)
    errs = {}
    errs["h"] = assert_close(got["h"], ref.h, f"{name}: h")
    errs["moe_out"] = assert_close(got["moe_out"], ref.moe_out, f"{name}: moe_out")
    if blk is None:
        errs["u"] = assert_close(got["u"], ref.u, f"{name}: u")
        errs["stream"] = assert_close(got["stream"], ref.stream, f"{name}: stream", is_bf16=False)
        errs["x_next"] = assert_close(got["x_next"], ref.x_next, f"{name}: x_next")
        return errs
    # u follows the bf16 rounding of moe_out, which either side may take one
    # unit apart; over a long contraction such units add up.  So u is checked
    # on the GPU's own moe_out (the oracle's unpooler of it), and end to end
    # within the tolerance plus what the measured moe_out difference moves it.
    u_tf = oracle.unpool(got["moe_out"], blk.unpool_w)
    errs["u_tf"] = assert_close(got["u"], u_tf, f"{name}: u on GPU moe_out")
    drift = np.abs(f(u_tf) - f(ref.u))
    e_u = np.abs(f(got["u"]) - f(ref.u))
    bad = e_u > BF16_ATOL + BF16_RTOL * np.abs(f(ref.u)) + drift
    assert not bad.any(), f"{name}: u end to end outside tolerance at {np.argwhere(bad)[:5].tolist()}"
    errs["u"] = float(e_u.max())
    eps = blk.dims.norm_eps
    s_tf, x_tf = oracle.boundary(got["u"], blk.stream, blk.gate, blk.ffn_norm_w, blk.next_norm_w, eps)
    errs["stream_tf"] = assert_close(got["stream"], s_tf, f"{name}: stream on GPU u", atol=1e-5,
                                     rtol=1e-5, is_bf16=False)
    errs["x_next_tf"] = assert_close(got["x_next"], x_tf, f"{name}: x_next on GPU u")
    # End to end, allowing one bf16 unit of u to propagate through the boundary.
    uf = f(ref.u)
    rs_u = 1.0 / np.sqrt(np.mean(uf * uf, axis=1, keepdims=True) + eps)
    wpff = 1.0 if blk.ffn_norm_w is None else np.abs(f(blk.ffn_norm_w))
    win = 1.0 if blk.next_norm_w is None else np.abs(f(blk.next_norm_w))
    ds = np.abs(f(blk.gate)) * wpff * rs_u * _ulp_bf16(uf)
    sref = ref.stream.astype(np.float64)
    rs_s = 1.0 / np.sqrt(np.mean(sref * sref, axis=1, keepdims=True) + eps)
    e_s = np.abs(got["stream"].astype(np.float64) - sref)
    bad = e_s > BF16_ATOL + BF16_RTOL * np.abs(sref) + ds
    assert not bad.any(), f"{name}: stream end to end outside tolerance at {np.argwhere(bad)[:5].tolist()}"
    xr = f(ref.x_next)
    e_x = np.abs(f(got["x_next"]) - xr)
    bad = e_x > BF16_ATOL + BF16_RTOL * np.abs(xr) + rs_s * win * ds
    assert not bad.any(), f"{name}: x_next end to end outside tolerance at {np.argwhere(bad)[:5].tolist()}"
    errs["stream"], errs["x_next"] = float(e_s.max()), float(e_x.max())
    return errs


def slice_result(ref: oracle.BlockResult, b: int, experts: int) -> oracle.BlockResult:
    """The oracle's result on the first b rows (rows are independent; the
    grouping is rebuilt from the first b rows' ids)."""
    r = ref.routing
    g = oracle.group_routes(r.ids[:b], experts)
    rr = oracle.Routing(r.logits[:b], r.scores[:b], r.keys[:b], r.ids[:b], r.weights[:b],
                        g["count"], g["offset"], g["route_list"], g["active"], int(g["n_active"]))
    return oracle.BlockResult(rr, ref.h[:b], ref.moe_out[:b], ref.u[:b], ref.stream[:b],
                              ref.x_next[:b])
