"""Python binding of libmb.so, the MI355X routed-MoE block (include/mb.h).

Argument marshalling only: every function below hands device pointers of
torch tensors and the current HIP stream to the C entry point of the same
name; every step of the block runs in the library's HIP kernels.  There is no
fallback: if libmb.so is missing, or its call fails, the call raises.

bf16 tensors may be torch.bfloat16 or int16/uint16 bit patterns; all tensors
must be contiguous CUDA (HIP) tensors.  The caller keeps every tensor alive
while work that reads it is in flight.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmb.so")

EXPORTS = (
    "mb_workspace_bytes",
    "mb_route",
    "mb_pool",
    "mb_experts",
    "mb_unpool_boundary",
    "mb_moe_block",
    "mb_moe_block_noalloc",
    "mb_packed_experts_bytes",
    "mb_pack_experts",
    "mb_packed_projections_bytes",
    "mb_pack_projections",
    "mb_attn_boundary",
    "mb_next_qkv",
    "mb_effective_norm_weight",
    "mb_workspace_status",
    "mb_workspace_reset",
    "mb_status_string",
)

(MB_OK, MB_ERR_NULL, MB_ERR_DIMS, MB_ERR_UNSUPPORTED, MB_ERR_ALIGN, MB_ERR_WORKSPACE, MB_ERR_HIP,
 MB_ERR_ABORTED, MB_ERR_SCRATCH) = range(9)
MB_SCORING_SIGMOID, MB_SCORING_SOFTMAX = 0, 1
MB_LOGITS_OUT, MB_LOGITS_IN = 1, 2

_c_i32, _c_f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class Dims(ctypes.Structure):
    _fields_ = [("rows", _c_i32), ("hidden", _c_i32), ("pooled", _c_i32), ("inter", _c_i32),
                ("experts", _c_i32), ("top_k", _c_i32), ("scoring", _c_i32),
                ("route_scale", _c_f32), ("router_multiplier", _c_f32),
                ("division_eps", _c_f32), ("norm_eps", _c_f32), ("act_quant", _c_i32),
                ("qkv_rows", _c_i32)]


_WEIGHT_FIELDS = ("router_w", "expert_bias", "pool_w", "pre_norm_w", "w13", "w13_scale", "w2",
                  "w2_scale", "post_norm_w", "unpool_w", "ffn_norm_w", "gate", "next_norm_w",
                  "experts_packed", "next_qkv_w", "proj_packed")
_TAP_FIELDS = ("logits", "topk_ids", "topk_w", "count", "offset", "route_list", "active",
               "n_active", "h", "moe_out", "u", "timeline", "act", "qkvg")


class Weights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in _WEIGHT_FIELDS]


class Taps(ctypes.Structure):
    _fields_ = [(n, _vp) for n in _TAP_FIELDS]


class MbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m routed_expert_layer_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.mb_workspace_bytes.argtypes = [P(Dims), P(ctypes.c_size_t)]
        L.mb_route.argtypes = [P(Dims), _vp, P(Weights), _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.mb_pool.argtypes = [P(Dims), _vp, P(Weights), _vp, _vp, ctypes.c_size_t, _vp]
        L.mb_experts.argtypes = [P(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, P(Weights), _vp,
                                 _vp, ctypes.c_size_t, _vp]
        L.mb_unpool_boundary.argtypes = [P(Dims), _vp, P(Weights), _vp, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]
        L.mb_moe_block.argtypes = [P(Dims), _vp, P(Weights), _vp, _vp, P(Taps), _vp,
                                   ctypes.c_size_t, _vp]
        L.mb_moe_block_noalloc.argtypes = [P(Dims), _vp, P(Weights), _vp, _vp, P(Taps), _vp]
        L.mb_packed_experts_bytes.argtypes = [P(Dims), P(ctypes.c_size_t)]
        L.mb_pack_experts.argtypes = [P(Dims), P(Weights), _vp, ctypes.c_size_t, _vp]
        L.mb_packed_projections_bytes.argtypes = [P(Dims), P(ctypes.c_size_t)]
        L.mb_pack_projections.argtypes = [P(Dims), P(Weights), _vp, ctypes.c_size_t, _vp]
        L.mb_attn_boundary.argtypes = [P(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.mb_next_qkv.argtypes = [P(Dims), _vp, _vp, ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp]
        L.mb_effective_norm_weight.argtypes = [_vp, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, _vp, _vp]
        L.mb_workspace_status.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
        L.mb_workspace_reset.argtypes = [_vp, ctypes.c_size_t, _vp]
        L.mb_status_string.argtypes = [ctypes.c_int]
        L.mb_status_string.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name != "mb_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mb_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MB_OK:
        raise MbError(status, where)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, got {type(t)}")
    if not t.is_cuda:
        raise ValueError("libmb takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmb takes contiguous tensors only")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def make_dims(rows, hidden, pooled, inter, experts, top_k, scoring, route_scale,
              router_multiplier=None, division_eps=None, norm_eps=1e-6, act_quant=0, qkv_rows=0) -> Dims:
    """Dims from Python values; scoring is "sigmoid" / "softmax" or 0 / 1; an
    absent multiplier is 1.0 and an absent division eps is 0.0; act_quant 1
    quantizes the experts' activations to MXFP4 (the W4A4 variant); qkv_rows > 0
    fuses the next layer's QKV projection into mb_moe_block."""
    if isinstance(scoring, str):
        scoring = {"sigmoid": MB_SCORING_SIGMOID, "softmax": MB_SCORING_SOFTMAX}.get(scoring, -1)
    return Dims(int(rows), int(hidden), int(pooled), int(inter), int(experts), int(top_k),
                int(scoring), float(route_scale),
                1.0 if router_multiplier is None else float(router_multiplier),
                0.0 if division_eps is None else float(division_eps), float(norm_eps),
                int(act_quant), int(qkv_rows))


def make_weights(**tensors) -> Weights:
    """Weights from device tensors named as the fields of mb_weights."""
    unknown = set(tensors) - set(_WEIGHT_FIELDS)
    if unknown:
        raise KeyError(f"unknown weight names {sorted(unknown)}")
    return Weights(*[_p(tensors.get(n)) for n in _WEIGHT_FIELDS])


def make_taps(**tensors) -> Taps:
    unknown = set(tensors) - set(_TAP_FIELDS)
    if unknown:
        raise KeyError(f"unknown tap names {sorted(unknown)}")
    return Taps(*[_p(tensors.get(n)) for n in _TAP_FIELDS])


def mb_workspace_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mb_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)), "mb_workspace_bytes")
    return int(n.value)


def mb_packed_experts_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mb_packed_experts_bytes(ctypes.byref(dims), ctypes.byref(n)),
           "mb_packed_experts_bytes")
    return int(n.value)


def mb_pack_experts(dims: Dims, weights: Weights, packed: torch.Tensor) -> None:
    _check(lib().mb_pack_experts(ctypes.byref(dims), ctypes.byref(weights), _p(packed),
                                 packed.numel() * packed.element_size(), _stream()),
           "mb_pack_experts")


def pack_experts(dims: Dims, weights: Weights, device="cuda") -> torch.Tensor:
    """A new device buffer holding the experts of `weights` in the streaming
    layout (set it as the experts_packed weight; keep it alive with them)."""
    packed = torch.empty(mb_packed_experts_bytes(dims), dtype=torch.uint8, device=device)
    mb_pack_experts(dims, weights, packed)
    return packed


def mb_packed_projections_bytes(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mb_packed_projections_bytes(ctypes.byref(dims), ctypes.byref(n)),
           "mb_packed_projections_bytes")
    return int(n.value)


def mb_pack_projections(dims: Dims, weights: Weights, packed: torch.Tensor) -> None:
    _check(lib().mb_pack_projections(ctypes.byref(dims), ctypes.byref(weights), _p(packed),
                                     packed.numel() * packed.element_size(), _stream()),
           "mb_pack_projections")


def pack_projections(dims: Dims, weights: Weights, device="cuda") -> torch.Tensor:
    """A new device buffer holding the pooler's and unpooler's weights of
    `weights` in the streaming layout (set it as the proj_packed weight; keep
    it alive with them)."""
    packed = torch.empty(mb_packed_projections_bytes(dims), dtype=torch.uint8, device=device)
    mb_pack_projections(dims, weights, packed)
    return packed


def workspace(dims: Dims, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of mb_workspace_bytes(dims) bytes."""
    return torch.zeros(mb_workspace_bytes(dims), dtype=torch.uint8, device=device)


def mb_route(dims: Dims, x, weights: Weights, topk_ids, topk_w, count, offset, route_list,
             active, n_active, ws: torch.Tensor, logits=None, flags: int = 0) -> None:
    _check(lib().mb_route(ctypes.byref(dims), _p(x), ctypes.byref(weights), _p(logits),
                          int(flags), _p(topk_ids), _p(topk_w), _p(count), _p(offset),
                          _p(route_list), _p(active), _p(n_active), _p(ws), ws.numel(),
                          _stream()), "mb_route")


def mb_pool(dims: Dims, x, weights: Weights, h, ws: torch.Tensor) -> None:
    _check(lib().mb_pool(ctypes.byref(dims), _p(x), ctypes.byref(weights), _p(h), _p(ws),
                         ws.numel(), _stream()), "mb_pool")


def mb_experts(dims: Dims, h, topk_ids, topk_w, count, offset, route_list, active, n_active,
               weights: Weights, moe_out, ws: torch.Tensor) -> None:
    _check(lib().mb_experts(ctypes.byref(dims), _p(h), _p(topk_ids), _p(topk_w), _p(count),
                            _p(offset), _p(route_list), _p(active), _p(n_active),
                            ctypes.byref(weights), _p(moe_out), _p(ws), ws.numel(), _stream()),
           "mb_experts")


def mb_unpool_boundary(dims: Dims, moe_out, weights: Weights, stream, x_next,
                       ws: torch.Tensor, u_out=None) -> None:
    _check(lib().mb_unpool_boundary(ctypes.byref(dims), _p(moe_out), ctypes.byref(weights),
                                    _p(stream), _p(x_next), _p(u_out), _p(ws), ws.numel(),
                                    _stream()), "mb_unpool_boundary")


def mb_attn_boundary(dims: Dims, partial, gate, stream, out, post_attn_norm_w=None,
                     pre_ffn_norm_w=None) -> None:
    """The attention boundary (post_attn_norm, gated add into the fp32 stream
    in place, pre_ffn_norm into out): the block's input x."""
    _check(lib().mb_attn_boundary(ctypes.byref(dims), _p(partial), _p(post_attn_norm_w), _p(gate),
                                  _p(pre_ffn_norm_w), _p(stream), _p(out), _stream()),
           "mb_attn_boundary")


def mb_next_qkv(dims: Dims, x_next, w_qkvg, qkvg, ws: torch.Tensor) -> None:
    """qkvg = bf16(x_next @ w_qkvg^T), the next layer's QKV + o-gate projection."""
    _check(lib().mb_next_qkv(ctypes.byref(dims), _p(x_next), _p(w_qkvg), int(w_qkvg.shape[0]), _p(qkvg),
                             _p(ws), ws.numel(), _stream()), "mb_next_qkv")


def mb_effective_norm_weight(weight, gain_center: float = 0.0, zero_centered: bool = False):
    """The bf16 multiplier of a norm: bf16(weight (+ gain_center)), weight fp32 on the device."""
    out = torch.empty(weight.shape, dtype=torch.bfloat16, device=weight.device)
    _check(lib().mb_effective_norm_weight(_p(weight), int(weight.numel()), float(gain_center),
                                          int(bool(zero_centered)), _p(out), _stream()),
           "mb_effective_norm_weight")
    return out


def mb_workspace_status(ws: torch.Tensor) -> torch.Tensor:
    """A device int32 tensor receiving MB_OK, or MB_ERR_ABORTED if a launch on
    this workspace gave up a wait since it was zero-filled or reset (read it
    after the current stream has reached this call)."""
    out = torch.empty(1, dtype=torch.int32, device=ws.device)
    _check(lib().mb_workspace_status(_p(ws), ws.numel(), _p(out), _stream()), "mb_workspace_status")
    return out


def mb_workspace_reset(ws: torch.Tensor) -> None:
    """Clear the record mb_workspace_status reads."""
    _check(lib().mb_workspace_reset(_p(ws), ws.numel(), _stream()), "mb_workspace_reset")


def mb_moe_block(dims: Dims, x, weights: Weights, stream, x_next, ws: torch.Tensor,
                 taps: Optional[Taps] = None) -> None:
    _check(lib().mb_moe_block(ctypes.byref(dims), _p(x), ctypes.byref(weights), _p(stream),
                              _p(x_next), None if taps is None else ctypes.byref(taps), _p(ws),
                              ws.numel(), _stream()), "mb_moe_block")


def mb_moe_block_noalloc(dims: Dims, x, weights: Weights, stream, x_next,
                         taps: Optional[Taps] = None) -> None:
    """mb_moe_block on the library's static per-GPU scratch (no workspace)."""
    _check(lib().mb_moe_block_noalloc(ctypes.byref(dims), _p(x), ctypes.byref(weights), _p(stream),
                                      _p(x_next), None if taps is None else ctypes.byref(taps),
                                      _stream()), "mb_moe_block_noalloc")
