"""Upload a BlockInputs to the GPU as torch tensors (plumbing, no arithmetic).

bf16 arrays travel as their uint16 bit patterns and arrive as torch.bfloat16
views of the same bytes.
"""

from __future__ import annotations

import numpy as np
import torch

from .inputs import BlockInputs, Dims

WEIGHT_NAMES = ("router_w", "expert_bias", "pool_w", "pre_norm_w", "w13", "w13_scale", "w2",
                "w2_scale", "post_norm_w", "unpool_w", "ffn_norm_w", "gate", "next_norm_w")


def to_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def dims_kwargs(d: Dims) -> dict:
    return dict(rows=d.rows, hidden=d.hidden, pooled=d.pooled, inter=d.inter, experts=d.experts,
                top_k=d.top_k, scoring=d.scoring, route_scale=d.route_scale,
                router_multiplier=d.multiplier, division_eps=d.division_eps, norm_eps=d.norm_eps)


def upload_weights(blk: BlockInputs, device="cuda") -> dict:
    out = {}
    for n in WEIGHT_NAMES:
        a = getattr(blk, n)
        out[n] = None if a is None else to_tensor(a, device)
    return out


def upload(blk: BlockInputs, device="cuda") -> tuple[dict, torch.Tensor, torch.Tensor]:
    """(weight tensors by mb_weights field name, x bf16 [b, H], stream fp32 [b, H])."""
    return upload_weights(blk, device), to_tensor(blk.x, device), to_tensor(blk.stream, device)


def bits(t: torch.Tensor) -> np.ndarray:
    """A bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
