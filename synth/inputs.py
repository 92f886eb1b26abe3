"""Seeded input generators for the five block workloads.

Workloads (dims; scoring; scalars):

* ``c0`` tiny block: b=4, H=256, P=128, I=256, E=8, top_k=2; sigmoid;
  route_scale 2.5, division eps 1e-20, no router multiplier; seed 0.
* ``c1`` decode verify step: b=16, H=4096, P=2048, I=1024, E=64, top_k=4;
  sigmoid; route_scale 2.5, eps 1e-20; uniform routing (bias U(-0.01, 0.01));
  seed 1.
* ``c2`` larger block: b=64, H=7168, P=3072, I=1536, E=128, top_k=8; softmax;
  router multiplier 1.5, eps 1e-6, route_scale 2.5; router weights
  N(0, 1/sqrt(H)) so that logits are about N(0, 1); expert bias skewed towards
  16 hot experts; seed 2.
* ``c3`` row-bucket sweep at c2's dims with sigmoid scoring, b in
  {1, 2, 4, ..., 256}: one [256, H] activation draw, bucket b takes its first
  b rows; uniform or skewed bias; seed 3.
* ``c4`` 60 stacked c2-dims layers (c2's recipe), b=32; layer l's weights
  from seed 4 + l; the first layer's activations and the residual stream from
  seed 4.

Distributions (all workloads): x bf16 N(0,1); router weight fp32 N(0, 0.02)
(c0, c1) or N(0, 1/sqrt(H)) (c2-c4); pooler and unpooler bf16 N(0, 0.02);
MXFP4 expert codes uniform over all 16 E2M1 nibbles, packed two per byte with
the even element in the low nibble; one E8M0 scale byte per 32-element block
with exponent uniform in {-8..-4} (bytes 119..123); per-route norm weight bf16
N(1, 0.1); gate bf16 N(0.5, 0.1); residual stream fp32 N(0, 1).  The boundary
norm weights and the pre-expert norm weight are absent (None) in all five
workloads; ``norm_weights=True`` draws them as bf16 N(1, 0.1) for coverage.

Skewed bias: the hot experts are the first 16 ids of a permutation drawn from
an independent generator seeded ``[seed, 7]`` so the main draw order is not
disturbed.  ``skew="literal"`` puts +1.0 on them and 0 elsewhere (the
workload's literal statement); ``skew="calibrated"`` puts a value delta on
them instead, delta chosen by a committed script that runs the oracle so that
about half of all routes land on the 16 hot experts (the workload's stated
intent).  The deltas live in ``skew_calibration.json`` beside this file.

Draw order within one block: x, router weight, bias, pooler, unpooler, w13
codes, w13 scales, w2 codes, w2 scales, per-route norm weight, gate, stream,
then (only with ``norm_weights=True``) pre-expert, post-FFN and next-layer
norm weights.
"""

from __future__ import annotations

import dataclasses
import json
import os
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dims:
    rows: int
    hidden: int
    pooled: int
    inter: int
    experts: int
    top_k: int
    scoring: str  # "sigmoid" | "softmax"
    route_scale: float
    multiplier: Optional[float]  # None: no router output multiplier
    division_eps: Optional[float]  # None: no eps in the weight denominator
    norm_eps: float = 1e-6

    def with_rows(self, rows: int) -> "Dims":
        return dataclasses.replace(self, rows=rows)


C0 = Dims(4, 256, 128, 256, 8, 2, "sigmoid", 2.5, None, 1e-20)
C1 = Dims(16, 4096, 2048, 1024, 64, 4, "sigmoid", 2.5, None, 1e-20)
C2 = Dims(64, 7168, 3072, 1536, 128, 8, "softmax", 2.5, 1.5, 1e-6)
C3 = Dims(256, 7168, 3072, 1536, 128, 8, "sigmoid", 2.5, 1.5, 1e-6)
C4 = Dims(32, 7168, 3072, 1536, 128, 8, "softmax", 2.5, 1.5, 1e-6)

CONFIGS = {"c0": C0, "c1": C1, "c2": C2, "c3": C3, "c4": C4}
C3_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256)
C4_LAYERS = 60
SEEDS = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4": 4}
HOT_EXPERTS = 16


@dataclasses.dataclass
class BlockInputs:
    """One block's inputs.  bf16 tensors are held as uint16 bit patterns."""

    dims: Dims
    x: np.ndarray  # u16 [b, H]
    router_w: np.ndarray  # f32 [E, H]
    expert_bias: np.ndarray  # f32 [E]
    pool_w: np.ndarray  # u16 [P, H]
    unpool_w: np.ndarray  # u16 [H, P]
    w13: np.ndarray  # u8 [E, 2I, P/2]
    w13_scale: np.ndarray  # u8 [E, 2I, P/32]
    w2: np.ndarray  # u8 [E, P, I/2]
    w2_scale: np.ndarray  # u8 [E, P, I/32]
    post_norm_w: np.ndarray  # u16 [P]
    gate: np.ndarray  # u16 [H]
    stream: np.ndarray  # f32 [b, H]
    pre_norm_w: Optional[np.ndarray] = None  # u16 [P]
    ffn_norm_w: Optional[np.ndarray] = None  # u16 [H]
    next_norm_w: Optional[np.ndarray] = None  # u16 [H]

    def rows(self, b: int) -> "BlockInputs":
        """The same block on its first b activation / stream rows."""
        return dataclasses.replace(
            self,
            dims=self.dims.with_rows(b),
            x=np.ascontiguousarray(self.x[:b]),
            stream=np.ascontiguousarray(self.stream[:b]),
        )


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng, shape, mean, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std) + np.float32(mean))


def _mxfp4(rng, e, n, k):
    # Uniform bytes are two uniform nibbles; one scale byte per 32 elements.
    codes = rng.integers(0, 256, size=(e, n, k // 2), dtype=np.uint8)
    scales = rng.integers(127 - 8, 127 - 4 + 1, size=(e, n, k // 32), dtype=np.uint8)
    return codes, scales


def hot_experts(seed: int, experts: int) -> np.ndarray:
    return np.sort(np.random.default_rng([seed, 7]).permutation(experts)[:HOT_EXPERTS])


_CAL_PATH = os.path.join(os.path.dirname(__file__), "skew_calibration.json")


def skew_delta(name: str) -> float:
    """The calibrated hot-expert bias for workload ``name`` (c2, c3, c4)."""
    with open(_CAL_PATH) as f:
        return float(json.load(f)[name]["delta"])


def _bias(rng, dims: Dims, lo: float, hi: float, seed: int, skew: Optional[str], name: str):
    bias = rng.uniform(lo, hi, size=dims.experts).astype(np.float32)
    if skew is None:
        return bias
    if skew == "literal":
        delta = 1.0
    elif skew == "calibrated":
        delta = skew_delta(name)
    elif isinstance(skew, float):
        delta = skew
    else:
        raise ValueError(f"unknown skew {skew!r}")
    out = np.zeros(dims.experts, dtype=np.float32)
    out[hot_experts(seed, dims.experts)] = np.float32(delta)
    return out


def _draw(dims: Dims, seed: int, *, router_std: float, bias_range, skew, name,
          norm_weights: bool, x_rows: Optional[int] = None, routing_only: bool = False):
    rng = np.random.default_rng(seed)
    b, H, P, I, E = dims.rows, dims.hidden, dims.pooled, dims.inter, dims.experts
    xr = b if x_rows is None else x_rows
    x = _normal_bf16(rng, (xr, H), 0.0, 1.0)
    router_w = rng.standard_normal((E, H), dtype=np.float32) * np.float32(router_std)
    bias = _bias(rng, dims, bias_range[0], bias_range[1], seed, skew, name)
    if routing_only:
        return x, router_w, bias
    pool_w = _normal_bf16(rng, (P, H), 0.0, 0.02)
    unpool_w = _normal_bf16(rng, (H, P), 0.0, 0.02)
    w13, w13_scale = _mxfp4(rng, E, 2 * I, P)
    w2, w2_scale = _mxfp4(rng, E, P, I)
    post = _normal_bf16(rng, (P,), 1.0, 0.1)
    gate = _normal_bf16(rng, (H,), 0.5, 0.1)
    stream = rng.standard_normal((xr, H), dtype=np.float32)
    blk = BlockInputs(dims if x_rows is None else dims.with_rows(xr), x, router_w, bias,
                      pool_w, unpool_w, w13, w13_scale, w2, w2_scale, post, gate, stream)
    if norm_weights:
        blk.pre_norm_w = _normal_bf16(rng, (P,), 1.0, 0.1)
        blk.ffn_norm_w = _normal_bf16(rng, (H,), 1.0, 0.1)
        blk.next_norm_w = _normal_bf16(rng, (H,), 1.0, 0.1)
    return blk


def make_block(name: str, *, seed: Optional[int] = None, skew: Optional[str] = None,
               norm_weights: bool = False, dims: Optional[Dims] = None) -> BlockInputs:
    """Inputs of workload ``name`` (c0, c1, c2); ``dims`` overrides the shape."""
    d = dims if dims is not None else CONFIGS[name]
    s = SEEDS[name] if seed is None else seed
    if name in ("c0", "c1"):
        lo, hi = (-0.1, 0.1) if name == "c0" else (-0.01, 0.01)
        return _draw(d, s, router_std=0.02, bias_range=(lo, hi), skew=skew, name=name,
                     norm_weights=norm_weights)
    if name == "c2":
        sk = "calibrated" if skew is None else skew
        sk = None if sk == "uniform" else sk
        return _draw(d, s, router_std=1.0 / np.sqrt(d.hidden), bias_range=(-0.01, 0.01),
                     skew=sk, name=name, norm_weights=norm_weights)
    raise ValueError(name)


def make_c3_block(skew: Optional[str], *, seed: Optional[int] = None) -> BlockInputs:
    """The 256-row c3 block; ``.rows(b)`` gives bucket b.  skew: None = uniform."""
    d = CONFIGS["c3"]
    s = SEEDS["c3"] if seed is None else seed
    return _draw(d, s, router_std=1.0 / np.sqrt(d.hidden), bias_range=(-0.01, 0.01),
                 skew=skew, name="c3", norm_weights=False)


def make_c4_layer(layer: int, skew: Optional[str] = "calibrated") -> BlockInputs:
    """Layer ``layer`` (0..59) of the stack.  Its x and stream are placeholders:
    the stack feeds each layer the previous layer's outputs."""
    d = CONFIGS["c4"]
    return _draw(d, SEEDS["c4"] + layer, router_std=1.0 / np.sqrt(d.hidden),
                 bias_range=(-0.01, 0.01), skew=skew, name="c4", norm_weights=False)


def make_c4_stream():
    """(x0 bf16 bits [32, H], stream0 fp32 [32, H]) of the stack, from seed 4."""
    d = CONFIGS["c4"]
    rng = np.random.default_rng([SEEDS["c4"], 99])
    x0 = _normal_bf16(rng, (d.rows, d.hidden), 0.0, 1.0)
    s0 = rng.standard_normal((d.rows, d.hidden), dtype=np.float32)
    return x0, s0


def routing_inputs(name: str, skew: Optional[str] = None):
    """(x, router weight, bias) of workload ``name`` without drawing the rest:
    the same values ``make_block`` / ``make_c3_block`` / ``make_c4_layer(0)``
    draw first (c4: layer 0's router with the stack's first activations)."""
    d = CONFIGS[name]
    std = 0.02 if name in ("c0", "c1") else 1.0 / np.sqrt(d.hidden)
    rng_range = (-0.1, 0.1) if name == "c0" else (-0.01, 0.01)
    seed = SEEDS[name]
    x, w, bias = _draw(d, seed, router_std=std, bias_range=rng_range, skew=skew, name=name,
                       norm_weights=False, routing_only=True)
    if name == "c4":
        x = make_c4_stream()[0]
    return x, w, bias


def make_attn_side(rows: int, hidden: int, qkvg_rows: int, seed: int, norm_weights: bool = True) -> dict:
    """Inputs of the steps either side of the block: the attention's o_proj
    partial bf16 N(0, 1) [rows, H], the attention add's gate bf16 N(0.5, 0.1),
    the post-attention and pre-FFN norm weights bf16 N(1, 0.1) (or None), the
    stream fp32 N(0, 1), and the next layer's QKV + o-gate weight bf16
    N(0, 0.02) [qkvg_rows, H]; drawn in that order."""
    rng = np.random.default_rng(seed)
    out = {"partial": _normal_bf16(rng, (rows, hidden), 0.0, 1.0),
           "gate": _normal_bf16(rng, (hidden,), 0.5, 0.1)}
    out["post_attn_norm_w"] = _normal_bf16(rng, (hidden,), 1.0, 0.1) if norm_weights else None
    out["pre_ffn_norm_w"] = _normal_bf16(rng, (hidden,), 1.0, 0.1) if norm_weights else None
    out["stream"] = rng.standard_normal((rows, hidden)).astype(np.float32)
    out["w_qkvg"] = _normal_bf16(rng, (qkvg_rows, hidden), 0.0, 0.02)
    return out
