"""Seeded synthetic inputs for the MoE routing workloads.

This module is shared by the CPU oracle's tests, the HIP path's tests and the
benchmark.  It only draws random numbers and stores them in the dtypes the
routing entry points accept; it holds none of the routing arithmetic (no score
function, no selection, no permutation, no loss).

Recipe (one ``numpy.random.default_rng(seed)`` per workload, drawn in the order
the fields are listed): ``standard_normal(float64) * std + mean`` ->
``astype(float32)`` (round to nearest) -> bfloat16 by round-to-nearest-even on
the float32 bit pattern where a bfloat16 input is asked for.  bfloat16 arrays
are carried as ``uint16`` bit patterns so that both sides receive the same bits.

The routing problem statement these shapes follow: router logits of shape
(tokens, experts) in float32 or bfloat16 with an optional per-expert bias
(FlashInfer trtllm_gen_routing, Parameters), and a small-T decode front end
with hidden [T, H], gamma [H] and router weights [H, E] in bf16/fp16
(NKI rmsnorm_router_topk_a2av, Parameters).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

__all__ = [
    "RouteWorkload", "FrontEndWorkload", "WORKLOADS", "FRONT_END",
    "bf16_bits_from_f32", "f32_from_bf16_bits", "draw_normal",
    "route_inputs", "front_end_inputs", "skewed_logits", "constant_logits",
    "tie_heavy_logits",
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_normal(rng: np.random.Generator, shape, std: float, mean: float = 0.0,
                dtype: str = "f32") -> np.ndarray:
    """One draw in the recipe order; returns float32 values or bf16 bits."""
    x = (rng.standard_normal(shape) * std + mean).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclass(frozen=True)
class RouteWorkload:
    """A routing workload: shapes, method flags and the input distribution."""
    name: str
    seed: int
    T: int
    E: int
    k: int
    score_fn: str                  # "softmax" | "sigmoid"
    pre_softmax: bool              # softmax only: softmax over E before top-k
    n_group: int = 0               # 0/1: ungrouped
    topk_group: int = 0
    group_topn: int = 2            # experts summed into a group's score
    renorm: bool = True
    scale: float = 1.0
    logits_dtype: str = "f32"
    logits_std: float = 1.0
    bias_std: Optional[float] = None   # None: no bias
    bias_dtype: str = "f32"
    tile: int = 8
    aux_coeff: Optional[float] = None  # aux-loss coefficient when the workload has one
    description: str = ""

    @property
    def has_bias(self) -> bool:
        return self.bias_std is not None


@dataclass(frozen=True)
class FrontEndWorkload:
    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    eps: float = 1e-6
    act: str = "sigmoid"
    dtype: str = "bf16"
    hidden_std: float = 1.0
    gamma_mean: float = 1.0
    gamma_std: float = 0.1
    weight_std: float = 0.02
    router_bias_std: Optional[float] = None
    description: str = ""


# The five workloads, named by what they are.  Seeds: 1000 * position.
WORKLOADS = {
    "tiny_softmax_post": RouteWorkload(
        name="tiny_softmax_post", seed=1000, T=16, E=8, k=2, score_fn="softmax",
        pre_softmax=False, renorm=True, scale=1.0, logits_dtype="f32", tile=4,
        description="T=16 E=8 k=2 fp32 N(0,1), softmax after top-k, tile 4"),
    "mixtral_like": RouteWorkload(
        name="mixtral_like", seed=2000, T=4096, E=8, k=2, score_fn="softmax",
        pre_softmax=True, renorm=True, scale=1.0, logits_dtype="f32", tile=8,
        description="T=4096 E=8 k=2 fp32 N(0,1), softmax before top-k + renorm, tile 8"),
    "deepseek_v3_like": RouteWorkload(
        name="deepseek_v3_like", seed=3000, T=16384, E=256, k=8, score_fn="sigmoid",
        pre_softmax=False, n_group=8, topk_group=4, group_topn=2, renorm=True,
        scale=2.5, logits_dtype="bf16", logits_std=1.0, bias_std=0.01,
        bias_dtype="f32", tile=8,
        description="T=16384 E=256 k=8 bf16 N(0,1), grouped sigmoid + fp32 bias "
                    "N(0,0.01), 8 groups keep 4, top-2-sum group score, x2.5, tile 8"),
    "qwen_moe_like": RouteWorkload(
        name="qwen_moe_like", seed=4000, T=65536, E=128, k=8, score_fn="softmax",
        pre_softmax=True, renorm=True, scale=1.0, logits_dtype="bf16",
        logits_std=1.5, tile=16, aux_coeff=1e-2,
        description="T=65536 E=128 k=8 bf16 N(0,1.5), softmax before top-k + renorm, "
                    "aux loss coeff 1e-2, tile 16"),
}

FRONT_END = FrontEndWorkload(
    name="decode_front_end", seed=5000, T=128, H=7168, E=256, k=8,
    description="hidden [128,7168] bf16 N(0,1), gamma 1+N(0,0.1), W [7168,256] "
                "N(0,0.02), RMSNorm -> gate GEMM -> sigmoid top-8 on raw logits")


def route_inputs(w: RouteWorkload, T: Optional[int] = None, seed: Optional[int] = None):
    """Draw (logits, bias) for a workload; ``T`` overrides the token count.

    logits: float32 [T, E] or uint16 bf16 bits [T, E]; bias: float32 [E] /
    uint16 bits [E] / None.  Drawn in the order logits, bias.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T = w.T if T is None else T
    logits = draw_normal(rng, (T, w.E), w.logits_std, 0.0, w.logits_dtype)
    bias = None
    if w.has_bias:
        bias = draw_normal(rng, (w.E,), w.bias_std, 0.0, w.bias_dtype)
    return logits, bias


def front_end_inputs(f: FrontEndWorkload = FRONT_END, T: Optional[int] = None,
                     H: Optional[int] = None, E: Optional[int] = None,
                     seed: Optional[int] = None):
    """Draw (hidden, gamma, router_weights, router_bias) in that order (bf16 bits)."""
    rng = np.random.default_rng(f.seed if seed is None else seed)
    T = f.T if T is None else T
    H = f.H if H is None else H
    E = f.E if E is None else E
    hidden = draw_normal(rng, (T, H), f.hidden_std, 0.0, f.dtype)
    gamma = draw_normal(rng, (H,), f.gamma_std, f.gamma_mean, f.dtype)
    weights = draw_normal(rng, (H, E), f.weight_std, 0.0, f.dtype)
    rbias = None
    if f.router_bias_std is not None:
        rbias = draw_normal(rng, (E,), f.router_bias_std, 0.0, f.dtype)
    return hidden, gamma, weights, rbias


# ---- stress inputs (parity cases, not timed) ---------------------------------

def skewed_logits(T: int, E: int, seed: int, hot_expert: int = 0, shift: float = 3.0,
                  std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """N(0,std) logits with one expert's mean moved up: a hot expert."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, E)) * std).astype(np.float32)
    x[:, hot_expert] += np.float32(shift)
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def constant_logits(T: int, E: int, value: float = 0.25, dtype: str = "f32") -> np.ndarray:
    """Every logit equal: every selection is decided by the index rule."""
    x = np.full((T, E), value, dtype=np.float32)
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def tie_heavy_logits(T: int, E: int, seed: int, levels=(-1.0, 0.0, 0.5, 1.0),
                     dtype: str = "f32") -> np.ndarray:
    """Logits drawn from a small value set, so ties occur everywhere."""
    rng = np.random.default_rng(seed)
    x = rng.choice(np.asarray(levels, dtype=np.float32), size=(T, E))
    return x if dtype == "f32" else bf16_bits_from_f32(x)


def with_overrides(w: RouteWorkload, **kw) -> RouteWorkload:
    return replace(w, **kw)
