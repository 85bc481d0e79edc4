"""Front-end oracle: RMSNorm -> router projection -> top-k on raw logits -> activation.

TEST INFRASTRUCTURE (see the package header).

Source: NKI "RMSNorm Router Top-K A2AV Kernel API Reference", Background
(RMSNorm fused with router top-K for small T), Parameters (hidden_states
[B, S, H] bf16/fp16, gamma [1, H], router_weights [H, E], optional router_bias
[1, E], eps, top_k, router_act_fn SOFTMAX or SIGMOID), Returns (normalised
hidden [T, H], int32 top-K indices [T, K], bf16 masked affinities [T, E]) and
Notes (T <= 128, H divisible by 128, and the ACT2 pipeline: top-K is taken on
the raw logits and the activation is applied to the selected experts only).

Readings (listed in the design notes): RMSNorm is x * (mean(x^2) + eps)^(-1/2)
* gamma, rounded once to the input dtype; the projection consumes exactly the
rounded normalised values that are returned (so the routing half is checked
from the HIP path's own normalised output); router_bias is added to the logits;
sigmoid affinities are sigma(z) of the selected logits with no renormalisation;
softmax affinities are the softmax over the k selected logits; every other
affinity is exactly zero; ties go to the lower expert index.

Pins: tests/test_oracle_aux_front.py (constant rows, linearity in gamma, the
identity projection, library rounding of float16, affinities of given ids
against scipy's logistic and softmax).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def _decode(values, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        hi = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(values, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def bf16_round_bits(v) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest, ties to even); return bits.

    A normal bfloat16 carries 8 significant bits: write v = m * 2**e with
    0.5 <= |m| < 1 and round m * 2**8 to an integer, halves to even.  Below
    2**-126 the spacing is the fixed subnormal step 2**-133.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    small = np.abs(v) < 2.0 ** -126
    r = np.where(small, np.rint(np.ldexp(v, 133)) * 2.0 ** -133, r)
    if np.any(np.abs(r) > 3.3895313892515355e38):
        raise ValueError("overflow in bfloat16 rounding")
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _round_bits(v, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round_bits(v)
    if dtype == "f16":
        return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def rmsnorm(hidden, gamma, eps: float, dtype: str = "bf16"):
    """Return (normed float64 before rounding, normed bits rounded to ``dtype``)."""
    x = _decode(hidden, dtype)
    g = _decode(gamma, dtype).reshape(-1)
    if x.ndim != 2 or g.shape[0] != x.shape[1]:
        raise ValueError("hidden must be [T, H] and gamma [H]")
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + float(eps))
    y = x * r * g[None, :]
    return y, _round_bits(y, dtype)


@dataclass
class FrontEndResult:
    logits: np.ndarray        # float64 [T, E], from the given normed values
    abs_products: np.ndarray  # float64 [T, E], sum_h |normed[t,h] * W[h,e]|
    ids: np.ndarray           # int32 [T, k]
    affinities: np.ndarray    # uint16 bf16 bits [T, E]
    affinities64: np.ndarray  # float64 [T, E] before rounding


def front_end_route(normed_bits, router_weights, k: int, act: str = "sigmoid",
                    dtype: str = "bf16", router_bias=None) -> FrontEndResult:
    """Route from given normalised hidden states (bits in ``dtype``)."""
    a = _decode(normed_bits, dtype)
    w = _decode(router_weights, dtype)
    if a.ndim != 2 or w.ndim != 2 or a.shape[1] != w.shape[0]:
        raise ValueError("normed [T, H] and router_weights [H, E] required")
    z = a @ w
    absprod = np.abs(a) @ np.abs(w)
    if router_bias is not None:
        z = z + _decode(router_bias, dtype).reshape(1, -1)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-z, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    aff64 = affinities_for_ids(z, ids, act)
    return FrontEndResult(logits=z, abs_products=absprod, ids=ids,
                          affinities=bf16_round_bits(aff64), affinities64=aff64)


def affinities_for_ids(z: np.ndarray, ids, act: str = "sigmoid") -> np.ndarray:
    """Masked affinities [T, E] (float64, before rounding) of the given experts:
    the activation of the chosen logits only -- sigmoid of each, or the softmax
    over the k chosen -- at the chosen experts, zero everywhere else."""
    ids = np.asarray(ids).astype(np.int64)
    zs = np.take_along_axis(z, ids, axis=1)
    if act == "sigmoid":
        sel = 1.0 / (1.0 + np.exp(-zs))
    elif act == "softmax":
        e = np.exp(zs - zs.max(axis=1, keepdims=True))
        sel = e / e.sum(axis=1, keepdims=True)
    else:
        raise ValueError(act)
    aff64 = np.zeros(z.shape, dtype=np.float64)
    np.put_along_axis(aff64, ids, sel, axis=1)
    return aff64


def fp32_sum_near_ties(res: FrontEndResult, k: int, depth: int):
    """Tokens whose selection a float32 accumulation of the projection may
    decide differently from the exact logits.

    A sum of products accumulated in float32 along a chain of ``depth``
    roundings errs by at most depth * 2^-24 * sum_h |normed * W| per logit (the
    textbook forward error bound of recursive summation).  A token is exempt
    when, among its k+1 largest exact logits, two neighbours lie closer than
    the sum of their two bounds.  Returns (exempt [T] bool, bound [T, E], the
    logits sorted descending per token, their bounds in the same order)."""
    bound = depth * 2.0 ** -24 * res.abs_products
    order = np.argsort(-res.logits, axis=1, kind="stable")
    zs = np.take_along_axis(res.logits, order, 1)
    bs = np.take_along_axis(bound, order, 1)
    upto = min(k + 1, res.logits.shape[1])
    gaps = zs[:, :upto - 1] - zs[:, 1:upto]
    exempt = np.any(gaps < bs[:, :upto - 1] + bs[:, 1:upto], axis=1)
    return exempt, bound, zs, bs
