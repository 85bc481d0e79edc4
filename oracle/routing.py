"""Routing oracle: score function -> bias -> group-limited selection -> top-k -> weights.

TEST INFRASTRUCTURE (see the package header): only tests, the smoke check and
the benchmark's CPU baseline use it.

What each step follows (page title, section):

* score function, softmax or sigmoid, applied before top-k ("pre-softmax") or
  after it ("post-softmax"), optional expert bias, group top-k, scaling --
  TransformerEngine Fused Router, Description (FusedTopkScoreFunction) and
  I/O Contract (inputs ``score_function``, ``use_pre_softmax``, ``num_groups``,
  ``group_topk``, ``scaling_factor``, ``expert_bias``);
* grouped routing with ``n_group`` / ``topk_group`` (0 disables it), routing bias
  used by the DeepSeek-V3-style methods, ``routed_scaling_factor``,
  ``norm_topk_prob`` -- FlashInfer trtllm_gen_routing, Parameters;
* sigmoid scores in float32, selection by score plus correction bias, weights
  from the unbiased score, optional renormalisation to 1, then times the routed
  scaling factor -- MAX SigmoidTopKRouter, routing steps 2-4 and Parameters;
* softmax + top-k normalisation + routed scale in the gate -- LMDeploy MoeUtils,
  Description (invokeMoeGate_V2) and Usage Examples.

Readings where the pages are silent (each is listed in the design notes):
group score = sum of the ``group_topn`` largest keys of the group (the
DeepSeek-V3-like workload fixes top-2); groups are contiguous equal slices;
ties go to the lower expert index (and the lower group index); a token's ids
are listed by descending key; the bias enters the selection key only, never a
weight; renormalisation divides by the plain sum; full-E "scores" for the aux
loss are the softmax over E, or sigmoid scores divided by their sum.

Near ties (the parity rule the routing methods are held to): a token whose
exact-key gap at a deciding position lies in (0, 1e-6) relative is exempt from
bit-exact ids; ``within_near_ties`` states what such a token may still return.

Pins: tests/test_oracle_routing.py (closed forms, invariants, library
softmax, brute-force enumeration of every k-subset on tiny inputs, near-tie
cases with gaps of 15 and 18 float32 ulps on each side of 1e-6).
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass
from typing import Optional

import numpy as np

NEAR_TIE_REL = 1e-6


def decode_input(values, dtype: str) -> np.ndarray:
    """Widen a stored input exactly to float64.

    ``f32``: float32 array.  ``bf16``: uint16 bit patterns; a bfloat16 value is
    the float32 whose upper 16 bits are those bits and whose lower 16 are zero.
    ``f64``: float64 values as given (the finite-difference pins of the
    backward perturb logits below float32 resolution).
    """
    if dtype == "f64":
        return np.array(values, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        hi = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def selection_keys32(x64: np.ndarray, score_fn: str, pre_softmax: bool,
                     bias64: Optional[np.ndarray]) -> np.ndarray:
    """Selection keys in float32, the precision the selection is decided in.

    sigmoid: s = 1 / (1 + exp(-x)); key = s + bias.
    softmax before top-k: p = exp(x - max x) / sum exp(x - max x); key = p + bias.
    softmax after top-k: key = x + bias.
    """
    x = x64.astype(np.float32)                 # exact: inputs are f32 or bf16
    one = np.float32(1.0)
    with np.errstate(over="ignore", under="ignore"):
        if score_fn == "sigmoid":
            key = one / (one + np.exp(-x))
        elif score_fn == "softmax" and pre_softmax:
            m = x.max(axis=1, keepdims=True)
            e = np.exp(x - m)
            key = e / e.sum(axis=1, keepdims=True, dtype=np.float32)
        elif score_fn == "softmax":
            key = x.copy()
        else:
            raise ValueError(score_fn)
    key = key.astype(np.float32)
    if bias64 is not None:
        key = key + bias64.astype(np.float32)
    return key.astype(np.float32)


def exact_keys64(x64: np.ndarray, score_fn: str, pre_softmax: bool,
                 bias64: Optional[np.ndarray]) -> np.ndarray:
    """The same keys in float64; used only to measure near-tie gaps."""
    with np.errstate(over="ignore", under="ignore"):
        if score_fn == "sigmoid":
            key = 1.0 / (1.0 + np.exp(-x64))
        elif pre_softmax:
            m = x64.max(axis=1, keepdims=True)
            e = np.exp(x64 - m)
            key = e / e.sum(axis=1, keepdims=True)
        else:
            key = x64.copy()
    if bias64 is not None:
        key = key + bias64
    return key


def _group_scores(keys: np.ndarray, n_group: int, group_topn: int) -> np.ndarray:
    """Per group: sum of its ``group_topn`` largest keys, added largest first."""
    T, E = keys.shape
    kg = keys.reshape(T, n_group, E // n_group)
    top = -np.sort(-kg, axis=2)[:, :, :group_topn]
    score = np.zeros((T, n_group), dtype=keys.dtype)
    for i in range(group_topn):
        score = score + top[:, :, i]
    return score


def _keep_groups(score: np.ndarray, topk_group: int) -> np.ndarray:
    """Keep the ``topk_group`` best groups; ties go to the lower group index."""
    order = np.argsort(-score, axis=1, kind="stable")
    kept = np.zeros(score.shape, dtype=bool)
    np.put_along_axis(kept, order[:, :topk_group], True, axis=1)
    return kept


def grouping_active(n_group: int, topk_group: int) -> bool:
    """Grouping is off for n_group <= 1 or topk_group == 0 (TE example passes
    num_groups=1, group_topk=0; FlashInfer: 0 disables grouping); keeping every
    group is the same as no grouping."""
    return n_group > 1 and 0 < topk_group < n_group


def select_topk(keys32: np.ndarray, eligible: np.ndarray, k: int) -> np.ndarray:
    """The k largest eligible keys of each row, listed by descending key; equal
    keys go to the lower expert index (a stable sort of the negated keys)."""
    masked = np.where(eligible, keys32, np.float32(-np.inf)).astype(np.float32)
    order = np.argsort(-masked, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    return ids


def weights_for_ids(x: np.ndarray, ids, score_fn: str, pre_softmax: bool, renorm: bool,
                    scale: float) -> np.ndarray:
    """Routing weights (float64) of the given experts of each token.

    ``x``: decoded logits [T, E] (float64); ``ids``: [T, k] chosen experts, in
    any order (weight j belongs to ids[:, j]).  The bias never enters a weight.

    sigmoid: s = 1 / (1 + exp(-x)) of the chosen, divided by their sum when
    renormalising; softmax before top-k: the full softmax over E at the chosen,
    divided by their sum when renormalising; softmax after top-k: the softmax
    over the k chosen logits.  Then times ``scale``.
    """
    ids = np.asarray(ids).astype(np.int64)
    xs = np.take_along_axis(x, ids, axis=1)
    if score_fn == "sigmoid":
        w = 1.0 / (1.0 + np.exp(-xs))
        if renorm:
            w = w / w.sum(axis=1, keepdims=True)
    elif pre_softmax:
        m = x.max(axis=1, keepdims=True)
        p = np.exp(x - m)
        p = p / p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)
        if renorm:
            w = w / w.sum(axis=1, keepdims=True)
    else:
        # softmax over the k selected logits; already sums to one
        e = np.exp(xs - xs.max(axis=1, keepdims=True))
        w = e / e.sum(axis=1, keepdims=True)
    w = w * float(scale)
    return w


@dataclass
class RouteResult:
    ids: np.ndarray          # int32 [T, k], descending key, ties -> lower index
    weights: np.ndarray      # float64 [T, k]
    scores: np.ndarray       # float64 [T, E], full-E scores for the aux loss
    counts: np.ndarray       # int64 [E], tokens per expert
    exempt: np.ndarray       # bool [T], near-tie tokens (gap in (0, 1e-6) rel.)
    keys32: np.ndarray       # float32 [T, E], the decision keys (unmasked)
    keys64: np.ndarray       # float64 [T, E]
    eligible: np.ndarray     # bool [T, E], experts in kept groups
    group_scores64: Optional[np.ndarray] = None   # float64 [T, n_group] when grouped
    topk_group: int = 0


def route(logits, logits_dtype: str, k: int, score_fn: str = "softmax",
          pre_softmax: bool = True, n_group: int = 0, topk_group: int = 0,
          group_topn: int = 2, renorm: bool = True, scale: float = 1.0,
          bias=None, bias_dtype: str = "f32") -> RouteResult:
    """Route every token of ``logits`` [T, E]; see the module header for sources."""
    x = decode_input(logits, logits_dtype)
    if x.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = x.shape
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite logits are outside the supported domain")
    b = None if bias is None else decode_input(bias, bias_dtype).reshape(E)
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")

    # 1. score function and selection key (float32 decision, float64 gap)
    key32 = selection_keys32(x, score_fn, pre_softmax, b)
    key64 = exact_keys64(x, score_fn, pre_softmax, b)

    # 2. group-limited selection
    eligible = np.ones((T, E), dtype=bool)
    grouped = grouping_active(n_group, topk_group)
    if grouped:
        if E % n_group:
            raise ValueError("E must be a multiple of n_group")
        gsz = E // n_group
        if not 1 <= group_topn <= gsz:
            raise ValueError("group_topn must be in [1, E / n_group]")
        if k > topk_group * gsz:
            raise ValueError("k exceeds the experts of the kept groups")
        kept = _keep_groups(_group_scores(key32, n_group, group_topn), topk_group)
        eligible = np.repeat(kept, gsz, axis=1)

    # 3. top-k: key descending, ties by ascending expert index
    ids = select_topk(key32, eligible, k)

    # 4. weights (float64), bias never enters them
    w = weights_for_ids(x, ids, score_fn, pre_softmax, renorm, scale)

    # 5. full-E scores for the aux loss (no bias)
    if score_fn == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-x))
        scores = s / s.sum(axis=1, keepdims=True)
    else:
        m = x.max(axis=1, keepdims=True)
        p = np.exp(x - m)
        scores = p / p.sum(axis=1, keepdims=True)

    counts = np.bincount(ids.ravel().astype(np.int64), minlength=E).astype(np.int64)

    # 6. near-tie classification on the exact keys (reporting + parity exemption)
    exempt = _near_ties(key64, eligible, k, n_group, topk_group, group_topn, grouped)

    return RouteResult(ids=ids, weights=w, scores=scores, counts=counts,
                       exempt=exempt, keys32=key32, keys64=key64, eligible=eligible,
                       group_scores64=(_group_scores(key64, n_group, group_topn)
                                       if grouped else None),
                       topk_group=topk_group if grouped else 0)


def _rel_gaps(v: np.ndarray) -> np.ndarray:
    """(v_j - v_{j+1}) / |v_j| along axis 1 of descending-sorted rows."""
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = (v[:, :-1] - v[:, 1:]) / np.abs(v[:, :-1])
    return gap


def _near_ties(key64, eligible, k, n_group, topk_group, group_topn, grouped):
    """A token is exempt when an exact-key gap that decides its output lies in
    (0, NEAR_TIE_REL): the k-th/(k+1)-th gap (the chosen set), a gap inside the
    top k (the order of its ids), or with grouping the gap at the kept-group
    boundary.  Exact ties (gap 0) are never exempt: both sides see equal keys
    and the index rule decides."""
    T, E = key64.shape
    masked = np.where(eligible, key64, -np.inf)
    srt = -np.sort(-masked, axis=1)
    upto = min(k + 1, E)
    gap = _rel_gaps(srt[:, :upto])
    exempt = np.any((gap > 0) & (gap < NEAR_TIE_REL), axis=1)
    if grouped:
        gs = _group_scores(key64, n_group, group_topn)
        gsrt = -np.sort(-gs, axis=1)
        ggap = _rel_gaps(gsrt[:, topk_group - 1:topk_group + 1])[:, 0]
        exempt |= (ggap > 0) & (ggap < NEAR_TIE_REL)
    return exempt


def _kept_alternatives(res: RouteResult, t: int):
    """Eligibility rows of token t under every kept-group set that near ties at
    the kept-group boundary allow: groups whose exact score lies within
    NEAR_TIE_REL (relative) of the topk_group-th best exact score may stand in
    for one another; groups clearly above it are always kept.  The oracle's own
    kept set comes first."""
    yield res.eligible[t]
    if res.group_scores64 is None:
        return
    gs = res.group_scores64[t]
    G = gs.shape[0]
    gsz = res.keys64.shape[1] // G
    edge = -np.sort(-gs)[res.topk_group - 1]
    near = np.abs(gs - edge) <= NEAR_TIE_REL * abs(edge)
    sure = (gs > edge) & ~near
    need = res.topk_group - int(sure.sum())
    for combo in itertools.combinations(np.nonzero(near)[0].tolist(), need):
        kept = sure.copy()
        kept[list(combo)] = True
        yield np.repeat(kept, gsz)


def within_near_ties(res: RouteResult, t: int, ids_row) -> bool:
    """Whether ``ids_row`` is an acceptable top-k for token t of ``res`` given
    its near ties (the rule for exempt tokens).

    Acceptable: k distinct experts, all eligible under one kept-group set that
    the group near ties allow, and for every position j the exact key of
    ids_row[j] within NEAR_TIE_REL (relative) of the exact key of that kept
    set's j-th choice.  A near tie may thus swap two choices or replace the
    k-th choice by an expert whose key is within the tolerance of it; nothing
    else may differ."""
    k = res.ids.shape[1]
    E = res.keys64.shape[1]
    row = np.asarray(ids_row).astype(np.int64).reshape(-1)
    if row.shape[0] != k or np.any(row < 0) or np.any(row >= E) or np.unique(row).size != k:
        return False
    for elig in _kept_alternatives(res, t):
        if not np.all(elig[row]):
            continue
        ref = select_topk(res.keys32[t:t + 1], elig[None, :], k)[0].astype(np.int64)
        a = res.keys64[t, row]
        b = res.keys64[t, ref]
        if np.all(np.abs(a - b) <= NEAR_TIE_REL * np.abs(b)):
            return True
    return False
