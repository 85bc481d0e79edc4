"""Backward of the routing outputs with respect to the router logits.

TEST INFRASTRUCTURE (see the package header): only tests, the smoke check and
the benchmark's CPU baseline use it.

What it follows (page title, section): TransformerEngine Fused Router,
Description -- the fused top-k-with-score-function op and the
scores-for-aux-loss op each have a backward.  The pages print no formula: the
backward is the derivative of the forward (oracle.routing.route, steps 4 and
5) with the selection held fixed -- the top-k choice is piecewise constant in
the logits, so it passes no gradient, and the expert bias, which only enters
the selection, receives none.  Written out by the chain rule, in float64:

  weights  w' = scale * w, with w by score function and order:
    sigmoid:            s_j = sigma(x_{id_j});  w = s, or s / S with S = sum_j s_j
    softmax before top-k: p = softmax_E(x);     w = p_{id}, or p_{id} / S, S = sum_j p_{id_j}
    softmax after top-k:  w = softmax over the k chosen logits
  scores   sigmoid: q = s / sum_E s (s over all experts);  softmax: q = softmax_E(x)

  d/dx of  sum_j g_j w'_j  +  sum_e h_e q_e   (g = grad of the weights, h = grad
  of the scores), returned as a dense [T, E] float64 array.

Alongside the gradient it returns, per element, the sum of the absolute values
of the terms the chain rule adds (|a| * (|b| + |c|) for a term a * (b - c)):
the scale against which a float32 evaluation's rounding error is measured.

Pins: tests/test_oracle_backward.py -- central finite differences of
oracle.routing.route itself (no formula shared with this module), invariants
(outputs that sum to a constant pass no gradient along the all-ones
direction; softmax gradients are shift invariant), the identity
softmax-before-top-k + renorm == softmax-after-top-k, and zero gradient for
experts a token did not choose where the forward never reads them.
"""
from __future__ import annotations

import numpy as np

from .routing import decode_input


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softmax(x):
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def route_backward(logits, logits_dtype: str, ids, grad_weights=None, grad_scores=None,
                   score_fn: str = "softmax", pre_softmax: bool = True, renorm: bool = True,
                   scale: float = 1.0):
    """Gradient of the routing outputs with respect to the logits.

    ``ids`` [T, k]: the forward's choice.  ``grad_weights`` [T, k] (the
    gradient of topk_weights, entry j belonging to ids[:, j]) and/or
    ``grad_scores`` [T, E] (the gradient of the full-E aux-loss scores).
    Returns (grad_logits [T, E], term_scale [T, E]), both float64.
    """
    x = decode_input(logits, logits_dtype)
    T, E = x.shape
    ids = np.asarray(ids, dtype=np.int64)
    k = ids.shape[1]
    grad = np.zeros((T, E))
    mag = np.zeros((T, E))
    rows = np.arange(T)[:, None]

    if grad_weights is not None:
        g = float(scale) * np.asarray(grad_weights, dtype=np.float64).reshape(T, k)
        if score_fn == "sigmoid":
            s = _sigmoid(np.take_along_axis(x, ids, axis=1))          # [T, k]
            if renorm:
                S = s.sum(axis=1, keepdims=True)
                w = s / S
                c = (g * w).sum(axis=1, keepdims=True)
                ds = (g - c) / S                                        # d/ds_j
                ds_mag = (np.abs(g) + np.abs(g * w).sum(axis=1, keepdims=True)) / S
            else:
                ds, ds_mag = g, np.abs(g)
            dsig = s * (1.0 - s)
            np.add.at(grad, (rows, ids), ds * dsig)
            np.add.at(mag, (rows, ids), ds_mag * dsig)
        elif pre_softmax:
            p = _softmax(x)                                             # [T, E]
            ps = np.take_along_axis(p, ids, axis=1)
            if renorm:
                S = ps.sum(axis=1, keepdims=True)
                w = ps / S
                c = (g * w).sum(axis=1, keepdims=True)
                dps = (g - c) / S
                dps_mag = (np.abs(g) + np.abs(g * w).sum(axis=1, keepdims=True)) / S
            else:
                dps, dps_mag = g, np.abs(g)
            dp = np.zeros((T, E))
            dp_mag = np.zeros((T, E))
            np.put_along_axis(dp, ids, dps, axis=1)
            np.put_along_axis(dp_mag, ids, dps_mag, axis=1)
            # softmax Jacobian (transposed): dx = p * (dp - sum_e p_e dp_e)
            c2 = (p * dp).sum(axis=1, keepdims=True)
            grad += p * (dp - c2)
            mag += p * (dp_mag + (p * dp_mag).sum(axis=1, keepdims=True))
        else:
            xs = np.take_along_axis(x, ids, axis=1)
            w = _softmax(xs)                                            # over the k chosen
            c = (w * g).sum(axis=1, keepdims=True)
            np.add.at(grad, (rows, ids), w * (g - c))
            np.add.at(mag, (rows, ids), w * (np.abs(g) + np.abs(w * g).sum(axis=1, keepdims=True)))

    if grad_scores is not None:
        h = np.asarray(grad_scores, dtype=np.float64).reshape(T, E)
        if score_fn == "sigmoid":
            s = _sigmoid(x)
            Z = s.sum(axis=1, keepdims=True)
            q = s / Z
            c = (h * q).sum(axis=1, keepdims=True)
            dsig = s * (1.0 - s)
            grad += dsig * (h - c) / Z
            mag += dsig * (np.abs(h) + np.abs(h * q).sum(axis=1, keepdims=True)) / Z
        else:
            q = _softmax(x)
            c = (h * q).sum(axis=1, keepdims=True)
            grad += q * (h - c)
            mag += q * (np.abs(h) + np.abs(h * q).sum(axis=1, keepdims=True))
    return grad, mag
