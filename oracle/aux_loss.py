"""Aux-loss oracle: MoE load-balancing loss, forward and backward.

TEST INFRASTRUCTURE (see the package header).

Source: TransformerEngine Fused Router, Description (FusedAuxLoss computes the
load-balancing loss from probability distributions and tokens-per-expert
counts; forward and backward) and Code Reference / Signature (arguments
probs, tokens_per_expert, total_num_tokens, num_experts, topk, coeff).

The page prints no formula.  Reading (listed in the design notes): the
Switch-style balance loss that uses exactly those arguments,

    loss = coeff * E / (topk * T_tot**2) * sum_e (sum_t probs[t, e]) * c_e,

where ``T_tot = total_num_tokens`` may exceed the rows held locally.  It equals
``coeff`` for uniform probabilities with perfectly balanced counts, which is
what a load-balancing coefficient means.  The backward is the derivative of
that expression with respect to probs: it does not depend on probs.

Pins: tests/test_oracle_aux_loss.py (balanced closed form, linearity, central
finite differences of the float64 forward).
"""
from __future__ import annotations

import numpy as np


def _constant(total_num_tokens: int, num_experts: int, topk: int, coeff: float) -> float:
    return float(coeff) * num_experts / (topk * float(total_num_tokens) ** 2)


def aux_loss_fwd(probs, tokens_per_expert, total_num_tokens: int, num_experts: int,
                 topk: int, coeff: float) -> float:
    p = np.asarray(probs, dtype=np.float64)
    c = np.asarray(tokens_per_expert, dtype=np.float64)
    if p.ndim != 2 or p.shape[1] != num_experts or c.shape != (num_experts,):
        raise ValueError("probs must be [rows, E] and tokens_per_expert [E]")
    column_sums = p.sum(axis=0)
    return _constant(total_num_tokens, num_experts, topk, coeff) * float(np.dot(column_sums, c))


def aux_loss_bwd(tokens_per_expert, rows: int, total_num_tokens: int, num_experts: int,
                 topk: int, coeff: float, grad_loss: float = 1.0) -> np.ndarray:
    c = np.asarray(tokens_per_expert, dtype=np.float64)
    row = float(grad_loss) * _constant(total_num_tokens, num_experts, topk, coeff) * c
    return np.broadcast_to(row, (rows, num_experts)).copy()
