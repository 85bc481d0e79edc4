"""CPU oracle for MoE top-k expert routing — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy implementations of what the routing hot
path computes, written from the pages' problem statements.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  The HIP library never calls it, and it
shares no code with the HIP library: it does its own bfloat16 decoding and
rounding, its own score functions, selection, permutation and loss.

Precision: float64 everywhere, except the selection decision.  Where floating
point decides an integer (which experts are chosen, which groups are kept) the
oracle takes the decision in float32, the precision the MAX SigmoidTopKRouter
page fixes for the sigmoid scores and the correction bias (its steps 2-3 and the
``correction_bias_dtype`` parameter).  The pages fix no precision for softmax;
float32 is the kernel's, so softmax keys are also decided in float32.  The exact
(float64) scores are kept beside them to measure near-tie gaps.

Modules
-------
routing      score function, bias, grouped top-k, top-k, weights, full scores,
             per-expert counts, near-tie classification
permutation  tile-padded per-expert offsets, expanded->permuted and
             permuted->token maps, per-tile expert map and row limit
aux_loss     load-balancing loss forward and backward
front_end    RMSNorm -> router projection -> top-k on raw logits -> activation
backward     gradient of the routing weights and aux-loss scores w.r.t. logits
dispatch     token rows into permuted (expert) order and the weighted combine back
dense        dense [T, E] probs and routing map from the top-k outputs

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force on tiny inputs or library routines; see
the header of each module for which pin covers which step.
"""
from .routing import (route, RouteResult, decode_input, selection_keys32, exact_keys64,
                      weights_for_ids, within_near_ties)
from .permutation import permute, PermuteResult, max_padded_tokens, max_tiles
from .aux_loss import aux_loss_fwd, aux_loss_bwd
from .front_end import (rmsnorm, front_end_route, bf16_round_bits, FrontEndResult,
                        affinities_for_ids, fp32_sum_near_ties)
from .backward import route_backward
from .dispatch import dispatch, combine
from .dense import dense_outputs

__all__ = [
    "route", "RouteResult", "decode_input", "selection_keys32", "exact_keys64",
    "weights_for_ids", "within_near_ties",
    "permute", "PermuteResult", "max_padded_tokens", "max_tiles",
    "aux_loss_fwd", "aux_loss_bwd",
    "rmsnorm", "front_end_route", "bf16_round_bits", "FrontEndResult", "affinities_for_ids",
    "fp32_sum_near_ties",
    "route_backward", "dispatch", "combine", "dense_outputs",
]
