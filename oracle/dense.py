"""Dense [T, E] form of the routing outputs.

TEST INFRASTRUCTURE (see the package header): only tests, the smoke check and
the benchmark's CPU baseline use it.

What it follows (page title, section): TransformerEngine Fused Router, I/O
Contract -- fused_topk_with_score_function returns ``probs`` (the expert
selection probabilities) and ``routing_map`` (the expert assignment map), each
[*, num_experts].  The plainest reading of the pair in terms of the top-k
outputs: probs[t, e] = the weight of expert e if token t chose it, else 0;
routing_map[t, e] = whether token t chose expert e.  The values are copied,
not recomputed: probs holds exactly the top-k weights (bf16 weights widened
exactly to float32).

Pins: tests/test_oracle_dense.py -- k set entries per row for distinct ids,
each chosen entry equal to its weight, zeros elsewhere, row sums equal the
weight sums, a hand example, and ids outside [0, E) ignored.
"""
from __future__ import annotations

import numpy as np


def dense_outputs(ids, weights, E: int):
    """ids [T, k] int, weights [T, k] float -> (probs [T, E] float64, routing_map [T, E] bool)."""
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    T, k = ids.shape
    probs = np.zeros((T, E))
    rmap = np.zeros((T, E), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if 0 <= e < E:
                probs[t, e] = w[t, j]
                rmap[t, e] = True
    return probs, rmap
