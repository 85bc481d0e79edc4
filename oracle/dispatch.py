"""Token dispatch and combine around the grouped expert GEMM.

TEST INFRASTRUCTURE (see the package header): only tests, the smoke check and
the benchmark's CPU baseline use it.

What it follows (page title, section): Implementation:InternLM Lmdeploy Gemm
MoeUtils, Description -- dispatch sends the input tokens to expert-ordered
buffers by the routing decision, combine brings the expert outputs back into
token order applying the routing scales.  The pages give the names and the
signatures only; the plainest reading in this library's own index maps (the
FlashInfer trtllm_gen_routing Returns: permuted_idx_to_token_idx and
expanded_idx_to_permuted_idx):

  dispatch:  permuted[p, :] = hidden[permuted_idx_to_token_idx[p], :] for the
             slots p < total_num_padded_tokens; a padding slot (-1) is a zero
             row, so a tile's unused rows feed zeros to the expert GEMM.
  combine:   out[t, :] = sum_j topk_weights[t, j] * expert_out[e2p[t k + j], :]
             over the k choices of token t (a choice with e2p = -1, an expert
             outside the local range, contributes nothing); the sum is formed
             exactly (float64) and rounded once to the output dtype.

The routing's bias terms, destination scales and residual of LMDeploy's
combine signature are not followed (no workload uses them).

Pins: tests/test_oracle_dispatch.py -- every routed row is a bit copy of its
token's row and every padding row is zero; the slot of each (token, choice)
holds that token's row; combine of dispatched hidden states with
renormalised weights returns the hidden states; one-hot weights select one
expert row; linearity in the weights; a hand-checked example.
"""
from __future__ import annotations

import numpy as np

from .front_end import bf16_round_bits


def _decode(values, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        hi = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return hi.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def dispatch(hidden, permuted_idx_to_token_idx, total: int) -> np.ndarray:
    """Rows of ``hidden`` [T, H] (any dtype, copied bit for bit) in permuted
    order: [total, H]; padding slots are zero rows."""
    hidden = np.asarray(hidden)
    p2t = np.asarray(permuted_idx_to_token_idx, dtype=np.int64)[:total]
    out = np.zeros((total, hidden.shape[1]), dtype=hidden.dtype)
    routed = p2t >= 0
    out[routed] = hidden[p2t[routed]]
    return out


def combine(expert_out, dtype: str, expanded_idx_to_permuted_idx, topk_weights, T: int, k: int):
    """Token-order sum of the weighted expert output rows.

    ``expert_out`` [rows, H] in ``dtype`` (float32 values or bfloat16 bits);
    ``topk_weights`` [T, k] (float values).  Returns (out_f64 [T, H], out in
    ``dtype``: float32 values or bfloat16 bits, RNE)."""
    y = _decode(expert_out, dtype)
    e2p = np.asarray(expanded_idx_to_permuted_idx, dtype=np.int64).reshape(T, k)
    w = np.asarray(topk_weights, dtype=np.float64).reshape(T, k)
    out = np.zeros((T, y.shape[1]))
    for j in range(k):
        slot = e2p[:, j]
        ok = slot >= 0
        out[ok] += w[ok, j, None] * y[slot[ok]]
    if dtype == "f32":
        return out, out.astype(np.float32)
    return out, bf16_round_bits(out)
