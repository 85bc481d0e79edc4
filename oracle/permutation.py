"""Permutation oracle: the dispatch bookkeeping built from the chosen ids.

TEST INFRASTRUCTURE (see the package header).

Sources (page title, section):

* FlashInfer trtllm_gen_routing, Parameters (``tile_tokens_dim``: the token
  tile of the downstream grouped GEMM, a power of two, on which the padding
  outputs depend; ``local_expert_offset`` / ``local_num_experts``: the
  expert-parallel shard), Returns (the result fields: total_num_padded_tokens,
  expanded_idx_to_permuted_idx, permuted_idx_to_token_idx,
  cta_idx_xy_to_batch_idx, cta_idx_xy_to_mn_limit, num_non_exiting_ctas) and
  Notes (a permuted slot p lies in tile p // tile_tokens_dim, whose expert is
  cta_idx_xy_to_batch_idx[tile] + local_expert_offset);
* LMDeploy MoeUtils, Description and I/O Contract (per-expert token offsets).

Readings (listed in the design notes): each expert's segment holds its tokens
in ascending token order, then padding up to a multiple of the tile; padding
slots of permuted_idx_to_token_idx hold -1; expanded index i = t * k + j for
the j-th id of token t; ids outside the local expert range map to -1; the
per-tile row limit is the exclusive end of the tile's valid rows in permuted
space; the number of non-exiting CTAs is the number of tiles.

Pins: tests/test_oracle_permutation.py (the Notes invariant, bookkeeping
invariants, equality with a stable counting sort done by ``numpy.argsort``).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def max_padded_tokens(T: int, k: int, local_num_experts: int, tile: int) -> int:
    """Upper bound on total_num_padded_tokens: every local expert adds < tile pad."""
    return T * k + local_num_experts * (tile - 1)


def max_tiles(T: int, k: int, local_num_experts: int, tile: int) -> int:
    return max_padded_tokens(T, k, local_num_experts, tile) // tile


@dataclass
class PermuteResult:
    counts: np.ndarray           # int64 [E_loc]
    padded_offsets: np.ndarray   # int64 [E_loc + 1]
    total: int                   # total_num_padded_tokens
    num_tiles: int               # num_non_exiting_ctas
    e2p: np.ndarray              # int64 [T*k] expanded_idx_to_permuted_idx
    p2t: np.ndarray              # int64 [total] permuted_idx_to_token_idx
    batch_idx: np.ndarray        # int64 [num_tiles] cta_idx_xy_to_batch_idx
    mn_limit: np.ndarray         # int64 [num_tiles] cta_idx_xy_to_mn_limit


def permute(ids: np.ndarray, tile: int, local_expert_offset: int = 0,
            local_num_experts: int | None = None, num_experts: int | None = None) -> PermuteResult:
    """Build the permutation of expanded (token, slot) pairs into expert order."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim != 2:
        raise ValueError("ids must be [T, k]")
    if tile < 1 or (tile & (tile - 1)):
        raise ValueError("tile_tokens_dim must be a power of two")
    T, k = ids.shape
    if local_num_experts is None:
        if num_experts is None:
            raise ValueError("need local_num_experts or num_experts")
        local_num_experts = num_experts - local_expert_offset
    off, n_loc = local_expert_offset, local_num_experts

    # per-expert counts over the local experts
    counts = np.array([int(np.count_nonzero(ids == off + e)) for e in range(n_loc)],
                      dtype=np.int64)

    # each segment is padded up to a multiple of the tile
    padded = np.zeros(n_loc + 1, dtype=np.int64)
    for e in range(n_loc):
        padded[e + 1] = padded[e] + -(-counts[e] // tile) * tile
    total = int(padded[n_loc])
    num_tiles = total // tile

    # stable scatter: inside a segment, tokens in ascending order
    e2p = np.full(T * k, -1, dtype=np.int64)
    p2t = np.full(total, -1, dtype=np.int64)
    for e in range(n_loc):
        t_idx, j_idx = np.nonzero(ids == off + e)       # row-major: ascending t
        slots = padded[e] + np.arange(t_idx.size, dtype=np.int64)
        e2p[t_idx * k + j_idx] = slots
        p2t[slots] = t_idx

    # per-tile expert (local index) and exclusive end of its valid rows
    batch_idx = np.full(num_tiles, -1, dtype=np.int64)
    mn_limit = np.full(num_tiles, -1, dtype=np.int64)
    for e in range(n_loc):
        start = int(padded[e])
        for i in range(-(-int(counts[e]) // tile)):
            c = start // tile + i
            batch_idx[c] = e
            mn_limit[c] = min(start + (i + 1) * tile, start + int(counts[e]))

    return PermuteResult(counts=counts, padded_offsets=padded, total=total,
                         num_tiles=num_tiles, e2p=e2p, p2t=p2t,
                         batch_idx=batch_idx, mn_limit=mn_limit)
