"""Pins of the permutation oracle (no GPU): the FlashInfer Notes invariant,
bookkeeping invariants, and equality with a stable counting sort done by the
library's ``argsort``."""
import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, route_inputs, skewed_logits


def _random_ids(T, E, k, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def _check_invariants(ids, P, tile, off=0, n_loc=None):
    T, k = ids.shape
    n_loc = P.counts.size if n_loc is None else n_loc
    local = (ids >= off) & (ids < off + n_loc)
    # P8: counts, padded segment sizes, totals
    assert P.counts.sum() == local.sum()
    seg = np.diff(P.padded_offsets)
    assert np.array_equal(seg, -(-P.counts // tile) * tile)
    assert P.total == P.padded_offsets[-1] and P.total % tile == 0
    assert P.total <= oracle.max_padded_tokens(T, k, n_loc, tile)
    assert P.num_tiles == P.total // tile <= oracle.max_tiles(T, k, n_loc, tile)
    # P7 (Notes): slot -> token and slot -> tile -> expert agree with the ids
    for t in range(T):
        for j in range(k):
            p = P.e2p[t * k + j]
            if not local[t, j]:
                assert p == -1
                continue
            assert P.p2t[p] == t
            assert P.batch_idx[p // tile] + off == ids[t, j]
            assert p < P.mn_limit[p // tile]
    # e2p is injective onto the non-padding slots; p2t inverts it
    used = P.e2p[P.e2p >= 0]
    assert np.unique(used).size == used.size
    assert np.array_equal(np.sort(used), np.nonzero(P.p2t >= 0)[0])
    # inside every segment tokens ascend, then padding
    for e in range(n_loc):
        s, c = P.padded_offsets[e], P.counts[e]
        toks = P.p2t[s:s + c]
        assert np.all(np.diff(toks) > 0)
        assert np.all(P.p2t[s + c:P.padded_offsets[e + 1]] == -1)
    # every tile's row limit lies inside the tile and covers its valid rows
    for c in range(P.num_tiles):
        lo, hi = c * tile, (c + 1) * tile
        assert lo < P.mn_limit[c] <= hi
        assert np.all(P.p2t[lo:P.mn_limit[c]] >= 0)
        assert np.all(P.p2t[P.mn_limit[c]:hi] == -1)


def pin_permutation_invariants():
    for (T, E, k, tile, seed) in ((37, 8, 2, 4, 1), (100, 16, 3, 8, 2), (64, 5, 5, 1, 3),
                                  (50, 32, 4, 16, 4), (1, 4, 2, 2, 5)):
        ids = _random_ids(T, E, k, seed)
        P = oracle.permute(ids, tile, num_experts=E)
        _check_invariants(ids, P, tile)


def test_p7_p8_invariants():
    pin_permutation_invariants()


def pin_counting_sort():
    """P9: the permutation equals a stable sort of expanded indices by expert
    (``numpy.argsort(kind='stable')``) with each segment padded to the tile."""
    for (T, E, k, tile, seed) in ((200, 8, 2, 8, 7), (300, 16, 4, 4, 8), (128, 32, 8, 16, 9)):
        ids = _random_ids(T, E, k, seed)
        P = oracle.permute(ids, tile, num_experts=E)
        flat = ids.ravel()
        order = np.argsort(flat, kind="stable")          # expanded indices in expert order
        sorted_e = flat[order]
        counts = np.bincount(flat, minlength=E)
        assert np.array_equal(P.counts, counts)
        starts = np.concatenate([[0], np.cumsum(-(-counts // tile) * tile)])
        rank = np.arange(order.size) - np.concatenate([[0], np.cumsum(counts)])[sorted_e]
        slots = starts[sorted_e] + rank
        assert np.array_equal(P.e2p[order], slots)
        assert np.array_equal(P.p2t[slots], order // k)
        # tile = 1: no padding, p2t is exactly the sorted token list
        P1 = oracle.permute(ids, 1, num_experts=E)
        assert np.array_equal(P1.p2t, order // k)


def test_p9_counting_sort():
    pin_counting_sort()


def pin_local_expert_shard():
    ids = _random_ids(60, 16, 4, 11)
    off, n_loc, tile = 4, 8, 4
    P = oracle.permute(ids, tile, local_expert_offset=off, local_num_experts=n_loc)
    _check_invariants(ids, P, tile, off=off, n_loc=n_loc)
    full = oracle.permute(ids, tile, num_experts=16)
    assert np.array_equal(P.counts, full.counts[off:off + n_loc])
    assert np.all(P.batch_idx < n_loc)


def test_local_expert_shard():
    pin_local_expert_shard()


def test_empty_and_degenerate():
    P = oracle.permute(np.zeros((0, 2), np.int32), 8, num_experts=4)
    assert P.total == 0 and P.num_tiles == 0 and P.counts.tolist() == [0, 0, 0, 0]
    assert P.padded_offsets.tolist() == [0] * 5
    # every token on the same k experts: extreme imbalance
    ids = np.tile(np.array([[2, 0]], np.int32), (33, 1))
    P = oracle.permute(ids, 8, num_experts=4)
    assert P.counts.tolist() == [33, 0, 33, 0]
    assert P.padded_offsets.tolist() == [0, 40, 40, 80, 80]
    _check_invariants(ids, P, 8)
    with pytest.raises(ValueError):
        oracle.permute(ids, 6, num_experts=4)


def test_workload_permutations():
    for name in ("tiny_softmax_post", "mixtral_like", "deepseek_v3_like"):
        w = WORKLOADS[name]
        logits, bias = route_inputs(w, T=min(w.T, 300))
        r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn,
                         pre_softmax=w.pre_softmax, n_group=w.n_group,
                         topk_group=w.topk_group, group_topn=w.group_topn,
                         renorm=w.renorm, scale=w.scale, bias=bias)
        P = oracle.permute(r.ids, w.tile, num_experts=w.E)
        _check_invariants(r.ids, P, w.tile)
        assert np.array_equal(P.counts, r.counts)
    x = skewed_logits(500, 8, seed=3)
    r = oracle.route(x, "f32", 2, score_fn="softmax", pre_softmax=True)
    P = oracle.permute(r.ids, 8, num_experts=8)
    assert P.counts[0] >= 450
    _check_invariants(r.ids, P, 8)
