"""Pins of the routing oracle against closed forms, invariants, library routines
and brute-force enumeration (no GPU).

Each pin is a plain function so that tests/test_oracle_mutations.py can run it
against deliberately broken copies of the oracle.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import routing as R
from workloads import (WORKLOADS, route_inputs, tie_heavy_logits, constant_logits,
                       bf16_bits_from_f32)


def _route_w(w, T=None, **over):
    logits, bias = route_inputs(w, T=T)
    kw = dict(k=w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax, n_group=w.n_group,
              topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
              scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
    kw.update(over)
    return oracle.route(logits, w.logits_dtype, **kw), logits, bias


# ---- P1: renormalised weights sum to the routed scaling factor -------------------

def pin_weights_sum_to_scale():
    for w in WORKLOADS.values():
        res, _, _ = _route_w(w, T=512)
        s = res.weights.sum(axis=1)
        assert np.allclose(s, w.scale, rtol=1e-6, atol=0), (w.name, s[:4])


def test_p1_weights_sum_to_scale():
    pin_weights_sum_to_scale()


# ---- P2: sigmoid + correction bias --------------------------------------------------

def pin_sigmoid_bias_semantics():
    rng = np.random.default_rng(11)
    T, E, k, scale = 64, 32, 4, 2.5
    x = rng.standard_normal((T, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.05).astype(np.float32)
    res = oracle.route(x, "f32", k, score_fn="sigmoid", renorm=True, scale=scale, bias=b)
    # (a) weights are the unbiased sigmoid of the chosen logits, renormalised, scaled
    s = scipy.special.expit(x.astype(np.float64))
    sel = np.take_along_axis(s, res.ids.astype(np.int64), axis=1)
    assert np.allclose(res.weights, scale * sel / sel.sum(1, keepdims=True), rtol=1e-12)
    # (b) a common shift of every bias changes nothing (0.25 keeps float32 sums exact here)
    res2 = oracle.route(x, "f32", k, score_fn="sigmoid", renorm=True, scale=scale,
                        bias=b + np.float32(0.25))
    same = ~(res.exempt | res2.exempt)
    assert np.array_equal(res.ids[same], res2.ids[same])
    assert np.allclose(res.weights[same], res2.weights[same], rtol=1e-12)
    # (c) zero bias: plain top-k of the logits (the sigmoid is increasing)
    res0 = oracle.route(x, "f32", k, score_fn="sigmoid", renorm=False, scale=1.0,
                        bias=np.zeros(E, np.float32))
    top = np.argsort(-x, axis=1, kind="stable")[:, :k]
    assert np.array_equal(res0.ids, top)
    assert np.allclose(res0.weights, np.take_along_axis(s, top, axis=1), rtol=1e-12)
    # (d) the bias reaches the weights only through the ids: a bias that moves
    # selection yields the weights of the new ids, still unbiased
    big = np.zeros(E, np.float32)
    big[E - 1] = 10.0
    resb = oracle.route(x, "f32", k, score_fn="sigmoid", renorm=False, scale=1.0, bias=big)
    assert np.all(resb.ids[:, 0] == E - 1)
    assert np.allclose(resb.weights[:, 0], s[:, E - 1], rtol=1e-12)
    # keys are the float32 sum of the float32 sigmoid and the bias
    ref_keys = (scipy.special.expit(x).astype(np.float32) + b).astype(np.float32)
    assert np.max(np.abs(res.keys32 - ref_keys)) <= 2 * np.finfo(np.float32).eps


def test_p2_sigmoid_bias_semantics():
    pin_sigmoid_bias_semantics()


# ---- P3: brute force over every k-subset (and every kept-group subset) --------------

def _dominates(keys, a, b):
    return keys[a] > keys[b] or (keys[a] == keys[b] and a < b)


def _brute_force_token(keys, k, n_group, topk_group, group_topn):
    """Exhaustive search: return (kept groups, chosen set, chosen order)."""
    E = keys.size
    eligible = list(range(E))
    kept = None
    if n_group > 1 and 0 < topk_group < n_group:
        gsz = E // n_group
        # group score: the largest sum over every group_topn-subset of the group
        gscore = []
        for g in range(n_group):
            members = range(g * gsz, (g + 1) * gsz)
            best = max(sum(float(keys[i]) for i in c)
                       for c in itertools.combinations(members, group_topn))
            gscore.append(np.float32(best))
        gscore = np.array(gscore, np.float32)
        winners = [G for G in itertools.combinations(range(n_group), topk_group)
                   if all(_dominates(gscore, g, h) for g in G for h in range(n_group) if h not in G)]
        assert len(winners) == 1
        kept = set(winners[0])
        eligible = [e for e in range(E) if e // gsz in kept]
    sets = [S for S in itertools.combinations(eligible, k)
            if all(_dominates(keys, i, j) for i in S for j in eligible if j not in S)]
    assert len(sets) == 1
    S = sets[0]
    orders = [P for P in itertools.permutations(S)
              if all(_dominates(keys, P[i], P[i + 1]) for i in range(k - 1))]
    assert len(orders) == 1
    return kept, set(S), list(orders[0])


def pin_brute_force(seed=0, T=16):
    for E, k, n_group in itertools.product((4, 8, 16), (1, 2, 3), (1, 2, 4)):
        if E % n_group:
            continue
        gsz = E // n_group
        for topk_group in range(0, n_group + 1):
            for group_topn in (1, 2):
                if group_topn > gsz:
                    continue
                grouped = n_group > 1 and 0 < topk_group < n_group
                if grouped and k > topk_group * gsz:
                    continue
                x = tie_heavy_logits(T, E, seed=seed + 97 * E + 13 * k + n_group)
                res = oracle.route(x, "f32", k, score_fn="softmax", pre_softmax=False,
                                   n_group=n_group, topk_group=topk_group,
                                   group_topn=group_topn)
                for t in range(T):
                    _, S, order = _brute_force_token(x[t], k, n_group, topk_group, group_topn)
                    assert set(res.ids[t].tolist()) == S, (E, k, n_group, topk_group, t)
                    assert res.ids[t].tolist() == order, (E, k, n_group, topk_group, t)


def test_p3_brute_force_tiny():
    pin_brute_force()


# ---- P4: pre-softmax + renorm is the post-softmax result ----------------------------

def pin_pre_renorm_equals_post():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((256, 16)).astype(np.float32)
    a = oracle.route(x, "f32", 4, score_fn="softmax", pre_softmax=True, renorm=True)
    b = oracle.route(x, "f32", 4, score_fn="softmax", pre_softmax=False, renorm=True)
    ok = ~(a.exempt | b.exempt)
    assert np.array_equal(a.ids[ok], b.ids[ok])
    assert np.allclose(a.weights, b.weights, rtol=1e-12, atol=0)


def test_p4_pre_renorm_equals_post():
    pin_pre_renorm_equals_post()


# ---- P5: special cases ------------------------------------------------------------------

def pin_special_cases():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 8)).astype(np.float32)
    # k = E: every expert is chosen, the pre-softmax weights are the full softmax
    res = oracle.route(x, "f32", 8, score_fn="softmax", pre_softmax=True, renorm=False)
    assert all(sorted(r.tolist()) == list(range(8)) for r in res.ids)
    full = scipy.special.softmax(x.astype(np.float64), axis=1)
    assert np.allclose(res.weights, np.take_along_axis(full, res.ids.astype(np.int64), 1),
                       rtol=1e-12)
    assert np.allclose(res.scores, full, rtol=1e-12)
    # constant logits: ids 0..k-1 for every token, equal weights scale/k
    for score_fn, pre in (("softmax", True), ("softmax", False), ("sigmoid", False)):
        c = constant_logits(20, 8)
        r = oracle.route(c, "f32", 3, score_fn=score_fn, pre_softmax=pre, renorm=True, scale=1.5)
        assert np.all(r.ids == np.arange(3)[None, :])
        assert np.allclose(r.weights, 0.5, rtol=1e-12)
        assert np.array_equal(r.counts, np.array([20, 20, 20, 0, 0, 0, 0, 0]))


def test_p5_special_cases():
    pin_special_cases()


# ---- P6: grouping degenerates to no grouping ------------------------------------------

def pin_grouping_reductions():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((128, 32)).astype(np.float32)
    b = (rng.standard_normal(32) * 0.01).astype(np.float32)
    base = oracle.route(x, "f32", 6, score_fn="sigmoid", bias=b, scale=2.0)
    for n_group, topk_group in ((1, 1), (4, 4), (8, 8), (4, 0), (0, 0)):
        r = oracle.route(x, "f32", 6, score_fn="sigmoid", bias=b, scale=2.0,
                         n_group=n_group, topk_group=topk_group)
        assert np.array_equal(r.ids, base.ids)
        assert np.array_equal(r.weights, base.weights)
    # keeping fewer groups restricts the ids to the kept groups' experts
    r = oracle.route(x, "f32", 6, score_fn="sigmoid", bias=b, n_group=4, topk_group=2)
    groups = r.ids // 8
    assert all(len(set(g.tolist())) <= 2 for g in groups)


def test_p6_grouping_reductions():
    pin_grouping_reductions()


# ---- full-E scores, counts and the decode of stored inputs -------------------------------

def pin_scores_counts_decode():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 16)).astype(np.float32)
    r = oracle.route(x, "f32", 4, score_fn="softmax", pre_softmax=True)
    assert np.allclose(r.scores, scipy.special.softmax(x.astype(np.float64), axis=1), rtol=1e-12)
    assert r.counts.sum() == 64 * 4
    assert np.array_equal(r.counts, np.bincount(r.ids.ravel(), minlength=16))
    rs = oracle.route(x, "f32", 4, score_fn="sigmoid")
    s = scipy.special.expit(x.astype(np.float64))
    assert np.allclose(rs.scores, s / s.sum(1, keepdims=True), rtol=1e-12)
    # bf16 inputs decode to the float32 value of the upper 16 bits
    bits = bf16_bits_from_f32(x)
    dec = R.decode_input(bits, "bf16")
    assert np.all(np.abs(dec - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(R.decode_input(np.array([0x3F80, 0xC000, 0x0000], np.uint16), "bf16"),
                          np.array([1.0, -2.0, 0.0]))


def test_scores_counts_decode():
    pin_scores_counts_decode()


# ---- near-tie classification ----------------------------------------------------------------
# The parity rule: a token whose exact-key gap at a deciding position -- the
# k-th/(k+1)-th gap, a gap inside the top k, or with grouping the gap at the
# kept-group boundary -- lies in (0, 1e-6) relative is exempt; exact ties never
# are.  With softmax after top-k the key is the float32 logit itself, so the
# gaps below are exact: u = 2**-24 is the float32 spacing just below 1, a gap of
# 15u (8.9e-7) is inside the window and 18u (1.07e-6) is outside it.

U = 2.0 ** -24
IN, OUT = 15 * U, 18 * U


def _post(x, k, **kw):
    return oracle.route(np.asarray(x, np.float32), "f32", k, score_fn="softmax",
                        pre_softmax=False, **kw)


def pin_near_tie_classification():
    assert IN < R.NEAR_TIE_REL < OUT
    rows = [
        ([3.0, 1.0, 1.0 - IN, -1.0, -2.0, -3.0], True),    # k-th/(k+1)-th gap inside
        ([3.0, 1.0, 1.0 - OUT, -1.0, -2.0, -3.0], False),  # ... just outside
        ([1.0, 1.0 - IN, -1.0, -2.0, -3.0, -4.0], True),   # gap inside the top k
        ([1.0, 1.0 - OUT, -1.0, -2.0, -3.0, -4.0], False),
        ([3.0, 2.0, 1.0, 1.0 - IN, -2.0, -3.0], False),    # (k+1)/(k+2): decides nothing
        ([3.0, 1.0, 1.0, -1.0, -2.0, -3.0], False),        # exact tie: index rule
        ([1.0 - IN, 3.0, -1.0, 1.0, -2.0, -3.0], True),    # order of the row is irrelevant
    ]
    r = _post([x for x, _ in rows], 2)
    assert r.exempt.tolist() == [e for _, e in rows], r.exempt.tolist()
    assert r.ids[5].tolist() == [0, 1]
    # grouped (3 groups of 2, keep 1, top-2-sum score): the group gap at the
    # boundary decides; expert gaps are measured among kept experts only
    g = [
        ([1.0, 1.0, 1.0, 1.0 - 2 * IN, -3.0, -3.0], True),   # group scores 2 vs 2 - 30u: rel 15u
        ([1.0, 1.0, 1.0, 1.0 - 2 * OUT, -3.0, -3.0], False),
        ([3.0, 3.0, 1.0, 1.0 - 2 * IN, 1.0, 1.0], False),    # near tie below the boundary
        ([0.5, 0.5, 0.0, 0.0, 0.5 - IN / 2, -1.0], False),   # kept group 0; the near-tie
                                                             # partner lies in a dropped group
    ]
    r = _post([x for x, _ in g], 2, n_group=3, topk_group=1, group_topn=2)
    assert r.exempt.tolist() == [e for _, e in g], r.exempt.tolist()
    # k-th/(k+1)-th near tie between two kept experts (4 groups, keep 2, k = 3)
    x = [2.0, 1.9, 1.0, 1.0 - IN, -5.0, -5.0, -5.0, -5.0]
    r = _post([x, [2.0, 1.9, 1.0, 1.0 - OUT, -5.0, -5.0, -5.0, -5.0]], 3, n_group=4,
              topk_group=2, group_topn=1)
    assert r.exempt.tolist() == [True, False]


def test_near_tie_classification():
    pin_near_tie_classification()


def pin_within_near_ties():
    W = R.within_near_ties
    # every token of seeded runs accepts the oracle's own ids
    for w in WORKLOADS.values():
        res, _, _ = _route_w(w, T=128)
        assert all(W(res, t, res.ids[t]) for t in range(128)), w.name
    # ungrouped: a near tie at the k-th position may swap in the (k+1)-th expert
    r = _post([[3.0, 1.0, 1.0 - IN, -1.0, -2.0, -3.0],
               [3.0, 1.0, 1.0 - OUT, -1.0, -2.0, -3.0]], 2)
    assert W(r, 0, [0, 1]) and W(r, 0, [0, 2])
    assert not W(r, 0, [2, 0])                      # but not reorder far keys
    assert not W(r, 0, [0, 3])                      # nor take a far lower expert
    assert not W(r, 1, [0, 2])                      # an 18-ulp gap decides
    assert not W(r, 0, [0, 0]) and not W(r, 0, [0, 6]) and not W(r, 0, [0, -1])
    assert not W(r, 0, [0, 1, 2])
    # a near tie inside the top k may swap the two
    r = _post([[1.0, 1.0 - IN, -1.0, -2.0], [1.0, 1.0 - OUT, -1.0, -2.0]], 2)
    assert W(r, 0, [1, 0]) and not W(r, 1, [1, 0])
    # grouped: near-tied groups at the boundary may stand in for each other
    r = _post([[1.0, 1.0, 1.0, 1.0 - 2 * IN, -3.0, -3.0],
               [1.0, 1.0, 1.0, 1.0 - 2 * OUT, -3.0, -3.0]], 2,
              n_group=3, topk_group=1, group_topn=2)
    assert r.ids[0].tolist() == [0, 1]
    assert W(r, 0, [2, 3]) and not W(r, 1, [2, 3])
    assert not W(r, 0, [2, 0])                      # experts of two groups: no kept set
    assert not W(r, 0, [4, 5])                      # a group far below the boundary
    # 4 groups keep 2: one sure group and two near-tied candidates for the other slot
    x = np.array([[5.0, 5.0, 1.0, 1.0, 1.0, 1.0 - 2 * IN, -9.0, -9.0]], np.float32)
    r = _post(x, 3, n_group=4, topk_group=2, group_topn=2)
    assert r.ids[0].tolist() == [0, 1, 2]
    assert W(r, 0, [0, 1, 4]) and not W(r, 0, [0, 1, 6]) and not W(r, 0, [2, 3, 4])


def test_within_near_ties():
    pin_within_near_ties()


def pin_weights_for_ids():
    rng = np.random.default_rng(21)
    T, E, k = 32, 12, 4
    x = rng.standard_normal((T, E)).astype(np.float32)
    x64 = x.astype(np.float64)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)   # not the top-k
    sel = np.take_along_axis(x64, ids.astype(np.int64), axis=1)
    sig = scipy.special.expit(sel)
    full = np.take_along_axis(scipy.special.softmax(x64, axis=1), ids.astype(np.int64), axis=1)
    cases = [
        (("sigmoid", False, True, 2.5), 2.5 * sig / sig.sum(1, keepdims=True)),
        (("sigmoid", False, False, 1.0), sig),
        (("softmax", True, False, 1.0), full),
        (("softmax", True, True, 3.0), 3.0 * full / full.sum(1, keepdims=True)),
        (("softmax", False, True, 1.0), scipy.special.softmax(sel, axis=1)),
    ]
    for (fn, pre, ren, sc), want in cases:
        got = R.weights_for_ids(x64, ids, fn, pre, ren, sc)
        assert np.allclose(got, want, rtol=1e-12, atol=0), (fn, pre, ren)
        # listing the ids in another order lists the weights in that order
        perm = ids[:, ::-1]
        assert np.allclose(R.weights_for_ids(x64, perm, fn, pre, ren, sc), got[:, ::-1],
                           rtol=1e-12, atol=0)
    # at the chosen ids they are the routing weights
    for w in WORKLOADS.values():
        res, logits, _ = _route_w(w, T=64)
        got = R.weights_for_ids(R.decode_input(logits, w.logits_dtype), res.ids, w.score_fn,
                                w.pre_softmax, w.renorm, w.scale)
        assert np.allclose(got, res.weights, rtol=1e-12, atol=0), w.name


def test_weights_for_ids():
    pin_weights_for_ids()


def test_workload_shapes_route():
    for w in WORKLOADS.values():
        res, logits, bias = _route_w(w, T=256)
        assert res.ids.shape == (256, w.k) and res.ids.dtype == np.int32
        assert np.all((res.ids >= 0) & (res.ids < w.E))
        assert all(len(set(r.tolist())) == w.k for r in res.ids)


def test_invalid_arguments():
    x = np.zeros((2, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.route(x, "f32", 9)
    with pytest.raises(ValueError):
        oracle.route(x, "f32", 2, n_group=3, topk_group=1)
    with pytest.raises(ValueError):
        oracle.route(x, "f32", 5, n_group=4, topk_group=2)
    with pytest.raises(ValueError):
        oracle.route(np.array([[np.nan] * 8], np.float32), "f32", 2)
