"""Pins of the aux-loss and front-end oracles (no GPU)."""
import numpy as np
import scipy.special
import pytest

import oracle
from oracle import front_end as F
from workloads import bf16_bits_from_f32, front_end_inputs, FRONT_END


# ---- aux loss: P10 closed form and linearity, P11 finite differences ------------------

def pin_aux_closed_form():
    for (T, E, k, coeff) in ((64, 8, 2, 1e-2), (1024, 128, 8, 0.3), (12, 4, 1, 1.0)):
        probs = np.full((T, E), 1.0 / E)
        counts = np.full(E, T * k // E)
        assert T * k % E == 0
        loss = oracle.aux_loss_fwd(probs, counts, T, E, k, coeff)
        assert abs(loss - coeff) <= 1e-12 * coeff
    rng = np.random.default_rng(1)
    p = rng.random((50, 6))
    p /= p.sum(1, keepdims=True)
    c = rng.integers(0, 40, size=6)
    base = oracle.aux_loss_fwd(p, c, 50, 6, 2, 0.1)
    assert np.isclose(oracle.aux_loss_fwd(p, c, 50, 6, 2, 0.3), 3 * base, rtol=1e-12)
    assert np.isclose(oracle.aux_loss_fwd(p, 2 * c, 50, 6, 2, 0.1), 2 * base, rtol=1e-12)
    # a shard holding some rows with the global token count: the loss of the
    # whole equals the sum over shards
    a = oracle.aux_loss_fwd(p[:20], c, 50, 6, 2, 0.1)
    b = oracle.aux_loss_fwd(p[20:], c, 50, 6, 2, 0.1)
    assert np.isclose(a + b, base, rtol=1e-12)


def test_p10_aux_closed_form():
    pin_aux_closed_form()


def pin_aux_finite_difference():
    rng = np.random.default_rng(2)
    T, E, k, coeff = 7, 5, 2, 0.05
    p = rng.random((T, E))
    c = rng.integers(0, 10, size=E)
    g = oracle.aux_loss_bwd(c, T, 40, E, k, coeff, grad_loss=1.7)
    h = 1e-6
    for t in range(T):
        for e in range(E):
            pp, pm = p.copy(), p.copy()
            pp[t, e] += h
            pm[t, e] -= h
            fd = (oracle.aux_loss_fwd(pp, c, 40, E, k, coeff)
                  - oracle.aux_loss_fwd(pm, c, 40, E, k, coeff)) / (2 * h)
            assert abs(1.7 * fd - g[t, e]) <= 1e-7 * max(1.0, abs(g[t, e]))
    # the gradient does not depend on probs
    assert np.array_equal(g, oracle.aux_loss_bwd(c, T, 40, E, k, coeff, grad_loss=1.7))


def test_p11_aux_finite_difference():
    pin_aux_finite_difference()


# ---- front end: P12 RMSNorm, P13 identity projection, rounding ------------------------

def _bf16(values):
    return bf16_bits_from_f32(np.asarray(values, np.float32))


def pin_rmsnorm():
    H = 256
    for c in (0.5, 1.0, 3.0, -2.0):
        x = _bf16(np.full((1, H), c))
        g = _bf16(np.ones(H))
        y, bits = oracle.rmsnorm(x, g, 1e-6)
        cval = float(np.float32(c))
        assert np.allclose(y, cval / np.sqrt(cval * cval + 1e-6), rtol=1e-14)
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((4, H)))
    g = _bf16(1 + 0.1 * rng.standard_normal(H))
    y1, b1 = oracle.rmsnorm(x, g, 1e-6)
    # doubling gamma (exact in bf16) doubles the output and adds one to every exponent
    gd = (g.astype(np.uint32) + (1 << 7)).astype(np.uint16)
    y2, b2 = oracle.rmsnorm(x, gd, 1e-6)
    assert np.allclose(y2, 2 * y1, rtol=1e-14)
    nz = y1 != 0
    assert np.array_equal(b2[nz].astype(np.int64) - b1[nz].astype(np.int64),
                          np.full(nz.sum(), 1 << 7))
    # scaling a row leaves the result unchanged when eps = 0
    y3, _ = oracle.rmsnorm(_bf16(4 * F._decode(x, "bf16")), g, 0.0)
    y4, _ = oracle.rmsnorm(x, g, 0.0)
    assert np.allclose(y3, y4, rtol=1e-14)


def test_p12_rmsnorm():
    pin_rmsnorm()


def pin_bf16_rounding():
    """Round-to-nearest-even by brute force: pick the nearer of the two bf16
    neighbours found by stepping the float32 bit pattern; halves go to the
    even pattern."""
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, 2 ** -130]])
    got = oracle.bf16_round_bits(v)
    for val, bits in zip(v, got):
        f = np.float32(val)
        hi = np.uint32(f.view(np.uint32)) >> np.uint32(16)
        cands = []
        for d in (-1, 0, 1, 2):
            b = int(hi) + d
            cand = float((np.uint32(b & 0xFFFF) << np.uint32(16)).view(np.float32))
            if not np.isfinite(cand) or (b & 0xFFFF) != b:
                continue
            cands.append((abs(cand - val), b & 1, b & 0xFFFF))
        cands.sort()
        best = cands[0]
        if cands[1][0] == best[0] and best[1] == 1:
            best = cands[1]
        assert int(bits) == best[2], (val, hex(int(bits)), hex(best[2]))
    # float16 goes through the library conversion and must agree with it
    small = v[np.abs(v) < 6e4][:100]
    b16 = F._round_bits(small, "f16")
    assert np.array_equal(b16, small.astype(np.float16).view(np.uint16))


def test_bf16_rounding():
    pin_bf16_rounding()


def pin_identity_projection():
    rng = np.random.default_rng(5)
    T, H, E, k = 16, 128, 32, 4
    x = _bf16(rng.standard_normal((T, H)))
    g = _bf16(np.ones(H))
    _, normed = oracle.rmsnorm(x, g, 1e-6)
    W = np.zeros((H, E), np.float32)
    W[np.arange(E), np.arange(E)] = 1.0
    res = oracle.front_end_route(normed, _bf16(W), k, act="sigmoid")
    feat = F._decode(normed, "bf16")[:, :E]
    assert np.array_equal(res.logits, feat)
    top = np.argsort(-feat, axis=1, kind="stable")[:, :k]
    assert np.array_equal(res.ids, top)
    aff = F._decode(res.affinities, "bf16")
    sel = 1 / (1 + np.exp(-np.take_along_axis(feat, top, 1)))
    assert np.allclose(np.take_along_axis(aff, top, 1), sel, rtol=2 ** -8)
    mask = np.ones_like(aff, bool)
    np.put_along_axis(mask, top, False, 1)
    assert np.all(res.affinities[mask] == 0)
    # softmax activation: the chosen affinities sum to one (to bf16 rounding)
    rs = oracle.front_end_route(normed, _bf16(W), k, act="softmax")
    assert np.allclose(F._decode(rs.affinities, "bf16").sum(1), 1.0, atol=4 * 2 ** -8)
    # a router bias enters the logits: a large bias on one expert selects it first
    rb = np.zeros(E, np.float32)
    rb[E - 1] = 100.0
    r2 = oracle.front_end_route(normed, _bf16(W), k, act="sigmoid", router_bias=_bf16(rb))
    assert np.all(r2.ids[:, 0] == E - 1)


def test_p13_identity_projection():
    pin_identity_projection()


def pin_affinities_for_ids():
    rng = np.random.default_rng(6)
    T, E, k = 24, 20, 5
    z = rng.standard_normal((T, E)) * 2.0
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])       # not the top-k
    sel = np.take_along_axis(z, ids, 1)
    a = F.affinities_for_ids(z, ids, "sigmoid")
    assert np.allclose(np.take_along_axis(a, ids, 1), scipy.special.expit(sel), rtol=1e-12)
    mask = np.ones_like(a, bool)
    np.put_along_axis(mask, ids, False, 1)
    assert np.all(a[mask] == 0.0)
    b = F.affinities_for_ids(z, ids, "softmax")
    assert np.allclose(np.take_along_axis(b, ids, 1), scipy.special.softmax(sel, axis=1),
                       rtol=1e-12)
    assert np.all(b[mask] == 0.0)
    # the order the ids are listed in does not matter
    assert np.array_equal(F.affinities_for_ids(z, ids[:, ::-1], "sigmoid"), a)
    # at the routed ids they are the routing's affinities
    hidden, gamma, W, _ = front_end_inputs(FRONT_END, T=4, H=256, E=32)
    _, normed = oracle.rmsnorm(hidden, gamma, FRONT_END.eps)
    res = oracle.front_end_route(normed, W, 4, act="softmax")
    assert np.array_equal(F.affinities_for_ids(res.logits, res.ids, "softmax"), res.affinities64)


def test_affinities_for_ids():
    pin_affinities_for_ids()


def pin_fp32_sum_near_ties():
    # identity projection: z = normed[:, :E], sum |normed * W| = |z|, so the
    # bound of a logit is depth * 2^-24 * |z|; gaps on either side of the sum of
    # two neighbouring bounds
    depth = 64
    b = depth * 2.0 ** -24
    rows = np.array([[1.0, 0.5, 0.25, 0.125],           # wide gaps: decided
                      [1.0, 1.0 - 1.5 * b, 0.25, 0.1],    # 1st/2nd gap < b(1) + b(~1)
                      [1.0, 0.5, 0.5 - 0.75 * b, 0.1],    # k-th/(k+1)-th gap (k = 2)
                      [1.0, 0.5, 0.25, 0.25 - 0.4 * b]])  # (k+1)/(k+2): decides nothing
    res = F.FrontEndResult(logits=rows, abs_products=np.abs(rows), ids=None, affinities=None,
                           affinities64=None)
    ex, bound, zs, bs = F.fp32_sum_near_ties(res, 2, depth)
    assert ex.tolist() == [False, True, True, False]
    assert np.allclose(bound, b * np.abs(rows))
    assert np.array_equal(zs[:, 0], rows[:, 0]) and np.all(np.diff(zs, axis=1) <= 0)
    # a deeper sum widens the bound: the first row is decided only while its
    # smallest deciding gap (0.25) exceeds the two bounds (0.75 * b)
    ex2, *_ = F.fp32_sum_near_ties(res, 2, int(0.25 / (0.75 * 2.0 ** -24)) + 1)
    assert ex2[0]


def test_fp32_sum_near_ties():
    pin_fp32_sum_near_ties()


def test_front_end_workload_shapes():
    hidden, gamma, W, rb = front_end_inputs(FRONT_END, T=8)
    assert hidden.shape == (8, 7168) and W.shape == (7168, 256) and rb is None
    _, normed = oracle.rmsnorm(hidden, gamma, FRONT_END.eps)
    res = oracle.front_end_route(normed, W, FRONT_END.k)
    assert res.ids.shape == (8, 8)
    assert np.count_nonzero(res.affinities) <= 8 * 8
