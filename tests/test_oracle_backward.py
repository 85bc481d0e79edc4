"""Pins of oracle.backward (the gradient of the routing outputs w.r.t. logits).

Nothing here reuses the oracle's backward formulas: the reference for every
gradient is a central finite difference of oracle.routing.route, the forward
pinned by its own tests, evaluated in float64 with the selection held fixed
(the test asserts that the perturbation does not change the chosen ids)."""
import itertools

import numpy as np
import pytest

import oracle

MODES = [("sigmoid", False, True), ("sigmoid", False, False),
         ("softmax", True, True), ("softmax", True, False), ("softmax", False, True)]


def _logits(rng, T, E, std=1.0):
    # well-separated values: a 1e-5 step never changes the selection
    return rng.standard_normal((T, E)) * std


def _objective(x, ids, g, h, score_fn, pre, renorm, scale, k, bias=None):
    r = oracle.route(x, "f64", k, score_fn=score_fn, pre_softmax=pre, renorm=renorm,
                     scale=scale, bias=bias, bias_dtype="f64")
    assert np.array_equal(r.ids, ids), "a finite-difference step changed the selection"
    val = 0.0
    if g is not None:
        val += float((r.weights * g).sum())
    if h is not None:
        val += float((r.scores * h).sum())
    return val


def _fd(x, ids, g, h, score_fn, pre, renorm, scale, k, step=1e-5, bias=None):
    T, E = x.shape
    out = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            xp = x.copy(); xp[t, e] += step
            xm = x.copy(); xm[t, e] -= step
            out[t, e] = (_objective(xp, ids, g, h, score_fn, pre, renorm, scale, k, bias) -
                         _objective(xm, ids, g, h, score_fn, pre, renorm, scale, k, bias)) / (2 * step)
    return out


@pytest.mark.parametrize("score_fn,pre,renorm", MODES)
@pytest.mark.parametrize("with_w,with_s", [(True, False), (False, True), (True, True)])
def test_backward_matches_finite_differences(score_fn, pre, renorm, with_w, with_s):
    rng = np.random.default_rng(11)
    T, E, k, scale = 3, 12, 3, 2.5
    x = _logits(rng, T, E)
    ids = oracle.route(x, "f64", k, score_fn=score_fn, pre_softmax=pre, renorm=renorm,
                       scale=scale).ids
    g = rng.standard_normal((T, k)) if with_w else None
    h = rng.standard_normal((T, E)) if with_s else None
    grad, mag = oracle.route_backward(x, "f64", ids, g, h, score_fn=score_fn, pre_softmax=pre,
                                      renorm=renorm, scale=scale)
    ref = _fd(x, ids, g, h, score_fn, pre, renorm, scale, k)
    assert np.allclose(grad, ref, rtol=1e-6, atol=1e-8), np.abs(grad - ref).max()
    assert np.all(mag >= np.abs(grad) - 1e-15)


def test_backward_ignores_bias_and_grouping():
    # the bias changes which experts are chosen, not the gradient given the choice
    rng = np.random.default_rng(12)
    T, E, k = 2, 16, 4
    x = _logits(rng, T, E)
    bias = rng.standard_normal(E) * 0.3
    r = oracle.route(x, "f64", k, score_fn="sigmoid", renorm=True, scale=2.5, bias=bias,
                     bias_dtype="f64", n_group=4, topk_group=2)
    g = rng.standard_normal((T, k))
    grad, _ = oracle.route_backward(x, "f64", r.ids, g, None, score_fn="sigmoid", renorm=True,
                                    scale=2.5)
    ref = np.zeros((T, E))
    step = 1e-5
    for t, e in itertools.product(range(T), range(E)):
        vals = []
        for d in (step, -step):
            xp = x.copy(); xp[t, e] += d
            rp = oracle.route(xp, "f64", k, score_fn="sigmoid", renorm=True, scale=2.5, bias=bias,
                              bias_dtype="f64", n_group=4, topk_group=2)
            assert np.array_equal(rp.ids, r.ids)
            vals.append(float((rp.weights * g).sum()))
        ref[t, e] = (vals[0] - vals[1]) / (2 * step)
    assert np.allclose(grad, ref, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("score_fn,pre,renorm", [("sigmoid", False, True), ("softmax", True, True),
                                                 ("softmax", False, True)])
def test_constant_sum_outputs_pass_no_uniform_gradient(score_fn, pre, renorm):
    # renormalised weights sum to `scale` and scores sum to 1 whatever the
    # logits: a gradient equal on every entry changes nothing
    rng = np.random.default_rng(13)
    T, E, k = 4, 10, 3
    x = _logits(rng, T, E)
    ids = oracle.route(x, "f64", k, score_fn=score_fn, pre_softmax=pre, renorm=renorm).ids
    grad, _ = oracle.route_backward(x, "f64", ids, np.full((T, k), 0.7), np.full((T, E), -1.3),
                                    score_fn=score_fn, pre_softmax=pre, renorm=renorm, scale=3.0)
    assert np.abs(grad).max() < 1e-12


@pytest.mark.parametrize("pre,renorm", [(True, True), (True, False), (False, True)])
def test_softmax_gradients_are_shift_invariant(pre, renorm):
    # softmax outputs do not change when every logit of a token moves by the
    # same amount: each token's gradient sums to zero
    rng = np.random.default_rng(14)
    T, E, k = 5, 9, 4
    x = _logits(rng, T, E)
    ids = oracle.route(x, "f64", k, score_fn="softmax", pre_softmax=pre, renorm=renorm).ids
    grad, _ = oracle.route_backward(x, "f64", ids, rng.standard_normal((T, k)),
                                    rng.standard_normal((T, E)), score_fn="softmax",
                                    pre_softmax=pre, renorm=renorm, scale=1.7)
    assert np.abs(grad.sum(axis=1)).max() < 1e-12


def test_pre_softmax_renorm_equals_post_softmax():
    # softmax over E restricted to the chosen and renormalised is the softmax
    # of the chosen logits: both orders give the same gradient
    rng = np.random.default_rng(15)
    T, E, k = 6, 11, 3
    x = _logits(rng, T, E)
    ids = oracle.route(x, "f64", k, score_fn="softmax", pre_softmax=True, renorm=True).ids
    g = rng.standard_normal((T, k))
    a, _ = oracle.route_backward(x, "f64", ids, g, None, score_fn="softmax", pre_softmax=True,
                                 renorm=True, scale=1.5)
    b, _ = oracle.route_backward(x, "f64", ids, g, None, score_fn="softmax", pre_softmax=False,
                                 renorm=True, scale=1.5)
    assert np.abs(a - b).max() < 1e-12


@pytest.mark.parametrize("score_fn,pre", [("sigmoid", False), ("softmax", False)])
def test_unchosen_experts_get_no_weight_gradient(score_fn, pre):
    # sigmoid and softmax-after-top-k weights read only the chosen logits
    rng = np.random.default_rng(16)
    T, E, k = 4, 12, 3
    x = _logits(rng, T, E)
    ids = oracle.route(x, "f64", k, score_fn=score_fn, pre_softmax=pre).ids
    grad, _ = oracle.route_backward(x, "f64", ids, rng.standard_normal((T, k)), None,
                                    score_fn=score_fn, pre_softmax=pre, renorm=True)
    chosen = np.zeros((T, E), bool)
    np.put_along_axis(chosen, ids.astype(np.int64), True, axis=1)
    assert np.all(grad[~chosen] == 0.0)
    assert np.all(grad[chosen] != 0.0)


def test_sigmoid_without_renorm_closed_form():
    # w' = scale * sigma(x): d/dx = scale * g * sigma (1 - sigma), by hand
    x = np.array([[0.0, 2.0, -1.0, 0.5]])
    ids = np.array([[1, 3]])
    g = np.array([[1.0, -2.0]])
    grad, _ = oracle.route_backward(x, "f64", ids, g, None, score_fn="sigmoid", renorm=False,
                                    scale=2.0)
    s1, s3 = 1 / (1 + np.exp(-2.0)), 1 / (1 + np.exp(-0.5))
    assert np.allclose(grad, [[0.0, 2.0 * s1 * (1 - s1), 0.0, -4.0 * s3 * (1 - s3)]], rtol=1e-15)


# ---- compact pins for the planted-mistake checks (tests/test_oracle_mutations.py)

def pin_backward_finite_differences():
    rng = np.random.default_rng(21)
    T, E, k, scale = 2, 8, 3, 1.7
    for score_fn, pre, renorm in MODES:
        x = _logits(rng, T, E)
        ids = oracle.route(x, "f64", k, score_fn=score_fn, pre_softmax=pre, renorm=renorm,
                           scale=scale).ids
        g = rng.standard_normal((T, k))
        h = rng.standard_normal((T, E))
        for gg, hh in ((g, None), (None, h)):
            grad, _ = oracle.route_backward(x, "f64", ids, gg, hh, score_fn=score_fn,
                                            pre_softmax=pre, renorm=renorm, scale=scale)
            ref = _fd(x, ids, gg, hh, score_fn, pre, renorm, scale, k)
            assert np.allclose(grad, ref, rtol=1e-6, atol=1e-8), (score_fn, pre, renorm)


def pin_backward_invariants():
    test_sigmoid_without_renorm_closed_form()
    test_pre_softmax_renorm_equals_post_softmax()
    for pre, renorm in [(True, True), (True, False), (False, True)]:
        test_softmax_gradients_are_shift_invariant(pre, renorm)
