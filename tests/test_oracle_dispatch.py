"""Pins of oracle.dispatch (token dispatch and combine).  The routes and
permutations come from oracle.route / oracle.permute, pinned by their own
tests; nothing here reuses the dispatch module's arithmetic."""
import numpy as np

import oracle
from workloads import bf16_bits_from_f32, f32_from_bf16_bits


def _routed(T=40, E=8, k=2, H=24, tile=4, seed=3, off=0, n_loc=None):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, "f32", k, score_fn="softmax", pre_softmax=True, renorm=True)
    pm = oracle.permute(r.ids, tile, local_expert_offset=off,
                        local_num_experts=E if n_loc is None else n_loc, num_experts=E)
    hidden = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    return r, pm, hidden


def pin_dispatch_rows():
    r, pm, hidden = _routed()
    x = oracle.dispatch(hidden, pm.p2t, pm.total)
    T, k = r.ids.shape
    assert x.shape == (pm.total, hidden.shape[1]) and x.dtype == hidden.dtype
    for p in range(pm.total):
        t = pm.p2t[p]
        if t < 0:
            assert np.all(x[p] == 0)
        else:
            assert np.array_equal(x[p], hidden[t])
    # the slot of every (token, choice) holds that token's row
    for t in range(T):
        for j in range(k):
            assert np.array_equal(x[pm.e2p[t * k + j]], hidden[t])


def pin_combine_inverts_dispatch():
    # identity experts: out[t] = (sum_j w_j) hidden[t] = hidden[t] for renormalised weights
    r, pm, hidden = _routed(T=33, E=16, k=4, H=40, tile=8, seed=4)
    x = oracle.dispatch(hidden, pm.p2t, pm.total)
    out64, bits = oracle.combine(x, "bf16", pm.e2p, r.weights, 33, 4)
    h = f32_from_bf16_bits(hidden).astype(np.float64)
    assert np.allclose(out64, h, rtol=1e-12, atol=1e-12)
    assert np.array_equal(bits, hidden)            # exact sums round back to the inputs


def pin_combine_one_hot_and_linearity():
    r, pm, hidden = _routed(T=20, E=8, k=3, H=16, tile=2, seed=5)
    rng = np.random.default_rng(6)
    y = rng.standard_normal((pm.total, 16)).astype(np.float32)
    T, k = 20, 3
    for j in range(k):
        w = np.zeros((T, k)); w[:, j] = 1.0
        out64, _ = oracle.combine(y, "f32", pm.e2p, w, T, k)
        slots = pm.e2p.reshape(T, k)[:, j]
        assert np.array_equal(out64, y[slots].astype(np.float64))
    w1, w2 = rng.standard_normal((T, k)), rng.standard_normal((T, k))
    a, _ = oracle.combine(y, "f32", pm.e2p, w1, T, k)
    b, _ = oracle.combine(y, "f32", pm.e2p, w2, T, k)
    c, _ = oracle.combine(y, "f32", pm.e2p, 2 * w1 - 3 * w2, T, k)
    assert np.allclose(c, 2 * a - 3 * b, rtol=1e-12, atol=1e-12)


def pin_combine_local_shard_and_example():
    # a choice outside the local expert range (e2p = -1) contributes nothing
    r, pm, hidden = _routed(T=30, E=8, k=2, H=8, tile=4, seed=7, off=2, n_loc=4)
    y = np.ones((max(pm.total, 1), 8), dtype=np.float32)
    out64, _ = oracle.combine(y, "f32", pm.e2p, np.ones((30, 2)), 30, 2)
    local = ((r.ids >= 2) & (r.ids < 6)).sum(axis=1)
    assert np.array_equal(out64, np.repeat(local[:, None].astype(np.float64), 8, axis=1))
    # by hand: two tokens, k = 2, slots [[1, 0], [2, 0]]
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]], dtype=np.float32)
    out64, out32 = oracle.combine(y, "f32", np.array([1, 0, 2, 0]), np.array([[0.5, 2.0], [0.25, -1.0]]), 2, 2)
    assert np.array_equal(out64, [[7.0, 14.0], [24.0, 48.0]])


def test_dispatch_rows():
    pin_dispatch_rows()


def test_combine_inverts_dispatch():
    pin_combine_inverts_dispatch()


def test_combine_one_hot_and_linearity():
    pin_combine_one_hot_and_linearity()


def test_combine_local_shard_and_example():
    pin_combine_local_shard_and_example()
