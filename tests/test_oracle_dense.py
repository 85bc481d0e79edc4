"""Pins of oracle.dense (dense [T, E] probs and routing map).  Routes come from
oracle.route, pinned by its own tests."""
import numpy as np

import oracle


def pin_dense_structure():
    rng = np.random.default_rng(31)
    T, E, k = 50, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, "f32", k, score_fn="sigmoid", renorm=True, scale=2.5)
    probs, rmap = oracle.dense_outputs(r.ids, r.weights, E)
    assert np.array_equal(rmap.sum(axis=1), np.full(T, k))          # distinct ids
    for t in range(T):
        for j in range(k):
            assert rmap[t, r.ids[t, j]] and probs[t, r.ids[t, j]] == r.weights[t, j]
    assert np.all(probs[~rmap] == 0.0)
    assert np.allclose(probs.sum(axis=1), r.weights.sum(axis=1), rtol=1e-15)
    assert np.allclose(probs.sum(axis=1), 2.5, rtol=1e-12)         # renorm x scale


def pin_dense_example():
    ids = np.array([[2, 0], [1, 7], [-1, 1]])            # 7 and -1 are outside E = 3
    probs, rmap = oracle.dense_outputs(ids, np.array([[0.75, 0.25], [1.0, 9.0], [5.0, 0.5]]), 3)
    assert np.array_equal(probs, [[0.25, 0.0, 0.75], [0.0, 1.0, 0.0], [0.0, 0.5, 0.0]])
    assert np.array_equal(rmap, [[True, False, True], [False, True, False], [False, True, False]])


def test_dense_structure():
    pin_dense_structure()


def test_dense_example():
    pin_dense_example()
