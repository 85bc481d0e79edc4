"""GPU parity on seeded random routing configurations.

Each case draws, from its own seed, a method (softmax before/after top-k or
sigmoid, grouping with a top-1 or top-2 group score, renormalisation, scale,
an optional bias), shapes (E up to 2048, k up to 64, a ragged T), dtypes
(float32/bfloat16 logits, float32/bfloat16 weights), a tile size, an optional
local-expert shard and the optional full-E scores, and runs moe_route_permute
against the oracle under the usual parity rules.  Configurations outside the
kernels' stated limits (MOE_EUNSUPPORTED) are skipped with the limit named.
A second family draws large T (33 000 to 140 000 tokens: grids of several
rounds of route blocks, scatter blocks serving several route blocks) with
E up to 512 and k up to 16 (`MOE_RANDOM_LARGE_CASES`, 3 by default).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

from test_gpu_route import mr, run_and_check
from workloads import RouteWorkload, route_inputs

pytestmark = pytest.mark.gpu
CASES = int(os.environ.get("MOE_RANDOM_CASES", "48"))


def _config(i: int):
    rng = np.random.default_rng(9000 + i)
    score_fn = str(rng.choice(["softmax", "sigmoid"]))
    pre = bool(rng.integers(2)) if score_fn == "softmax" else False
    if rng.random() < 0.4:
        gsz = int(rng.choice([4, 8, 16, 32, 64]))
        n_group = int(rng.choice([2, 4, 8, 16]))
        while gsz * n_group > 2048:
            n_group //= 2
        E = gsz * n_group
        topk_group = int(rng.integers(1, n_group))
        topn = int(rng.choice([1, 2]))
        kmax = min(64, topk_group * gsz)
    else:
        E = int(rng.choice([8, 16, 24, 32, 60, 64, 96, 100, 128, 160, 256, 384, 512, 1000,
                            1024, 2048]))
        n_group = topk_group = 0
        topn = 2
        kmax = min(64, E)
    k = int(rng.integers(1, kmax + 1))
    T = int(rng.integers(1, max(2, min(2500, 2_000_000 // E))))
    tile = int(rng.choice([1, 2, 4, 8, 16, 64, 256]))
    bias_std = float(rng.choice([0.01, 0.1])) if rng.random() < 0.5 else None
    w = RouteWorkload(name=f"random{i}", seed=9100 + i, T=T, E=E, k=k, score_fn=score_fn,
                      pre_softmax=pre, n_group=n_group, topk_group=topk_group, group_topn=topn,
                      renorm=bool(rng.integers(2)), scale=float(rng.choice([1.0, 2.5])),
                      logits_dtype=str(rng.choice(["f32", "bf16"])),
                      logits_std=float(rng.choice([0.5, 1.0, 2.0, 4.0])), bias_std=bias_std,
                      bias_dtype=str(rng.choice(["f32", "bf16"])), tile=tile)
    off, n_loc = 0, None
    if rng.random() < 0.25 and E > 1:
        off = int(rng.integers(0, E))
        n_loc = int(rng.integers(1, E - off + 1))
    return (w, str(rng.choice(["f32", "bf16"])), bool(rng.random() < 0.3), off, n_loc)


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(i):
    w, wdt, scores, off, n_loc = _config(i)
    logits, bias = route_inputs(w)
    try:
        run_and_check(w, logits, bias, f"random {i}", weights_dtype=wdt, scores=scores,
                      off=off, n_loc=n_loc)
    except mr.MoeError as e:
        if e.status == mr.MOE_EUNSUPPORTED:
            pytest.skip(f"outside the kernels' limits: {e}")
        raise


LARGE_CASES = int(os.environ.get("MOE_RANDOM_LARGE_CASES", "3"))


def _large_config(i: int):
    # T large enough for grids of several rounds of route blocks and for the
    # scatter blocks that serve 2 or 4 route blocks (from 1024 / 2048 route
    # blocks of 64 tokens on); T * E bounded so that the oracle stays fast
    rng = np.random.default_rng(20000 + i)
    score_fn = str(rng.choice(["softmax", "sigmoid"]))
    pre = bool(rng.integers(2)) if score_fn == "softmax" else False
    E = int(rng.choice([64, 128, 160, 256, 384, 512]))
    n_group = topk_group = 0
    topn = 2
    if rng.random() < 0.4 and E in (64, 128, 256, 512):
        n_group = int(rng.choice([2, 4, 8]))
        topk_group = int(rng.integers(1, n_group))
        topn = int(rng.choice([1, 2]))
        kmax = min(16, topk_group * (E // n_group))
    else:
        kmax = min(16, E)
    k = int(rng.integers(1, kmax + 1))
    T = int(rng.integers(33000, min(140000, 40_000_000 // E) + 1))
    bias_std = float(rng.choice([0.01, 0.1])) if rng.random() < 0.5 else None
    w = RouteWorkload(name=f"large{i}", seed=20100 + i, T=T, E=E, k=k, score_fn=score_fn,
                      pre_softmax=pre, n_group=n_group, topk_group=topk_group, group_topn=topn,
                      renorm=bool(rng.integers(2)), scale=float(rng.choice([1.0, 2.5])),
                      logits_dtype=str(rng.choice(["f32", "bf16"])),
                      logits_std=float(rng.choice([0.5, 1.0, 2.0])), bias_std=bias_std,
                      bias_dtype=str(rng.choice(["f32", "bf16"])),
                      tile=int(rng.choice([1, 8, 16, 64, 256])))
    off, n_loc = 0, None
    if rng.random() < 0.25:
        off = int(rng.integers(0, E))
        n_loc = int(rng.integers(1, E - off + 1))
    scores = bool(rng.random() < 0.2) and T * E <= 20_000_000
    return (w, str(rng.choice(["f32", "bf16"])), scores, off, n_loc)


@pytest.mark.parametrize("i", range(LARGE_CASES))
def test_random_large_configuration(i):
    w, wdt, scores, off, n_loc = _large_config(i)
    logits, bias = route_inputs(w)
    try:
        run_and_check(w, logits, bias, f"random large {i}", weights_dtype=wdt, scores=scores,
                      off=off, n_loc=n_loc)
    except mr.MoeError as e:
        if e.status == mr.MOE_EUNSUPPORTED:
            pytest.skip(f"outside the kernels' limits: {e}")
        raise


FE_CASES = int(os.environ.get("MOE_RANDOM_FE_CASES", "24"))


@pytest.mark.parametrize("i", range(FE_CASES))
def test_random_front_end(i):
    # decode front end on random shapes within its limits: T <= 128, H a
    # multiple of 128, E a multiple of 16 up to 512
    from test_gpu_front_end import run_front_end
    from workloads import FRONT_END
    rng = np.random.default_rng(9500 + i)
    T = int(rng.integers(1, 129))
    H = 128 * int(rng.integers(1, 65))
    E = 16 * int(rng.integers(1, 33))
    run_front_end(FRONT_END, T, H, E, seed=9600 + i, act=str(rng.choice(["sigmoid", "softmax"])),
                  dtype=str(rng.choice(["bf16", "f16"])), rbias=bool(rng.integers(2)))


OTHER_CASES = int(os.environ.get("MOE_RANDOM_OTHER_CASES", "16"))


@pytest.mark.parametrize("i", range(OTHER_CASES))
def test_random_backward(i):
    # routing backward (E <= 2048): weight and/or score gradients, every mode
    from test_gpu_route_backward import check_backward
    rng = np.random.default_rng(9700 + i)
    score_fn = str(rng.choice(["softmax", "sigmoid"]))
    E = int(rng.choice([8, 16, 24, 32, 48, 64, 100, 128, 200, 256, 384, 512, 1000, 2048]))
    k = int(rng.integers(1, min(E, 64) + 1))
    w = RouteWorkload(name=f"bwd{i}", seed=9800 + i, T=1, E=E, k=k, score_fn=score_fn,
                      pre_softmax=bool(rng.integers(2)) if score_fn == "softmax" else False,
                      renorm=bool(rng.integers(2)), scale=float(rng.choice([1.0, 2.5])),
                      logits_dtype=str(rng.choice(["f32", "bf16"])),
                      logits_std=float(rng.choice([0.5, 1.0, 3.0])))
    with_w = bool(rng.integers(2))
    with_s = (not with_w) or bool(rng.integers(2))
    T = int(rng.integers(1, 2000))
    check_backward(w, T, 9900 + i, with_w=with_w, with_s=with_s, label=f"random {i}")


@pytest.mark.parametrize("i", range(OTHER_CASES))
def test_random_dense(i):
    from test_gpu_dense import _route, check_dense
    rng = np.random.default_rng(10000 + i)
    E = int(rng.choice([8, 12, 64, 100, 128, 136, 256, 320, 512, 1000, 2048]))
    k = int(rng.integers(1, min(E, 64) + 1))
    T = int(rng.integers(1, 3000))
    ids, wts = _route(T, E, k, 10100 + i)
    probs = bool(rng.integers(2))
    check_dense(ids, wts, E, w_dtype=str(rng.choice(["f32", "bf16"])),
                want_probs=probs, want_map=(not probs) or bool(rng.integers(2)),
                label=f"random {i}")


@pytest.mark.parametrize("i", range(OTHER_CASES))
def test_random_dispatch_combine(i):
    from test_gpu_dispatch import check_combine, check_dispatch
    rng = np.random.default_rng(10200 + i)
    E = int(rng.choice([8, 16, 60, 128, 256]))
    k = int(rng.integers(1, min(E, 16) + 1))
    T = int(rng.integers(1, 600))
    H = int(rng.choice([8, 24, 100, 512, 1024, 2880, 7168]))
    tile = int(rng.choice([1, 4, 8, 16, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    check_dispatch(T, E, k, H, tile, dtype, 10300 + i, label=f"random {i}")
    check_combine(T, E, k, H, tile, dtype, 10400 + i, label=f"random {i}",
                  w_dtype=str(rng.choice(["f32", "bf16"])))
