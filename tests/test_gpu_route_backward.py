"""GPU parity: moe_route_backward through the C ABI against oracle.route_backward.

The chosen ids come from the oracle's forward (nothing here comes from the HIP
path); the incoming gradients are seeded normals.  Tolerance: the kernel works
in float32; every element is a sum of chain-rule terms a * (b - c) whose
float32 evaluation (a few roundings, sums of at most 2048 terms, ~1 ulp
exp/reciprocal) errs by well under 1e-5 of sum |a| (|b| + |c|), the scale the
oracle returns beside each gradient element.  Elements with no term (experts a
token did not choose, where the forward never reads them) must be exactly 0."""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, to_dev
from workloads import WORKLOADS, route_inputs, with_overrides

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"
RTOL = 1e-5


def _run_backward(w, logits, ids, gw, gs):
    T, E = logits.shape
    args = mr.make_route_args(T, E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                              renorm=w.renorm, scale=w.scale, logits_dtype=w.logits_dtype)
    x = to_dev(logits, w.logits_dtype)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(DEV)
    gw_d = None if gw is None else torch.from_numpy(gw.astype(np.float32)).to(DEV)
    gs_d = None if gs is None else torch.from_numpy(gs.astype(np.float32)).to(DEV)
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    mr.moe_route_backward(args, x, ids_d, gw_d, gs_d, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_backward(w, T, seed, with_w=True, with_s=False, label=""):
    logits, bias = route_inputs(w, T=T, seed=seed)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                     n_group=w.n_group, topk_group=w.topk_group, group_topn=w.group_topn,
                     renorm=w.renorm, scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
    rng = np.random.default_rng(seed + 99)
    gw = rng.standard_normal((T, w.k)).astype(np.float32) if with_w else None
    gs = rng.standard_normal((T, w.E)).astype(np.float32) if with_s else None
    log(f"[gpu] route backward {label}: T={T} E={w.E} k={w.k} {w.score_fn} pre={w.pre_softmax} "
        f"renorm={w.renorm} dtype={w.logits_dtype} grad_w={with_w} grad_s={with_s}")
    got = _run_backward(w, logits, r.ids, gw, gs)
    ref, mag = oracle.route_backward(logits, w.logits_dtype, r.ids, gw, gs, score_fn=w.score_fn,
                                     pre_softmax=w.pre_softmax, renorm=w.renorm, scale=w.scale)
    assert np.all(np.isfinite(got)), label
    assert np.all(got[mag == 0] == 0.0), f"{label}: non-zero gradient where no term exists"
    err = np.abs(got - ref)
    bad = err > RTOL * mag
    assert not bad.any(), (label, int(bad.sum()), float((err / np.maximum(mag, 1e-300)).max()))


def test_backward_deepseek_full_size():
    w = WORKLOADS["deepseek_v3_like"]
    check_backward(w, w.T, w.seed, label="deepseek full")


def test_backward_qwen_full_size_weights_and_scores():
    w = WORKLOADS["qwen_moe_like"]
    check_backward(w, w.T, w.seed, with_w=True, with_s=True, label="qwen full")


@pytest.mark.parametrize("name", ["tiny_softmax_post", "mixtral_like"])
def test_backward_small_workloads(name):
    w = WORKLOADS[name]
    check_backward(w, w.T, w.seed, with_w=True, with_s=True, label=name)


@pytest.mark.parametrize("score_fn,pre,renorm", [("sigmoid", False, True), ("sigmoid", False, False),
                                                 ("softmax", True, True), ("softmax", True, False),
                                                 ("softmax", False, True)])
@pytest.mark.parametrize("E,k,T,dtype", [(16, 4, 1, "f32"), (64, 6, 257, "bf16"),
                                         (80, 8, 130, "f32"), (65, 5, 63, "bf16"),
                                         (256, 8, 4097, "bf16"), (512, 16, 300, "f32"),
                                         (8, 8, 33, "f32"), (128, 16, 515, "bf16"),
                                         (120, 12, 77, "f32"), (128, 17, 64, "bf16"),
                                         (1000, 6, 77, "bf16"), (1024, 8, 301, "bf16"),
                                         (2048, 16, 129, "f32")])
def test_backward_modes_and_shapes(score_fn, pre, renorm, E, k, T, dtype):
    base = WORKLOADS["mixtral_like"]
    w = with_overrides(base, E=E, k=k, score_fn=score_fn, pre_softmax=pre, renorm=renorm,
                       scale=2.5, logits_dtype=dtype, n_group=0, topk_group=0)
    check_backward(w, T, seed=3000 + E + k + T, with_w=True, with_s=(E % 2 == 0),
                   label=f"{score_fn}/{pre}/{renorm} E={E}")


def test_backward_scores_only():
    # (T = 0 is a host-side no-op, covered by the host validation tests)
    w = WORKLOADS["qwen_moe_like"]
    check_backward(w, 999, seed=5, with_w=False, with_s=True, label="scores only")


def test_backward_deterministic():
    w = WORKLOADS["deepseek_v3_like"]
    logits, bias = route_inputs(w, T=2048, seed=7)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn, n_group=w.n_group,
                     topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                     scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
    gw = np.random.default_rng(8).standard_normal((2048, w.k)).astype(np.float32)
    a = _run_backward(w, logits, r.ids, gw, None)
    b = _run_backward(w, logits, r.ids, gw, None)
    assert np.array_equal(a, b)


# Weight gradients alone (no score gradient) for the score functions whose
# weights read only the chosen logits: every other element must be exactly 0.
# E a multiple of 64 up to 512, ragged T, both logit types.
@pytest.mark.parametrize("score_fn,pre,renorm", [("sigmoid", False, True), ("sigmoid", False, False),
                                                 ("softmax", False, True)])
@pytest.mark.parametrize("E,k,T,dtype", [(64, 1, 5, "f32"), (64, 16, 301, "bf16"),
                                         (128, 8, 1000, "bf16"), (256, 8, 4099, "f32"),
                                         (256, 16, 65, "bf16"), (512, 12, 333, "f32")])
def test_backward_weights_only(score_fn, pre, renorm, E, k, T, dtype):
    base = WORKLOADS["mixtral_like"]
    w = with_overrides(base, E=E, k=k, score_fn=score_fn, pre_softmax=pre, renorm=renorm,
                       scale=2.5, logits_dtype=dtype, n_group=0, topk_group=0)
    check_backward(w, T, seed=4000 + E + k + T, with_w=True, with_s=False,
                   label=f"weights only {score_fn}/{renorm} E={E} k={k}")


def _backward_given_ids(w, logits, ids_gpu, gw_gpu, ids_ref, gw_ref, label):
    got = _run_backward(w, logits, ids_gpu, gw_gpu, None)
    ref, mag = oracle.route_backward(logits, w.logits_dtype, ids_ref, gw_ref, None,
                                     score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                                     renorm=w.renorm, scale=w.scale)
    assert np.all(np.isfinite(got)), label
    assert np.all(got[mag == 0] == 0.0), label
    bad = np.abs(got - ref) > RTOL * mag
    assert not bad.any(), (label, int(bad.sum()))


@pytest.mark.parametrize("score_fn,pre", [("sigmoid", False), ("softmax", False), ("softmax", True)])
def test_backward_foreign_ids(score_fn, pre):
    # ids outside [0, E) contribute nothing, as if that choice were absent
    w = with_overrides(WORKLOADS["deepseek_v3_like"], score_fn=score_fn, pre_softmax=pre,
                       n_group=0, topk_group=0, bias_std=None)
    T = 515
    logits, _ = route_inputs(w, T=T, seed=21)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                     renorm=w.renorm, scale=w.scale)
    gw = np.random.default_rng(22).standard_normal((T, w.k)).astype(np.float32)
    ids = r.ids.astype(np.int64).copy()
    ids[:, 2] = -1
    ids[:, 5] = w.E
    keep = [j for j in range(w.k) if j not in (2, 5)]
    _backward_given_ids(w, logits, ids, gw, ids[:, keep], gw[:, keep], f"{score_fn}/{pre} foreign")
