"""GPU parity: moe_topk_to_dense through the C ABI against oracle.dense_outputs.

ids and weights come from the oracle's forward (nothing here comes from the
HIP path).  The kernel copies values, so probs and routing_map are bit-exact."""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, to_dev
from workloads import WORKLOADS, route_inputs, bf16_bits_from_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"


def check_dense(ids, weights32, E, w_dtype="f32", want_probs=True, want_map=True, label=""):
    T, k = ids.shape
    log(f"[gpu] dense {label}: T={T} E={E} k={k} weights {w_dtype} probs={want_probs} map={want_map}")
    if w_dtype == "bf16":
        bits = bf16_bits_from_f32(weights32)
        w_used = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
        w_dev = to_dev(bits, "bf16")
    else:
        w_used = weights32
        w_dev = to_dev(weights32, "f32")
    probs = torch.full((T, E), -5.0, dtype=torch.float32, device=DEV) if want_probs else None
    rmap = torch.full((T, E), 7, dtype=torch.uint8, device=DEV) if want_map else None
    mr.moe_topk_to_dense(T, E, k, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(DEV), w_dev,
                         mr.MOE_BF16 if w_dtype == "bf16" else mr.MOE_F32, probs, rmap)
    torch.cuda.synchronize()
    ref_p, ref_m = oracle.dense_outputs(ids, w_used.astype(np.float64), E)
    if want_probs:
        got = probs.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref_p.astype(np.float32).view(np.uint32)), label
    if want_map:
        assert np.array_equal(rmap.cpu().numpy(), ref_m.astype(np.uint8)), label


def _route(T, E, k, seed, score_fn="sigmoid"):
    logits = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, "f32", k, score_fn=score_fn, renorm=True, scale=2.5)
    return r.ids, r.weights.astype(np.float32)


def test_dense_full_size():
    w = WORKLOADS["deepseek_v3_like"]
    logits, bias = route_inputs(w)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn, n_group=w.n_group,
                     topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                     scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
    check_dense(r.ids, r.weights.astype(np.float32), w.E, label="deepseek full")


@pytest.mark.parametrize("T,E,k,w_dtype", [(1, 8, 2, "f32"), (33, 8, 8, "bf16"), (300, 64, 6, "f32"),
                                           (257, 100, 5, "f32"), (400, 128, 8, "bf16"),
                                           (999, 256, 8, "f32"), (130, 512, 16, "bf16"),
                                           (77, 384, 64, "f32"), (300, 1000, 8, "f32"),
                                           (257, 1024, 16, "bf16"), (129, 2048, 64, "f32")])
def test_dense_shapes(T, E, k, w_dtype):
    ids, wts = _route(T, E, k, seed=T + E + k)
    check_dense(ids, wts, E, w_dtype=w_dtype, label=f"{T}x{E}")


def test_dense_one_output_and_foreign_ids():
    ids, wts = _route(200, 256, 8, seed=4)
    check_dense(ids, wts, 256, want_map=False, label="probs only")
    check_dense(ids, wts, 256, want_probs=False, label="map only")
    ids = ids.copy()
    ids[::7, 3] = -1                 # ids outside [0, E) are ignored
    ids[::11, 5] = 256
    check_dense(ids, wts, 256, label="foreign ids")


def test_dense_repeated_ids():
    # of choices naming one expert, the last one's weight stays (the oracle's loop order)
    ids, wts = _route(301, 256, 8, seed=6)
    ids = ids.copy()
    ids[::3, 4] = ids[::3, 1]
    ids[::4, 7] = ids[::4, 0]
    check_dense(ids, wts, 256, label="repeated ids")
    ids2, wts2 = _route(150, 128, 8, seed=9)
    ids2 = ids2.copy()
    ids2[:, 6] = ids2[:, 6 - 1]
    check_dense(ids2, wts2, 128, w_dtype="bf16", label="repeated ids E=128")
