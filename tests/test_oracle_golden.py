"""The oracle against the hand-derived worked examples in tests/golden/ (no GPU)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _route_case(d):
    m = d["method"]
    bias = None if "bias" not in d else np.array(d["bias"], np.float32)
    return oracle.route(np.array(d["logits"], np.float32), "f32", m["k"],
                        score_fn=m["score_fn"], pre_softmax=m["pre_softmax"],
                        n_group=m.get("n_group", 0), topk_group=m.get("topk_group", 0),
                        group_topn=m.get("group_topn", 2), renorm=m["renorm"],
                        scale=m["scale"], bias=bias)


def pin_golden_routing():
    for name in ("softmax_pre_renorm.json", "softmax_post_ties.json", "grouped_sigmoid_bias.json"):
        d = _load(name)
        r = _route_case(d)
        assert r.ids.tolist() == d["ids"], name
        assert np.allclose(r.weights, d["weights"], atol=d["abs_tol"], rtol=0), name
        if "scores" in d:
            assert np.allclose(r.scores, d["scores"], atol=d["abs_tol"], rtol=0), name


def test_golden_routing():
    pin_golden_routing()


def pin_golden_permutation():
    d = _load("permutation_tile4.json")
    P = oracle.permute(np.array(d["ids"], np.int32), d["tile"], num_experts=d["num_experts"])
    assert P.counts.tolist() == d["counts"]
    assert P.padded_offsets.tolist() == d["padded_offsets"]
    assert P.total == d["total"] and P.num_tiles == d["num_tiles"]
    assert P.e2p.tolist() == d["e2p"]
    assert P.p2t.tolist() == d["p2t"]
    assert P.batch_idx.tolist() == d["batch_idx"]
    assert P.mn_limit.tolist() == d["mn_limit"]


def test_golden_permutation():
    pin_golden_permutation()


def pin_golden_aux_loss():
    d = _load("aux_loss_small.json")
    for c in d["cases"]:
        loss = oracle.aux_loss_fwd(np.array(c["probs"]), np.array(c["counts"]),
                                   d["total_num_tokens"], d["num_experts"], d["topk"], d["coeff"])
        assert abs(loss - c["loss"]) <= d["abs_tol"]
        g = oracle.aux_loss_bwd(np.array(c["counts"]), 2, d["total_num_tokens"],
                                d["num_experts"], d["topk"], d["coeff"])
        assert np.allclose(g, np.array([c["grad_row"]] * 2), atol=d["abs_tol"], rtol=0)


def test_golden_aux_loss():
    pin_golden_aux_loss()


def pin_golden_rmsnorm():
    d = _load("rmsnorm_small.json")
    from workloads import bf16_bits_from_f32
    for c in d["cases"]:
        x = bf16_bits_from_f32(np.array(c["hidden"], np.float32))
        g = bf16_bits_from_f32(np.array(c["gamma"], np.float32))
        _, bits = oracle.rmsnorm(x, g, c["eps"])
        assert bits.tolist() == c["normed_bits"]


def test_golden_rmsnorm():
    pin_golden_rmsnorm()
