"""Plant plausible mistakes in copies of the oracle and check that the pins catch
each one (no GPU).  The mistakes live only in throw-away module copies built
from the oracle's source text; the oracle itself is never modified."""
import importlib
import os
import types

import pytest

import oracle
import test_oracle_aux_front as T_AF
import test_oracle_backward as T_B
import test_oracle_dispatch as T_D
import test_oracle_dense as T_X
import test_oracle_golden as T_G
import test_oracle_permutation as T_P
import test_oracle_routing as T_R

ORACLE_DIR = os.path.dirname(oracle.__file__)

PINS = [
    T_R.pin_weights_sum_to_scale, T_R.pin_sigmoid_bias_semantics, T_R.pin_brute_force,
    T_R.pin_pre_renorm_equals_post, T_R.pin_special_cases, T_R.pin_grouping_reductions,
    T_R.pin_scores_counts_decode, T_R.pin_near_tie_classification, T_R.pin_within_near_ties,
    T_R.pin_weights_for_ids,
    T_P.pin_permutation_invariants, T_P.pin_counting_sort, T_P.pin_local_expert_shard,
    T_AF.pin_aux_closed_form, T_AF.pin_aux_finite_difference, T_AF.pin_rmsnorm,
    T_AF.pin_bf16_rounding, T_AF.pin_identity_projection, T_AF.pin_affinities_for_ids,
    T_AF.pin_fp32_sum_near_ties,
    T_G.pin_golden_routing, T_G.pin_golden_permutation, T_G.pin_golden_aux_loss,
    T_G.pin_golden_rmsnorm,
    T_B.pin_backward_finite_differences, T_B.pin_backward_invariants,
    T_D.pin_dispatch_rows, T_D.pin_combine_inverts_dispatch, T_D.pin_combine_one_hot_and_linearity,
    T_D.pin_combine_local_shard_and_example,
    T_X.pin_dense_structure, T_X.pin_dense_example,
]

# (module, text in the oracle, planted replacement, what the mistake is)
MUTATIONS = [
    ("routing", 'order = np.argsort(-masked, axis=1, kind="stable")',
     'order = (E - 1) - np.argsort(-masked[:, ::-1], axis=1, kind="stable")',
     "ties go to the higher expert index"),
    ("routing", "key = key + bias64.astype(np.float32)", "key = key",
     "bias dropped from the selection key"),
    ("routing", "w = w * float(scale)", "w = w",
     "routed scaling factor not applied"),
    ("routing", "        w = 1.0 / (1.0 + np.exp(-xs))\n        if renorm:\n            w = w / w.sum(axis=1, keepdims=True)",
     "        w = 1.0 / (1.0 + np.exp(-xs))",
     "sigmoid weights not renormalised"),
    ("routing", "    w = weights_for_ids(x, ids, score_fn, pre_softmax, renorm, scale)",
     "    w = weights_for_ids(x + (0.0 if b is None else b[None, :]), ids, score_fn, pre_softmax, renorm, scale)",
     "bias leaks into the weights"),
    ("routing", "    for i in range(group_topn):\n", "    for i in range(1):\n",
     "group score is the group max, not the top-n sum"),
    ("routing", 'order = np.argsort(-score, axis=1, kind="stable")',
     'order = (score.shape[1] - 1) - np.argsort(-score[:, ::-1], axis=1, kind="stable")',
     "group ties go to the higher group index"),
    ("routing", "key = e / e.sum(axis=1, keepdims=True, dtype=np.float32)",
     "key = e / e.sum(axis=0, keepdims=True, dtype=np.float32)",
     "softmax normalised over the wrong axis"),
    ("routing", "    ids = order[:, :k].astype(np.int32)", "    ids = np.sort(order[:, :k], axis=1).astype(np.int32)",
     "ids listed by index instead of by descending key"),
    ("routing", "        scores = p / p.sum(axis=1, keepdims=True)\n\n    counts",
     "        scores = p\n\n    counts", "full-E softmax scores not normalised"),
    ("routing", "upto = min(k + 1, E)", "upto = min(k, E)",
     "near ties: the k-th/(k+1)-th gap is not examined"),
    ("routing", "        exempt |= (ggap > 0) & (ggap < NEAR_TIE_REL)\n", "",
     "near ties: the kept-group boundary gap is not examined"),
    ("routing", "masked = np.where(eligible, key64, -np.inf)", "masked = key64",
     "near ties: gaps measured over experts of dropped groups too"),
    ("routing", "exempt = np.any((gap > 0) & (gap < NEAR_TIE_REL), axis=1)",
     "exempt = np.any(gap < NEAR_TIE_REL, axis=1)", "near ties: exact ties counted as near ties"),
    ("routing", "ggap = _rel_gaps(gsrt[:, topk_group - 1:topk_group + 1])[:, 0]",
     "ggap = _rel_gaps(gsrt[:, topk_group:topk_group + 2])[:, 0]",
     "near ties: the group gap taken one position late"),
    ("routing", "near = np.abs(gs - edge) <= NEAR_TIE_REL * abs(edge)", "near = gs == edge",
     "acceptance: near-tied groups may not stand in for each other"),
    ("routing", "if np.all(np.abs(a - b) <= NEAR_TIE_REL * np.abs(b)):",
     "if np.all(a - b <= NEAR_TIE_REL * np.abs(b)):",
     "acceptance: a choice far below the oracle's is accepted"),
    ("routing", "if not np.all(elig[row]):", "if False:",
     "acceptance: experts of dropped groups accepted"),
    ("routing", "    xs = np.take_along_axis(x, ids, axis=1)", "    xs = np.take_along_axis(x, np.sort(ids, axis=1), axis=1)",
     "weights for given ids: weights listed in index order, not the ids' order"),
    ("permutation", "padded[e + 1] = padded[e] + -(-counts[e] // tile) * tile",
     "padded[e + 1] = padded[e] + counts[e]", "segments not padded to the tile"),
    ("permutation", "slots = padded[e] + np.arange(t_idx.size, dtype=np.int64)",
     "slots = padded[e] + np.arange(t_idx.size, dtype=np.int64)[::-1]",
     "tokens placed in descending order inside a segment"),
    ("permutation", "mn_limit[c] = min(start + (i + 1) * tile, start + int(counts[e]))",
     "mn_limit[c] = start + (i + 1) * tile", "row limit ignores the segment end"),
    ("permutation", "batch_idx[c] = e", "batch_idx[c] = e + off",
     "tile map holds the global expert, not the local one"),
    ("permutation", "e2p[t_idx * k + j_idx] = slots", "e2p[t_idx * k + (k - 1 - j_idx)] = slots",
     "expanded index built with a transposed slot index"),
    ("aux_loss", "return float(coeff) * num_experts / (topk * float(total_num_tokens) ** 2)",
     "return float(coeff) * num_experts / (topk * float(total_num_tokens))",
     "token count not squared"),
    ("aux_loss", "column_sums = p.sum(axis=0)", "column_sums = p.sum(axis=0) / p.shape[0]",
     "column sums averaged over local rows"),
    ("aux_loss", "row = float(grad_loss) * _constant(total_num_tokens, num_experts, topk, coeff) * c",
     "row = _constant(total_num_tokens, num_experts, topk, coeff) * c",
     "upstream gradient ignored"),
    ("front_end", "r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + float(eps))",
     "r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True))", "eps dropped"),
    ("front_end", "y = x * r * g[None, :]", "y = x * r", "gamma not applied"),
    ("front_end", "r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)",
     "r = np.ldexp(np.floor(np.ldexp(m, 8)), e - 8)", "bf16 rounding truncates"),
    ("front_end", "    z = a @ w\n", "    z = a[:, ::-1] @ w\n", "hidden features reversed in the projection"),
    ("front_end", "        sel = 1.0 / (1.0 + np.exp(-zs))", "        sel = 1.0 / (1.0 + np.exp(-zs)); sel = sel / sel.sum(axis=1, keepdims=True)",
     "sigmoid affinities renormalised"),
    ("front_end", "    np.put_along_axis(aff64, ids, sel, axis=1)",
     "    np.put_along_axis(aff64, np.sort(ids, axis=1), sel, axis=1)",
     "affinities placed at the experts in index order"),
    ("backward", "                ds = (g - c) / S", "                ds = g / S",
     "backward: renormalisation's coupling term dropped"),
    ("backward", "            dsig = s * (1.0 - s)\n            np.add.at(grad",
     "            dsig = s\n            np.add.at(grad", "backward: sigmoid derivative taken as sigma"),
    ("backward", "            grad += p * (dp - c2)", "            grad += p * (dp + c2)",
     "backward: softmax Jacobian with the wrong sign"),
    ("backward", "        g = float(scale) * np.asarray(grad_weights", "        g = np.asarray(grad_weights",
     "backward: routed scaling factor not applied"),
    ("backward", "            grad += dsig * (h - c) / Z", "            grad += dsig * (h - c)",
     "backward: sigmoid scores' normaliser dropped"),
    ("backward", "            np.add.at(grad, (rows, ids), w * (g - c))",
     "            np.add.at(grad, (rows, ids[:, ::-1]), w * (g - c))",
     "backward: gradient scattered to the chosen experts in reverse order"),
    ("dispatch", "    out[routed] = hidden[p2t[routed]]", "    out[:] = hidden[np.maximum(p2t, 0)]",
     "dispatch: padding slots copy token 0 instead of zeros"),
    ("dispatch", "        out[ok] += w[ok, j, None] * y[slot[ok]]", "        out[ok] += y[slot[ok]]",
     "combine: routing weights ignored"),
    ("dispatch", "        ok = slot >= 0", "        ok = slot >= -1",
     "combine: a non-local choice reads the last row"),
    ("dispatch", "        out[ok] += w[ok, j, None] * y[slot[ok]]", "        out[ok] += w[ok, k - 1 - j, None] * y[slot[ok]]",
     "combine: weights paired with the wrong choice"),
    ("dense", "                probs[t, e] = w[t, j]", "                probs[t, e] = w[t, k - 1 - j]",
     "dense: weights placed at the wrong choice's expert"),
    ("dense", "            if 0 <= e < E:", "            if e < E:",
     "dense: negative ids wrap to the last experts"),
]


def _mutated_module(modname, old, new):
    path = os.path.join(ORACLE_DIR, modname + ".py")
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found in {modname}: {old!r}"
    mod = types.ModuleType(f"oracle.{modname}")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new, 1), path + " (mutated)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("modname,old,new,what", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, modname, old, new, what):
    orig = importlib.import_module(f"oracle.{modname}")
    mut = _mutated_module(modname, old, new)
    for name, val in list(mut.__dict__.items()):
        if callable(val) and getattr(val, "__module__", None) in (None, f"oracle.{modname}"):
            monkeypatch.setattr(orig, name, val, raising=False)
            if hasattr(oracle, name):
                monkeypatch.setattr(oracle, name, val)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception as exc:  # an assertion or a crash both reveal the mistake
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {what}"
