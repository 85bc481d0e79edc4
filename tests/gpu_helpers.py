"""Helpers for the GPU parity tests: move the seeded inputs to the device with
the same bits, run the HIP path through the C ABI, and compare with the
oracle under the parity rules (bit-exact ids and bookkeeping except near-tie
tokens, 1e-5 relative fp32 weights, 1e-2 relative bf16 outputs)."""
from __future__ import annotations

import sys

import numpy as np

import oracle

FP32_RTOL = 1e-5
BF16_RTOL = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype: str, device="cuda:0"):
    import torch
    if arr is None:
        return None
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype in ("bf16", "f16"):
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).to(device)
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    raise ValueError(dtype)


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
    return (bits << np.uint32(16)).view(np.float32).astype(np.float64)


def weights_to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_tensor_to_f64(t)
    return t.cpu().numpy().astype(np.float64)


def compare_route(ref: "oracle.RouteResult", ids: np.ndarray, w: np.ndarray, k: int,
                  weights_bf16: bool = False, label: str = "", weights_of=None):
    """Bit-exact ids on non-exempt tokens, weights within tolerance.  Exempt
    (near-tie) tokens must return a top-k the oracle's near-tie rule accepts
    (``oracle.within_near_ties``), and their weights must match the oracle's
    weights of the GPU's own ids (``weights_of(rows, ids_rows)``).  Returns
    (exempt tokens, tokens whose ids differ from the oracle's)."""
    T = ids.shape[0]
    assert ids.shape == ref.ids.shape, (label, ids.shape, ref.ids.shape)
    ok = ~ref.exempt
    bad = np.nonzero(np.any(ids[ok] != ref.ids[ok], axis=1))[0]
    if bad.size:
        t = np.nonzero(ok)[0][bad[0]]
        raise AssertionError(f"{label}: {bad.size} tokens differ in ids; first token {t}: "
                             f"gpu {ids[t].tolist()} oracle {ref.ids[t].tolist()} "
                             f"keys {ref.keys32[t][ref.ids[t]].tolist()}")
    rtol = BF16_RTOL if weights_bf16 else FP32_RTOL
    err = np.abs(w[ok] - ref.weights[ok]) - rtol * np.abs(ref.weights[ok])
    if np.any(err > 0):
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{label}: weight mismatch {w[ok][i]} vs {ref.weights[ok][i]}")
    ex = np.nonzero(ref.exempt)[0]
    for t in ex:
        assert oracle.within_near_ties(ref, int(t), ids[t]), (
            f"{label}: near-tie token {t} outside the near-tie rule: gpu {ids[t].tolist()} "
            f"oracle {ref.ids[t].tolist()}")
    if ex.size:
        assert weights_of is not None, f"{label}: exempt tokens need the oracle's weights_of"
        want = weights_of(ex, ids[ex])
        err = np.abs(w[ex] - want) - rtol * np.abs(want)
        assert not np.any(err > 0), f"{label}: weights of near-tie tokens differ"
    differ = int(np.sum(np.any(ids != ref.ids, axis=1)))
    return int(ex.size), differ


def route_weights_of(logits, logits_dtype, score_fn, pre_softmax, renorm, scale):
    """weights_of for compare_route: the oracle's weights of given ids of given rows."""
    x = oracle.decode_input(logits, logits_dtype)

    def f(rows, ids_rows):
        return oracle.weights_for_ids(x[rows], ids_rows, score_fn, pre_softmax, renorm, scale)
    return f


def compare_permutation(gpu: dict, ids_gpu: np.ndarray, tile: int, off: int, n_loc: int,
                        label: str = ""):
    """The bookkeeping must equal the oracle's permutation of the GPU's own ids
    (pure integer work): bit-exact in every field."""
    P = oracle.permute(ids_gpu, tile, local_expert_offset=off, local_num_experts=n_loc)
    assert np.array_equal(gpu["counts"], P.counts), label
    assert np.array_equal(gpu["padded_offsets"], P.padded_offsets), label
    assert gpu["total"] == P.total, (label, gpu["total"], P.total)
    assert gpu["num_tiles"] == P.num_tiles, label
    assert np.array_equal(gpu["e2p"], P.e2p), label
    assert np.array_equal(gpu["p2t"][:P.total], P.p2t), label
    assert np.array_equal(gpu["batch_idx"][:P.num_tiles], P.batch_idx), label
    assert np.array_equal(gpu["mn_limit"][:P.num_tiles], P.mn_limit), label
    return P


def fetch_permutation(out) -> dict:
    return dict(
        counts=out.expert_counts.cpu().numpy().astype(np.int64),
        padded_offsets=out.padded_offsets.cpu().numpy().astype(np.int64),
        total=int(out.total_num_padded_tokens.cpu().item()),
        num_tiles=int(out.num_non_exiting_ctas.cpu().item()),
        e2p=out.expanded_idx_to_permuted_idx.cpu().numpy().astype(np.int64),
        p2t=out.permuted_idx_to_token_idx.cpu().numpy().astype(np.int64),
        batch_idx=out.cta_idx_xy_to_batch_idx.cpu().numpy().astype(np.int64),
        mn_limit=out.cta_idx_xy_to_mn_limit.cpu().numpy().astype(np.int64),
    )


def count_region_ready(ws, label=""):
    """The routing workspace's counting region is ready for the next call: its
    two sets of counting rows are followed by a header whose first word names
    the set the next call adds into, and that set must be entirely zero."""
    import torch
    from top_expert_routing_amd import moe_route_count_region_bytes
    region = moe_route_count_region_bytes()
    set_bytes = (region - 256) // 2
    hdr = ws[2 * set_bytes:2 * set_bytes + 16].view(torch.int32).cpu().tolist()
    nxt = hdr[0]
    assert nxt in (0, 1), (label, hdr)
    used = ws[nxt * set_bytes:(nxt + 1) * set_bytes]
    assert int(used.count_nonzero().item()) == 0, f"{label}: counting set {nxt} not clear"
