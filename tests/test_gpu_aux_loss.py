"""GPU parity: moe_aux_loss (forward and backward) through the C ABI against the
oracle.  Inputs: the oracle's full-E softmax scores of seeded logits as probs
and the oracle's per-expert counts (nothing here comes from the HIP path)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import log
from workloads import WORKLOADS, route_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"
RTOL = 1e-5


def _probs_counts(w, T, seed):
    logits, _ = route_inputs(w, T=T, seed=seed)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn,
                     pre_softmax=w.pre_softmax)
    return r.scores.astype(np.float32), r.counts.astype(np.int32)


def _run(probs, counts, total, E, k, coeff, grad=None, fwd=True, bwd=True):
    rows = probs.shape[0] if probs is not None else 0
    p = torch.from_numpy(probs).to(DEV) if probs is not None else None
    c = torch.from_numpy(counts).to(DEV)
    loss = torch.full((1,), np.nan, dtype=torch.float32, device=DEV) if fwd else None
    g = torch.tensor([grad], dtype=torch.float32, device=DEV) if grad is not None else None
    gp = torch.full((rows, E), np.nan, dtype=torch.float32, device=DEV) if bwd else None
    ws = torch.zeros(max(mr.moe_aux_loss_workspace_size(rows, E), 1), dtype=torch.uint8,
                     device=DEV)
    mr.moe_aux_loss(p, c, rows, total, E, k, coeff, loss=loss, grad_loss=g, grad_probs=gp,
                    workspace=ws)
    torch.cuda.synchronize()
    return (loss.item() if fwd else None), (gp.cpu().numpy() if bwd else None)


def _check(probs, counts, total, E, k, coeff, grad=1.0, label=""):
    log(f"[gpu] aux {label}: rows={probs.shape[0]} E={E} k={k} total={total}")
    loss, gp = _run(probs, counts, total, E, k, coeff, grad=grad)
    ref = oracle.aux_loss_fwd(probs, counts, total, E, k, coeff)
    assert abs(loss - ref) <= RTOL * abs(ref), (label, loss, ref)
    gref = oracle.aux_loss_bwd(counts, probs.shape[0], total, E, k, coeff, grad_loss=grad)
    assert np.allclose(gp, gref, rtol=RTOL, atol=0), label


def test_aux_full_size():
    w = WORKLOADS["qwen_moe_like"]
    probs, counts = _probs_counts(w, w.T, w.seed)
    _check(probs, counts, w.T, w.E, w.k, w.aux_coeff, label="qwen full")


@pytest.mark.parametrize("rows,E,k", [(1, 8, 2), (63, 8, 2), (1000, 60, 4), (4097, 128, 8),
                                      (777, 256, 8), (300, 2048, 16), (5, 3, 1)])
def test_aux_shapes(rows, E, k):
    rng = np.random.default_rng(rows * 7 + E)
    logits = (rng.standard_normal((rows, E)) * 1.5).astype(np.float32)
    r = oracle.route(logits, "f32", k, score_fn="softmax", pre_softmax=True)
    probs = r.scores.astype(np.float32)
    counts = r.counts.astype(np.int32)
    _check(probs, counts, rows, E, k, 1e-2, grad=0.7, label=f"rows={rows} E={E}")


def test_aux_sharded_rows_and_grad_scalar():
    w = WORKLOADS["qwen_moe_like"]
    probs, counts = _probs_counts(w, 5000, 77)
    # this shard holds 5000 rows of a 20000-token batch; the counts are global
    _check(probs, counts * 4, 20000, w.E, w.k, 3e-2, grad=2.5, label="shard")


def test_aux_backward_only_and_forward_only():
    w = WORKLOADS["qwen_moe_like"]
    probs, counts = _probs_counts(w, 333, 5)
    log("[gpu] aux backward only / forward only")
    # backward without probs (it does not read them)
    c = torch.from_numpy(counts).to(DEV)
    gp_t = torch.full((333, w.E), np.nan, dtype=torch.float32, device=DEV)
    mr.moe_aux_loss(None, c, 333, 333, w.E, w.k, 1e-2, grad_probs=gp_t)
    torch.cuda.synchronize()
    gref = oracle.aux_loss_bwd(counts, 333, 333, w.E, w.k, 1e-2)
    assert np.allclose(gp_t.cpu().numpy(), gref, rtol=RTOL, atol=0)
    loss, _ = _run(probs, counts, 333, w.E, w.k, 1e-2, bwd=False)
    ref = oracle.aux_loss_fwd(probs, counts, 333, w.E, w.k, 1e-2)
    assert abs(loss - ref) <= RTOL * abs(ref)


def test_aux_balanced_closed_form():
    T, E, k = 4096, 64, 4
    probs = np.full((T, E), 1.0 / E, dtype=np.float32)
    counts = np.full(E, T * k // E, dtype=np.int32)
    log("[gpu] aux balanced")
    loss, gp = _run(probs, counts, T, E, k, 0.05)
    assert abs(loss - 0.05) <= RTOL * 0.05


def test_aux_empty_rows():
    E, k = 16, 2
    counts = np.arange(E, dtype=np.int32)
    log("[gpu] aux rows=0")
    loss, _ = _run(np.zeros((0, E), np.float32), counts, 100, E, k, 0.1, bwd=False)
    assert loss == 0.0


def test_aux_workspace_reuse_and_determinism():
    # one workspace for forwards of decreasing and increasing sizes: the sync
    # region is zero after every call, and repeating a call gives the same bits
    sync = mr.moe_aux_loss_sync_region_bytes()
    E, k = 128, 8
    big = 400000
    ws = torch.zeros(mr.moe_aux_loss_workspace_size(big, E), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(4242)
    for rows in (big, 1000, 1, 70001, 0, big):
        log(f"[gpu] aux reuse rows={rows}")
        probs = rng.random((rows, E), dtype=np.float32)
        counts = rng.integers(0, 5000, E).astype(np.int32)
        p = torch.from_numpy(probs).to(DEV)
        c = torch.from_numpy(counts).to(DEV)
        outs = []
        for _ in range(3):
            loss = torch.full((1,), np.nan, dtype=torch.float32, device=DEV)
            mr.moe_aux_loss(p, c, rows, max(rows, 1), E, k, 1e-2, loss=loss, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:sync].count_nonzero()) == 0, rows
            outs.append(loss.item())
        assert outs[0] == outs[1] == outs[2], (rows, outs)
        ref = oracle.aux_loss_fwd(probs, counts, max(rows, 1), E, k, 1e-2)
        assert abs(outs[0] - ref) <= RTOL * abs(ref), (rows, outs[0], ref)
