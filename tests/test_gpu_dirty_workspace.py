"""Workspaces whose synchronisation region is not clean on entry (never zeroed,
or left by a launch that failed mid-call), and the front end's give-up path.

For every entry point: no access leaves the caller's arrays (guard words past
the end of every permutation output stay intact), what the library detects it
reports (-1 totals and counts for the routing bookkeeping), and the region is
clean again for the next calls, whose outputs match the oracle.  The front
end's give-up is forced from the host with a spin limit of 0
(MOE_ROUTE_FRONT_END_SPIN_LIMIT): every wait gives up at once and every kernel
still ends normally."""
import numpy as np
import pytest

import oracle
from gpu_helpers import (compare_permutation, compare_route, count_region_ready,
                         fetch_permutation, log, route_weights_of, to_dev, weights_to_f64)
from workloads import WORKLOADS, FRONT_END, FrontEndWorkload, front_end_inputs, route_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"
GUARD = 4096                    # int32 guard words after each permutation output
SENTINEL = 0x5A5A5A5A


def _args(w, T):
    return mr.make_route_args(T, w.E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                              n_group=w.n_group, topk_group=w.topk_group,
                              group_topn=w.group_topn, renorm=w.renorm, scale=w.scale,
                              logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)


def _guarded(n):
    """An int32 output of n entries followed by GUARD sentinel words."""
    full = torch.full((n + GUARD,), SENTINEL, dtype=torch.int32, device=DEV)
    return full, full[:n]


def _guards_intact(fulls, label):
    for name, (full, n) in fulls.items():
        tail = full[n:].cpu().numpy()
        assert np.all(tail == SENTINEL), f"{label}: a write past the end of {name}"


def _permute_call(w, T, seed, ws):
    logits, bias = route_inputs(w, T=T, seed=seed)
    args = _args(w, T)
    out = mr.alloc_route_outputs(args, DEV, counts=True, permute=True, tile=w.tile)
    out.workspace = ws
    fulls = {}
    for name in ("expert_counts", "padded_offsets", "expanded_idx_to_permuted_idx",
                 "permuted_idx_to_token_idx", "cta_idx_xy_to_batch_idx",
                 "cta_idx_xy_to_mn_limit"):
        n = getattr(out, name).numel()
        full, view = _guarded(n)
        setattr(out, name, view)
        fulls[name] = (full, n)
    x = to_dev(logits, w.logits_dtype)
    b = to_dev(bias, w.bias_dtype) if bias is not None else None
    mr.route_permute(_args(w, T), x, b, tile=w.tile, out=out)
    torch.cuda.synchronize()
    ref = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn,
                       pre_softmax=w.pre_softmax, n_group=w.n_group, topk_group=w.topk_group,
                       group_topn=w.group_topn, renorm=w.renorm, scale=w.scale, bias=bias,
                       bias_dtype=w.bias_dtype)
    wof = route_weights_of(logits, w.logits_dtype, w.score_fn, w.pre_softmax, w.renorm, w.scale)
    return out, fulls, ref, wof


def _check_exact(w, T, seed, ws, label):
    out, fulls, ref, wof = _permute_call(w, T, seed, ws)
    ids = out.topk_ids.cpu().numpy()
    compare_route(ref, ids, weights_to_f64(out.topk_weights), w.k, label=label, weights_of=wof)
    compare_permutation(fetch_permutation(out), ids, w.tile, 0, w.E, label)
    _guards_intact(fulls, label)
    count_region_ready(ws, label)


def _region():
    return mr.moe_route_count_region_bytes()


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_dirty_count_region_is_reported_and_repaired(fill):
    w = WORKLOADS["deepseek_v3_like"]
    T = 16384
    need = mr.moe_route_workspace_size(_args(w, T), w.tile, w.E)
    if fill == "ones":
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    else:
        rng = np.random.default_rng(31337)
        ws = torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).to(DEV)
    label = f"dirty region ({fill})"
    log(f"[gpu] {label}: {w.name} T={T}")
    out, fulls, ref, wof = _permute_call(w, T, 5, ws)
    # ids and weights do not depend on the region
    ids = out.topk_ids.cpu().numpy()
    compare_route(ref, ids, weights_to_f64(out.topk_weights), w.k, label=label, weights_of=wof)
    # the bookkeeping reports the dirty region, and nothing is written out of bounds
    assert int(out.total_num_padded_tokens.item()) == -1, label
    assert int(out.num_non_exiting_ctas.item()) == -1, label
    assert np.all(out.expert_counts.cpu().numpy() == -1), label
    mp = mr.moe_max_padded_tokens(T, w.k, w.E, w.tile)
    e2p = out.expanded_idx_to_permuted_idx.cpu().numpy()
    assert np.all((e2p >= -1) & (e2p < mp)), label
    _guards_intact(fulls, label)
    count_region_ready(ws, label)
    # the next calls are exact: each set of counting rows gets used once
    for i in range(3):
        _check_exact(w, T if i != 1 else 5000, 40 + i, ws, f"{label}, call {i + 2}")


def test_dirty_rows_under_a_clean_header():
    w = WORKLOADS["deepseek_v3_like"]
    T = 16384
    need = mr.moe_route_workspace_size(_args(w, T), w.tile, w.E)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    rows = ws[:_region()].view(torch.int32)
    # a count far below zero in the set the first call adds into: detected
    rows[3] = -(1 << 24)
    label = "negative garbage count"
    log(f"[gpu] {label}")
    out, fulls, _, _ = _permute_call(w, T, 6, ws)
    assert int(out.total_num_padded_tokens.item()) == -1, label
    _guards_intact(fulls, label)
    count_region_ready(ws, label)
    _check_exact(w, T, 7, ws, label + ", next call")
    # a small positive one looks like a count: not detected, and the call's
    # bookkeeping is off by it, but stays in bounds; the calls after are exact
    ws.zero_()
    rows[5] = 1
    label = "small garbage count"
    log(f"[gpu] {label}")
    out, fulls, ref, _ = _permute_call(w, T, 8, ws)
    got = out.expert_counts.cpu().numpy()
    want = np.bincount(out.topk_ids.cpu().numpy().ravel(), minlength=w.E)
    assert got[5] == want[5] + 1 and np.array_equal(np.delete(got, 5), np.delete(want, 5)), label
    _guards_intact(fulls, label)
    for i in range(2):
        _check_exact(w, T, 9 + i, ws, f"{label}, call {i + 2}")


def test_dirty_count_region_route_counts():
    w = WORKLOADS["qwen_moe_like"]
    T = 4097
    args = _args(w, T)
    out = mr.alloc_route_outputs(args, DEV, counts=True)
    out.workspace = torch.full((mr.moe_route_workspace_size(args, w.tile, w.E),), 0xFF,
                               dtype=torch.uint8, device=DEV)
    logits, bias = route_inputs(w, T=T, seed=12)
    x = to_dev(logits, w.logits_dtype)
    log("[gpu] moe_route counts on a dirty region")
    mr.route(args, x, None, counts=True, out=out)
    torch.cuda.synchronize()
    assert np.all(out.expert_counts.cpu().numpy() == -1)
    for i in range(2):
        logits, _ = route_inputs(w, T=T, seed=13 + i)
        mr.route(args, to_dev(logits, w.logits_dtype), None, counts=True, out=out)
        torch.cuda.synchronize()
        ids = out.topk_ids.cpu().numpy()
        assert np.array_equal(out.expert_counts.cpu().numpy(),
                              np.bincount(ids.ravel(), minlength=w.E)), i
        count_region_ready(out.workspace, f"counts call {i + 2}")
    # the repaired region serves moe_route_permute as well
    _check_exact(w, T, 15, out.workspace, "permute after the repaired counts region")


def _front_end(ws, T=128, H=1024, E=256, seed=3):
    f = FrontEndWorkload(name="fe", seed=seed, T=T, H=H, E=E, k=FRONT_END.k, act="sigmoid",
                         dtype="bf16", router_bias_std=None)
    hidden, gamma, W, _ = front_end_inputs(f)
    normed = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.full((T, f.k), -7, dtype=torch.int32, device=DEV)
    aff = torch.full((T, E), 7.0, dtype=torch.bfloat16, device=DEV)
    mr.rmsnorm_gate_route(to_dev(hidden, "bf16"), to_dev(gamma, "bf16"), to_dev(W, "bf16"), None,
                          mr.MOE_BF16, T, H, E, f.eps, f.k, mr.MOE_SIGMOID, normed, ids, aff,
                          workspace=ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), aff.view(torch.int16).cpu().numpy()


def _fail_line(ws):
    return ws[:16].view(torch.int32).cpu().tolist()


def test_front_end_give_up_and_dirty_failure_word(monkeypatch):
    T, H, E = 128, 1024, 256
    ws = torch.zeros(mr.rmsnorm_gate_route_workspace_size(T, H, E), dtype=torch.uint8, device=DEV)
    region = mr.rmsnorm_gate_route_sync_region_bytes()
    log("[gpu] front end: reference call")
    ids_ref, aff_ref = _front_end(ws)
    assert np.all((ids_ref >= 0) & (ids_ref < E))
    assert int(torch.count_nonzero(ws[:region])) == 0
    # every wait gives up at once: -1 ids, one failure counted, the region clean
    monkeypatch.setenv("MOE_ROUTE_FRONT_END_SPIN_LIMIT", "0")
    log("[gpu] front end: forced give-up")
    ids, _ = _front_end(ws)
    assert np.all(ids == -1)
    assert _fail_line(ws) == [0, 1, 0, 0]
    assert int(torch.count_nonzero(ws[256:region])) == 0        # the scale slots
    monkeypatch.delenv("MOE_ROUTE_FRONT_END_SPIN_LIMIT")
    log("[gpu] front end: after the give-up")
    ids, aff = _front_end(ws)
    assert np.array_equal(ids, ids_ref) and np.array_equal(aff, aff_ref)
    assert _fail_line(ws) == [0, 1, 0, 0]
    # a failure word that is not clean on entry is reported as a give-up of
    # that call (counted once, whatever the readers' counter held) and cleared
    ws[:4].view(torch.int32).fill_(1)
    ws[8:12].view(torch.int32).fill_(12345)
    log("[gpu] front end: dirty failure word")
    ids, _ = _front_end(ws)
    assert np.all(ids == -1)
    assert _fail_line(ws) == [0, 2, 0, 0]
    log("[gpu] front end: after the dirty failure word")
    ids, aff = _front_end(ws)
    assert np.array_equal(ids, ids_ref) and np.array_equal(aff, aff_ref)
    assert _fail_line(ws) == [0, 2, 0, 0]


def test_aux_dirty_slots():
    # a dirty slot reads as a published partial: the forward that reads it gives
    # a wrong loss, touches no slot past its blocks, and may leave slots set (a
    # block can publish after the summing block, which did not wait for it, has
    # cleared them); after the caller zeroes the region the forward is exact
    rows, E, k = 30000, 128, 8
    nb = -(-rows // -(-8192 // E))          # blocks of about 32 KiB of probs
    rng = np.random.default_rng(404)
    probs = rng.random((rows, E), dtype=np.float32)
    counts = rng.integers(0, 3000, E).astype(np.int32)
    p = torch.from_numpy(probs).to(DEV)
    c = torch.from_numpy(counts).to(DEV)
    sync = mr.moe_aux_loss_sync_region_bytes()
    ws = torch.full((mr.moe_aux_loss_workspace_size(rows, E),), 0x33, dtype=torch.uint8,
                    device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    log("[gpu] aux forward on dirty slots")
    mr.moe_aux_loss(p, c, rows, rows, E, k, 1e-2, loss=loss, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.all(ws[nb * 8:sync] == 0x33))
    ws.zero_()
    ref = oracle.aux_loss_fwd(probs, counts, rows, E, k, 1e-2)
    for i in range(2):
        mr.moe_aux_loss(p, c, rows, rows, E, k, 1e-2, loss=loss, workspace=ws)
        torch.cuda.synchronize()
        assert abs(loss.item() - ref) <= 1e-5 * abs(ref), i
        assert int(torch.count_nonzero(ws[:nb * 8])) == 0


def test_aux_forced_give_up(monkeypatch):
    # the summing block's wait forced to give up at once: the loss is the
    # documented timeout NaN, the workspace is left dirty, and after zeroing it
    # the next forward is exact
    rows, E, k = 30000, 128, 8
    rng = np.random.default_rng(505)
    probs = rng.random((rows, E), dtype=np.float32)
    counts = rng.integers(0, 3000, E).astype(np.int32)
    p = torch.from_numpy(probs).to(DEV)
    c = torch.from_numpy(counts).to(DEV)
    ws = torch.zeros(mr.moe_aux_loss_workspace_size(rows, E), dtype=torch.uint8, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    monkeypatch.setenv("MOE_ROUTE_AUX_SPIN_LIMIT", "0")
    log("[gpu] aux forward, forced give-up")
    mr.moe_aux_loss(p, c, rows, rows, E, k, 1e-2, loss=loss, workspace=ws)
    torch.cuda.synchronize()
    assert int(loss.view(torch.int32).item()) & 0xFFFFFFFF == 0x7FC0A0A0
    assert int(torch.count_nonzero(ws)) > 0                   # the partials stay behind
    monkeypatch.delenv("MOE_ROUTE_AUX_SPIN_LIMIT")
    ws.zero_()
    mr.moe_aux_loss(p, c, rows, rows, E, k, 1e-2, loss=loss, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.aux_loss_fwd(probs, counts, rows, E, k, 1e-2)
    assert abs(loss.item() - ref) <= 1e-5 * abs(ref)
    assert int(torch.count_nonzero(ws)) == 0
