"""GPU parity: rmsnorm_gate_route through the C ABI against the oracle.

normed is compared with the oracle's RMSNorm at bf16/f16 tolerance (1e-2
relative).  Routing is then checked from the HIP path's own normed output: the
oracle projects those exact values in float64.  The kernel accumulates the
projection in float32 (MFMA partials over k-chunks, then the chunk sums), so a
token is exempt only where a deciding logit gap is below the worst-case forward
error bound of that summation: depth * 2^-24 * sum_h |normed * W| for each of
the two logits, depth = k-chunk MFMA steps + chunks + products per MFMA + 1.
Exempt tokens are counted; their ids must still be k distinct experts whose
j-th logit lies within the two bounds of the oracle's j-th logit, and their
affinities must be the oracle's affinities of those ids."""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, to_dev
from workloads import FRONT_END, front_end_inputs, FrontEndWorkload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"


def _kchunk(H):
    # the library's k-chunk (fixes the fp32 summation depth of the projection)
    for kc in (448, 384, 256, 128):
        if H % kc == 0 and (H // kc) % 8 == 0:
            return kc
    for kc in (448, 384, 256, 128):
        if H % kc == 0 and H // kc >= 8:
            return kc
    return 128


def _decode(bits, dtype):
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def run_front_end(f: FrontEndWorkload, T, H, E, seed, act="sigmoid", dtype="bf16", rbias=False,
                  ws=None):
    f2 = FrontEndWorkload(name="fe", seed=seed, T=T, H=H, E=E, k=f.k if f.k <= E else E,
                          act=act, dtype="bf16", router_bias_std=0.05 if rbias else None)
    hidden, gamma, W, rb = front_end_inputs(f2)
    if dtype == "f16":
        # the generator emits bf16 bits; re-draw as float16 bits from the same values
        hidden = _decode(hidden, "bf16").astype(np.float16).view(np.uint16)
        gamma = _decode(gamma, "bf16").astype(np.float16).view(np.uint16)
        W = _decode(W, "bf16").astype(np.float16).view(np.uint16)
        if rb is not None:
            rb = _decode(rb, "bf16").astype(np.float16).view(np.uint16)
    k = f2.k
    log(f"[gpu] front end T={T} H={H} E={E} k={k} act={act} dtype={dtype} bias={rbias}")
    h_d, g_d, w_d = to_dev(hidden, dtype), to_dev(gamma, dtype), to_dev(W, dtype)
    b_d = to_dev(rb, dtype) if rb is not None else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    normed = torch.empty((T, H), dtype=tdt, device=DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    aff = torch.full((T, E), 7.0, dtype=torch.bfloat16, device=DEV)
    if ws is None:
        ws = torch.zeros(max(mr.rmsnorm_gate_route_workspace_size(T, H, E), 1), dtype=torch.uint8,
                         device=DEV)
    mr.rmsnorm_gate_route(h_d, g_d, w_d, b_d, mr.MOE_BF16 if dtype == "bf16" else mr.MOE_F16,
                          T, H, E, f2.eps, k, mr.MOE_SIGMOID if act == "sigmoid" else mr.MOE_SOFTMAX,
                          normed, ids, aff, workspace=ws)
    torch.cuda.synchronize()
    # the in-launch handshake leaves the synchronisation region zero-filled again
    region = mr.rmsnorm_gate_route_sync_region_bytes()
    assert int(torch.count_nonzero(ws[:region])) == 0, "sync region not left zero-filled"
    normed_bits = normed.view(torch.int16).cpu().numpy().view(np.uint16)
    # 1. RMSNorm
    ref_y, ref_bits = oracle.rmsnorm(hidden, gamma, f2.eps, dtype=dtype)
    got = _decode(normed_bits, dtype)
    refv = _decode(ref_bits, dtype)
    assert np.all(np.abs(got - refv) <= 1e-2 * np.abs(refv)), "normed beyond tolerance"
    assert np.mean(normed_bits == ref_bits) > 0.999, "too many rounding flips in normed"
    # 2. routing from the HIP path's normed values
    res = oracle.front_end_route(normed_bits, W, k, act=act, dtype=dtype, router_bias=rb)
    kc = _kchunk(H)
    depth = kc // 32 + H // kc + 32 + 1
    assert mr.rmsnorm_gate_route_sum_depth(H) == depth
    exempt, bound, zs, bs = oracle.fp32_sum_near_ties(res, k, depth)
    ids_h = ids.cpu().numpy()
    ok = ~exempt
    assert np.array_equal(ids_h[ok], res.ids[ok]), "ids differ on a non-exempt token"
    aff_h = aff.view(torch.int16).cpu().numpy().view(np.uint16)
    a_got = _decode(aff_h, "bf16")
    a_ref = res.affinities64
    mask = np.zeros_like(a_ref, bool)
    np.put_along_axis(mask, res.ids.astype(np.int64), True, 1)
    okm = mask & ok[:, None]
    assert np.all(np.abs(a_got[okm] - a_ref[okm]) <= 1e-2 * np.abs(a_ref[okm])), "affinities"
    assert np.all(aff_h[~mask & ok[:, None]] == 0), "non-selected affinities must be exactly 0"
    # exempt tokens: k distinct experts; the j-th choice's logit lies within the
    # error bounds of the oracle's j-th logit (a near tie may swap two choices or
    # replace the k-th); the affinities are the oracle's of the GPU's own ids
    ex = np.nonzero(exempt)[0]
    for t in ex:
        assert len(set(ids_h[t].tolist())) == k and np.all((ids_h[t] >= 0) & (ids_h[t] < E))
        g = ids_h[t].astype(np.int64)
        assert np.all(np.abs(res.logits[t, g] - zs[t, :k]) <= bound[t, g] + bs[t, :k]), (t, g)
    if ex.size:
        a_ex = oracle.affinities_for_ids(res.logits[ex], ids_h[ex], act)
        m_ex = np.zeros_like(a_ex, bool)
        np.put_along_axis(m_ex, ids_h[ex].astype(np.int64), True, 1)
        assert np.all(np.abs(a_got[ex][m_ex] - a_ex[m_ex]) <= 1e-2 * np.abs(a_ex[m_ex])), \
            "affinities of exempt tokens"
        assert np.all(aff_h[ex][~m_ex] == 0), "non-selected affinities must be exactly 0"
    differ = int(np.sum(np.any(ids_h != res.ids, axis=1)))
    log(f"[gpu] front end ok: exempt tokens {int(exempt.sum())} ({differ} with ids other than "
        f"the oracle's), normed flips {int(np.sum(normed_bits != ref_bits))}")
    return int(exempt.sum()), differ


def test_front_end_full_size():
    f = FRONT_END
    run_front_end(f, f.T, f.H, f.E, f.seed)


@pytest.mark.parametrize("T,H,E,act,dtype,rbias", [
    (1, 128, 16, "sigmoid", "bf16", False),
    (5, 1024, 64, "softmax", "bf16", True),
    (37, 2048, 256, "sigmoid", "f16", False),
    (128, 7168, 512, "softmax", "bf16", False),
    (64, 4096, 128, "sigmoid", "bf16", True),
    (128, 384, 32, "softmax", "f16", True),
])
def test_front_end_shapes(T, H, E, act, dtype, rbias):
    run_front_end(FRONT_END, T, H, E, seed=700 + T + H + E, act=act, dtype=dtype, rbias=rbias)


def test_front_end_deterministic():
    f = FRONT_END
    hidden, gamma, W, _ = front_end_inputs(f, T=64)
    h_d, g_d, w_d = to_dev(hidden, "bf16"), to_dev(gamma, "bf16"), to_dev(W, "bf16")
    outs = []
    log("[gpu] front end determinism")
    for _ in range(2):
        normed = torch.empty((64, f.H), dtype=torch.bfloat16, device=DEV)
        ids = torch.empty((64, f.k), dtype=torch.int32, device=DEV)
        aff = torch.empty((64, f.E), dtype=torch.bfloat16, device=DEV)
        ws = torch.zeros(mr.rmsnorm_gate_route_workspace_size(64, f.H, f.E), dtype=torch.uint8,
                         device=DEV)
        mr.rmsnorm_gate_route(h_d, g_d, w_d, None, mr.MOE_BF16, 64, f.H, f.E, f.eps, f.k,
                              mr.MOE_SIGMOID, normed, ids, aff, workspace=ws)
        torch.cuda.synchronize()
        outs.append((normed.clone(), ids.clone(), aff.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_front_end_workspace_reuse_across_sizes():
    # one zero-filled workspace, sized for the largest call, serves a sequence
    # of calls of different sizes (each call leaves it zero-filled)
    ws = torch.zeros(mr.rmsnorm_gate_route_workspace_size(128, 7168, 512), dtype=torch.uint8,
                     device=DEV)
    for (T, H, E, act) in [(128, 7168, 256, "sigmoid"), (37, 2048, 512, "softmax"),
                           (1, 128, 16, "sigmoid"), (128, 7168, 512, "sigmoid")]:
        run_front_end(FRONT_END, T, H, E, seed=900 + T + E, act=act, ws=ws)
