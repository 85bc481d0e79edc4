"""GPU parity: moe_dispatch / moe_combine through the C ABI against oracle.dispatch.

The routes and permutations come from the oracle (nothing here comes from the
HIP path); hidden states and expert outputs are seeded normals.  Dispatch is a
bit copy: bit-exact.  Combine: the kernel sums the k weighted rows in float32
in choice order and rounds once, so |GPU - exact| <= 2^-8 |exact| (the bf16
half-ulp, doubled) + 1e-6 sum_j |w_j y_j| (k <= 64 float32 roundings of the
running sum); float32 outputs drop the first term to 2^-22 |exact|."""
import numpy as np
import pytest

import oracle
from gpu_helpers import log, to_dev
from workloads import WORKLOADS, route_inputs, bf16_bits_from_f32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

DEV = "cuda:0"
SENTINEL = 0x7B7B   # bf16 bits a dispatch must not touch (rows past the total)


def _route_perm(T, E, k, tile, seed, off=0, n_loc=None, score_fn="softmax", scale=1.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(logits, "f32", k, score_fn=score_fn, pre_softmax=True, renorm=True, scale=scale)
    pm = oracle.permute(r.ids, tile, local_expert_offset=off,
                        local_num_experts=E - off if n_loc is None else n_loc, num_experts=E)
    return r, pm


def _rows(rng, n, H, dtype):
    v = rng.standard_normal((n, H)).astype(np.float32)
    return bf16_bits_from_f32(v) if dtype == "bf16" else v


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def run_dispatch(hidden, dtype, pm, max_rows):
    T, H = hidden.shape
    p2t = np.full(max_rows, -7, np.int32)
    p2t[:pm.total] = pm.p2t
    out = to_dev(np.full((max_rows, H), SENTINEL if dtype == "bf16" else 0, np.uint16 if dtype == "bf16"
                         else np.float32), dtype) if dtype == "bf16" else \
        torch.full((max_rows, H), -3.0, dtype=torch.float32, device=DEV)
    mr.moe_dispatch(to_dev(hidden, dtype), mr.MOE_BF16 if dtype == "bf16" else mr.MOE_F32, T, H,
                    _dev_i32(p2t), _dev_i32([pm.total]), max_rows, out)
    torch.cuda.synchronize()
    return out


def check_dispatch(T, E, k, H, tile, dtype, seed, label):
    log(f"[gpu] dispatch {label}: T={T} E={E} k={k} H={H} tile={tile} {dtype}")
    r, pm = _route_perm(T, E, k, tile, seed)
    rng = np.random.default_rng(seed + 1)
    hidden = _rows(rng, T, H, dtype)
    max_rows = int(oracle.max_padded_tokens(T, k, E, tile))
    out = run_dispatch(hidden, dtype, pm, max_rows)
    ref = oracle.dispatch(hidden, pm.p2t, pm.total)
    if dtype == "bf16":
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[:pm.total], ref), label
        assert np.all(got[pm.total:] == SENTINEL), f"{label}: rows past the total were written"
    else:
        got = out.cpu().numpy()
        assert np.array_equal(got[:pm.total].view(np.uint32), ref.view(np.uint32)), label
        assert np.all(got[pm.total:] == -3.0), label


def check_combine(T, E, k, H, tile, dtype, seed, label, w_dtype="f32", off=0, n_loc=None):
    log(f"[gpu] combine {label}: T={T} E={E} k={k} H={H} {dtype} weights {w_dtype} loc {off}+{n_loc}")
    r, pm = _route_perm(T, E, k, tile, seed, off=off, n_loc=n_loc, scale=2.5)
    rng = np.random.default_rng(seed + 2)
    rows = max(pm.total, 1)
    y = _rows(rng, rows, H, dtype)
    w32 = r.weights.astype(np.float32)
    if w_dtype == "bf16":
        wbits = bf16_bits_from_f32(w32)
        w_used = (wbits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        w_dev = to_dev(wbits, "bf16")
    else:
        w_used = w32.astype(np.float64)
        w_dev = to_dev(w32, "f32")
    out = torch.empty((T, H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=DEV)
    mr.moe_combine(to_dev(y, dtype), mr.MOE_BF16 if dtype == "bf16" else mr.MOE_F32, T, H, k,
                   _dev_i32(pm.e2p), w_dev, mr.MOE_BF16 if w_dtype == "bf16" else mr.MOE_F32, out)
    torch.cuda.synchronize()
    exact, _ = oracle.combine(y, dtype, pm.e2p, w_used, T, k)
    yabs = np.abs(y.astype(np.float32)) if dtype == "f32" else \
        np.abs((y.astype(np.uint32) << np.uint32(16)).view(np.float32))
    scale, _ = oracle.combine(yabs.astype(np.float32), "f32", pm.e2p, np.abs(w_used), T, k)
    if dtype == "bf16":
        got = (out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32)
               << np.uint32(16)).view(np.float32).astype(np.float64)
        tol = 2.0 ** -8 * np.abs(exact) + 1e-6 * scale
    else:
        got = out.cpu().numpy().astype(np.float64)
        tol = 2.0 ** -22 * np.abs(exact) + 1e-6 * scale
    err = np.abs(got - exact)
    assert np.all(err <= tol), (label, float((err - tol).max()))


@pytest.mark.parametrize("T,E,k,H,tile,dtype", [
    (40, 8, 2, 24, 4, "bf16"), (1, 8, 2, 8, 4, "bf16"), (257, 16, 4, 512, 8, "f32"),
    (300, 64, 6, 20, 8, "bf16"),          # 40-byte rows: element-wise path
    (777, 128, 8, 1000, 16, "bf16"),      # 2000-byte rows: element-wise path
    (2048, 256, 8, 7168, 8, "bf16"),
])
def test_dispatch_shapes(T, E, k, H, tile, dtype):
    check_dispatch(T, E, k, H, tile, dtype, seed=T + E + H, label=f"{T}x{H}")


@pytest.mark.parametrize("T,E,k,H,dtype,w_dtype", [
    (40, 8, 2, 24, "bf16", "f32"), (1, 8, 2, 8, "bf16", "f32"), (257, 16, 4, 512, "f32", "f32"),
    (300, 64, 6, 20, "bf16", "bf16"),     # element-wise path
    (777, 128, 8, 1000, "bf16", "f32"),
    (200, 256, 64, 64, "f32", "bf16"),    # k = 64
    (2048, 256, 8, 7168, "bf16", "f32"),
])
def test_combine_shapes(T, E, k, H, dtype, w_dtype):
    check_combine(T, E, k, H, 8, dtype, seed=T + E + H, label=f"{T}x{H}", w_dtype=w_dtype)


def test_combine_local_expert_shard():
    # choices outside the local experts (expanded index -1) add nothing
    check_combine(500, 64, 6, 256, 8, "bf16", seed=9, label="shard", off=16, n_loc=24)


def test_dispatch_combine_full_size_sampled():
    # the DeepSeek-V3-like route at full size with its hidden size (7168):
    # sampled permuted rows and sampled tokens, computed by the oracle one by one
    w = WORKLOADS["deepseek_v3_like"]
    logits, bias = route_inputs(w)
    r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn, n_group=w.n_group,
                     topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                     scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
    pm = oracle.permute(r.ids, w.tile, num_experts=w.E)
    H = 7168
    log(f"[gpu] dispatch/combine full size: T={w.T} k={w.k} H={H} rows={pm.total}")
    rng = np.random.default_rng(77)
    hidden = bf16_bits_from_f32(rng.standard_normal((w.T, H)).astype(np.float32))
    max_rows = int(oracle.max_padded_tokens(w.T, w.k, w.E, w.tile))
    out = run_dispatch(hidden, "bf16", pm, max_rows)
    sample = rng.choice(pm.total, size=512, replace=False)
    got = out.view(torch.int16)[torch.from_numpy(sample).to(DEV)].cpu().numpy().view(np.uint16)
    for i, p in enumerate(sample):
        t = pm.p2t[p]
        assert np.array_equal(got[i], hidden[t] if t >= 0 else np.zeros(H, np.uint16)), p
    # combine the dispatched rows (identity experts): out[t] = round(sum_j w_j) * hidden[t]
    res = torch.empty((w.T, H), dtype=torch.bfloat16, device=DEV)
    mr.moe_combine(out, mr.MOE_BF16, w.T, H, w.k, _dev_i32(pm.e2p),
                   to_dev(r.weights.astype(np.float32), "f32"), mr.MOE_F32, res)
    torch.cuda.synchronize()
    toks = rng.choice(w.T, size=256, replace=False)
    got = res.view(torch.int16)[torch.from_numpy(toks).to(DEV)].cpu().numpy().view(np.uint16)
    e2p = pm.e2p.reshape(w.T, w.k)[toks].ravel()
    ysub = oracle.dispatch(hidden, pm.p2t, pm.total)[np.unique(e2p)]
    remap = {s: i for i, s in enumerate(np.unique(e2p))}
    exact, _ = oracle.combine(ysub, "bf16", np.array([remap[s] for s in e2p]),
                              r.weights.astype(np.float32)[toks].astype(np.float64), len(toks), w.k)
    gotf = (got.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    hf = (hidden[toks].astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    tol = 2.0 ** -8 * np.abs(exact) + 1e-6 * np.abs(hf) * r.weights[toks].sum(axis=1, keepdims=True)
    assert np.all(np.abs(gotf - exact) <= tol)
