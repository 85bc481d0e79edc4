"""GPU: the entry points captured into a HIP graph and replayed.

The benchmark replays moe_route_permute, moe_aux_loss and rmsnorm_gate_route
from captured graphs (and one test captures a layer's whole routing data
path: route and permute, dispatch, combine, dense outputs and backward), whose kernels keep the routing counting region and the
front-end synchronisation region ready themselves (no memset nodes).  Each
test captures one call, then replays it several times with the program's own
eager work and synchronisations between the replays, poisoning the outputs
before every replay; every replay must reproduce the eager call's outputs bit
for bit, the front end's region must be zero again afterwards and the routing
workspace's set of counting rows for the next call must be clear.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import count_region_ready, log, to_dev
from workloads import FRONT_END, WORKLOADS, front_end_inputs, route_inputs, with_overrides

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def _args(mr, w, T):
    return mr.make_route_args(T, w.E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                              n_group=w.n_group, topk_group=w.topk_group, group_topn=w.group_topn,
                              renorm=w.renorm, scale=w.scale, logits_dtype=w.logits_dtype,
                              bias_dtype=w.bias_dtype)


_ROUTE_FIELDS = ("topk_ids", "topk_weights", "expert_counts", "padded_offsets",
                 "total_num_padded_tokens", "num_non_exiting_ctas", "expanded_idx_to_permuted_idx")


@pytest.mark.parametrize("name,T", [("deepseek_v3_like", 4097), ("qwen_moe_like", 20000),
                                    ("tiny_softmax_post", 16)])
def test_route_permute_graph_replays(name, T):
    import torch
    import top_expert_routing_amd as mr
    w = with_overrides(WORKLOADS[name], T=T)
    logits, bias = route_inputs(w, T=T, seed=7100 + T)
    logits2, _ = route_inputs(w, T=T, seed=7200 + T)
    args = _args(mr, w, T)
    x, x2 = to_dev(logits, w.logits_dtype), to_dev(logits2, w.logits_dtype)
    b = to_dev(bias, w.bias_dtype) if bias is not None else None
    log(f"[gpu] graph replays: {name} T={T}")
    ref = mr.route_permute(args, x, b, tile=w.tile)
    torch.cuda.synchronize()
    out = mr.alloc_route_outputs(args, DEV, permute=True, tile=w.tile)
    mr.route_permute(args, x, b, tile=w.tile, out=out)        # first call outside the capture
    torch.cuda.synchronize()
    g = _capture(lambda: mr.route_permute(args, x, b, tile=w.tile, out=out))
    total = int(ref.total_num_padded_tokens.item())
    ntiles = int(ref.num_non_exiting_ctas.item())
    for rep in range(REPLAYS):
        for f in _ROUTE_FIELDS + ("permuted_idx_to_token_idx", "cta_idx_xy_to_batch_idx",
                                  "cta_idx_xy_to_mn_limit"):
            getattr(out, f).fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for f in _ROUTE_FIELDS:
            assert torch.equal(getattr(out, f), getattr(ref, f)), (name, rep, f)
        assert torch.equal(out.permuted_idx_to_token_idx[:total], ref.permuted_idx_to_token_idx[:total])
        assert torch.equal(out.cta_idx_xy_to_batch_idx[:ntiles], ref.cta_idx_xy_to_batch_idx[:ntiles])
        assert torch.equal(out.cta_idx_xy_to_mn_limit[:ntiles], ref.cta_idx_xy_to_mn_limit[:ntiles])
        count_region_ready(out.workspace, f"{name} replay {rep}")
        # the program's own eager work between replays, on other buffers
        other = mr.route_permute(args, x2, b, tile=w.tile)
        torch.cuda.synchronize()
        assert int(other.expert_counts.sum().item()) == T * w.k


def test_aux_loss_graph_replays():
    import torch
    import top_expert_routing_amd as mr
    rows, E, k, coeff = 30000, 128, 8, 1e-2
    rng = np.random.default_rng(7300)
    probs = torch.from_numpy(rng.random((rows, E), dtype=np.float32)).to(DEV)
    counts = torch.from_numpy(rng.integers(0, 3000, E).astype(np.int32)).to(DEV)
    gl = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    ws = torch.zeros(mr.moe_aux_loss_workspace_size(rows, E), dtype=torch.uint8, device=DEV)
    loss_ref = torch.empty(1, dtype=torch.float32, device=DEV)
    grad_ref = torch.empty((rows, E), dtype=torch.float32, device=DEV)
    mr.moe_aux_loss(probs, counts, rows, rows, E, k, coeff, loss=loss_ref, grad_loss=gl,
                    grad_probs=grad_ref, workspace=ws)
    torch.cuda.synchronize()
    loss = torch.empty_like(loss_ref)
    grad = torch.empty_like(grad_ref)
    g = _capture(lambda: mr.moe_aux_loss(probs, counts, rows, rows, E, k, coeff, loss=loss,
                                         grad_loss=gl, grad_probs=grad, workspace=ws))
    log(f"[gpu] graph replays: aux loss rows={rows} E={E}")
    for rep in range(REPLAYS):
        loss.fill_(float("nan"))
        grad.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss, loss_ref), rep
        assert torch.equal(grad, grad_ref), rep
        assert int(ws[:mr.moe_aux_loss_sync_region_bytes()].count_nonzero()) == 0, rep
        # eager work between replays: the same op on other data, sharing nothing
        other = torch.empty_like(loss_ref)
        ws2 = torch.zeros_like(ws)
        mr.moe_aux_loss(probs[: rows // 2], counts, rows // 2, rows, E, k, coeff, loss=other,
                        workspace=ws2)
        torch.cuda.synchronize()


def test_front_end_graph_replays():
    import torch
    import top_expert_routing_amd as mr
    f = FRONT_END
    hidden, gamma, W, _ = front_end_inputs(f)
    h, gm, wt = to_dev(hidden, "bf16"), to_dev(gamma, "bf16"), to_dev(W, "bf16")
    T, H, E, k = f.T, f.H, f.E, f.k
    ws = torch.zeros(mr.rmsnorm_gate_route_workspace_size(T, H, E), dtype=torch.uint8, device=DEV)

    def outputs():
        return (torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
                torch.empty((T, k), dtype=torch.int32, device=DEV),
                torch.empty((T, E), dtype=torch.bfloat16, device=DEV))

    nm_r, ids_r, aff_r = outputs()
    mr.rmsnorm_gate_route(h, gm, wt, None, mr.MOE_BF16, T, H, E, f.eps, k, mr.MOE_SIGMOID,
                          nm_r, ids_r, aff_r, workspace=ws)
    torch.cuda.synchronize()
    nm, ids, aff = outputs()
    g = _capture(lambda: mr.rmsnorm_gate_route(h, gm, wt, None, mr.MOE_BF16, T, H, E, f.eps, k,
                                               mr.MOE_SIGMOID, nm, ids, aff, workspace=ws))
    region = mr.rmsnorm_gate_route_sync_region_bytes()
    log(f"[gpu] graph replays: front end T={T} H={H} E={E}")
    for rep in range(REPLAYS):
        nm.fill_(7.0)
        ids.fill_(-7)
        aff.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(nm.view(torch.int16), nm_r.view(torch.int16)), rep
        assert torch.equal(ids, ids_r), rep
        assert torch.equal(aff.view(torch.int16), aff_r.view(torch.int16)), rep
        assert int(ws[:region].count_nonzero().item()) == 0, rep
        # eager work between replays, with its own workspace
        ws2 = torch.zeros_like(ws)
        o = outputs()
        mr.rmsnorm_gate_route(h, gm, wt, None, mr.MOE_BF16, T, H, E, f.eps, k, mr.MOE_SIGMOID,
                              *o, workspace=ws2)
        torch.cuda.synchronize()
        assert torch.equal(o[1], ids_r), rep


def test_concurrent_streams():
    """Calls on different streams with their own workspaces run at the same
    time (the library keeps no per-call state outside the workspace); each
    result equals the same call made alone."""
    import torch
    import top_expert_routing_amd as mr
    w1 = with_overrides(WORKLOADS["deepseek_v3_like"], T=8192)
    w2 = with_overrides(WORKLOADS["qwen_moe_like"], T=8192)
    calls = []
    for w, seed in ((w1, 7400), (w2, 7401)):
        logits, bias = route_inputs(w, T=w.T, seed=seed)
        x = to_dev(logits, w.logits_dtype)
        b = to_dev(bias, w.bias_dtype) if bias is not None else None
        args = _args(mr, w, w.T)
        ref = mr.route_permute(args, x, b, tile=w.tile)
        calls.append((w, args, x, b, ref))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in calls]
    outs = [mr.alloc_route_outputs(args, DEV, permute=True, tile=w.tile)
            for w, args, _, _, _ in calls]
    log("[gpu] two routing calls on two streams, ten rounds")
    for rep in range(10):
        for (w, args, x, b, _), s, o in zip(calls, streams, outs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                o.topk_ids.fill_(-7)
                mr.route_permute(args, x, b, tile=w.tile, out=o)
        torch.cuda.synchronize()
        for (w, _, _, _, ref), o in zip(calls, outs):
            total = int(ref.total_num_padded_tokens.item())
            for f in _ROUTE_FIELDS:
                assert torch.equal(getattr(o, f), getattr(ref, f)), (w.name, rep, f)
            assert torch.equal(o.permuted_idx_to_token_idx[:total], ref.permuted_idx_to_token_idx[:total])


def test_layer_data_path_graph_replays():
    # one captured graph holding a layer's whole routing data path: route and
    # permute, dispatch of the hidden rows, combine of the dispatched rows, the
    # dense outputs and the routing backward; every replay equals the eager calls
    import torch
    import top_expert_routing_amd as mr
    w = with_overrides(WORKLOADS["deepseek_v3_like"], T=1000)
    T, E, k, H = w.T, w.E, w.k, 256
    logits, bias = route_inputs(w, T=T, seed=7600)
    args = _args(mr, w, T)
    x, b = to_dev(logits, w.logits_dtype), to_dev(bias, w.bias_dtype)
    rng = np.random.default_rng(7601)
    hidden = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    gw = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    mp = mr.moe_max_padded_tokens(T, k, E, w.tile)

    def run(o):
        mr.route_permute(args, x, b, tile=w.tile, out=o["route"])
        r = o["route"]
        mr.moe_dispatch(hidden, mr.MOE_BF16, T, H, r.permuted_idx_to_token_idx,
                        r.total_num_padded_tokens, mp, o["disp"])
        mr.moe_combine(o["disp"], mr.MOE_BF16, T, H, k, r.expanded_idx_to_permuted_idx,
                       r.topk_weights, mr.MOE_F32, o["comb"])
        mr.moe_topk_to_dense(T, E, k, r.topk_ids, r.topk_weights, mr.MOE_F32, o["probs"], o["rmap"])
        mr.moe_route_backward(args, x, r.topk_ids, gw, None, o["grad"])

    def buffers():
        return {"route": mr.alloc_route_outputs(args, DEV, permute=True, tile=w.tile),
                "disp": torch.empty((mp, H), dtype=torch.bfloat16, device=DEV),
                "comb": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
                "probs": torch.empty((T, E), dtype=torch.float32, device=DEV),
                "rmap": torch.empty((T, E), dtype=torch.uint8, device=DEV),
                "grad": torch.empty((T, E), dtype=torch.float32, device=DEV)}

    log(f"[gpu] graph replays: layer data path T={T} H={H}")
    ref = buffers()
    run(ref)
    torch.cuda.synchronize()
    total = int(ref["route"].total_num_padded_tokens.item())
    out = buffers()
    run(out)                                               # first call outside the capture
    torch.cuda.synchronize()
    g = _capture(lambda: run(out))
    for rep in range(REPLAYS):
        for key in ("disp", "comb", "probs", "grad"):
            out[key].fill_(float("nan"))
        out["rmap"].fill_(7)
        out["route"].topk_ids.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["route"].topk_ids, ref["route"].topk_ids), rep
        assert torch.equal(out["disp"][:total].view(torch.int16), ref["disp"][:total].view(torch.int16)), rep
        for key in ("comb", "probs", "rmap", "grad"):
            assert torch.equal(out[key].view(torch.uint8), ref[key].view(torch.uint8)), (rep, key)
        count_region_ready(out["route"].workspace, f"layer path replay {rep}")
        other = mr.route_permute(args, x, b, tile=w.tile)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other.topk_ids, ref["route"].topk_ids)
