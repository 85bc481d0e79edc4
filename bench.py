#!/usr/bin/env python3
"""Benchmark of the MoE routing hot path on one MI355X.

One step = one moe_route_permute call (score function, bias, grouped top-k,
top-k, weights, per-expert counts, tile-padded offsets, both index maps and
the per-tile expert map) over one batch of synthetic logits already resident
in HBM.  Default workload: T=16384 tokens, E=256 experts, k=8, bf16 logits,
grouped sigmoid with an fp32 correction bias (8 groups, keep 4, top-2-sum
group score), routed scaling 2.5, tile 8.

Timing: the K timed steps are captured once into a HIP graph and replayed
(the per-call host cost of a ctypes call is larger than the GPU time of a
step).  Step i reads rotating buffer set i mod R, with R sets spanning more
than twice the 256 MB Infinity Cache, so every step starts cold.  The route
kernel's average duration comes from HIP events the library records on the
launch stream around each launch (a separate eager pass with a backlogged
queue, so host latency does not enter the brackets).

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="deepseek_v3_like",
                    help="a routing workload, or decode_front_end for the front end alone")
    ap.add_argument("--rotate-mb", type=int, default=2 * 256 + 64,
                    help="bytes spanned by the rotating buffer sets (MiB)")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the single-buffer-set (cache-warm) number")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other workloads (reported under other_configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="seconds of oracle work timed for the headline cpu_baseline")
    ap.add_argument("--cpu-seconds-other", type=float, default=3.0,
                    help="seconds of oracle work timed beside each other workload")
    ap.add_argument("--only-other", default=None,
                    help="comma-separated other_configs entries to run (the rest are skipped)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="finish with plain device copies of this many MiB (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    return ap.parse_args()


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_expert_routing_amd", "csrc")
    for name in ("route_kernel.hpp", "route_sigmoid.hip", "device_common.hpp", "kernels.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per route-kernel launch from the committed rocprofv3 --pmc summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None when
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"route_kernel_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- (source_sha256|traffic_bytes_per_launch): *`?([0-9a-f]+)`?\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_sha256") != kernel_sources_digest():
        return None
    v = fields.get("traffic_bytes_per_launch")
    return int(v) if v is not None else None


def graph_ms(torch, step, K, warmup=3):
    """Average milliseconds of step(i), i = 0..K-1, captured into one HIP graph."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def n_sets(set_bytes, rotate_mb):
    return max(2, min(256, math.ceil(max(rotate_mb * 2 ** 20, 2 * MALL_BYTES + 1) / set_bytes)))


def plain_op_entry(torch, rotate_mb, K, desc, nbytes, make, op):
    """A plain PyTorch kernel that moves about the same HBM bytes as a streaming
    row, timed in the same harness (cold rotating sets, one HIP graph): what a
    generic device kernel reaches at this size, beside the row's own kernel."""
    R = n_sets(nbytes, rotate_mb)
    sets = [make() for _ in range(R)]
    ms = graph_ms(torch, lambda i: op(*sets[i % R]), K)
    del sets
    return {"op": desc, "us_per_call": ms * 1e3, "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "buffer_sets": R}


def route_permute_bytes(w, T, total, ntiles):
    lsz = 2 if w.logits_dtype == "bf16" else 4
    return (T * w.E * lsz + (w.E * 4 if w.has_bias else 0) + 3 * T * w.k * 4 + total * 4 +
            2 * ntiles * 4 + w.E * 4 + (w.E + 1) * 4 + 8)


def other_configs(mr, torch, np, dev, rotate_mb, K, cpu_seconds=None, only=None):
    """The other workloads, each cold (rotating sets past 2x the MALL): ms per
    call and algorithmic GB/s; with cpu_seconds, the oracle timed beside each
    (cpu_baseline) and the near-tie count of the GPU's output.  `only`: the names
    of the entries to run (all when None)."""
    from workloads import WORKLOADS, FRONT_END, front_end_inputs, route_inputs, with_overrides
    res = {}

    def want(name):
        return only is None or name in only

    def dev_logits(w, arr):
        if w.logits_dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(arr).to(dev)

    for name in ("tiny_softmax_post", "mixtral_like", "qwen_moe_like"):
        if not want(name):
            continue
        w = WORKLOADS[name]
        logits, bias = route_inputs(w)
        x0 = dev_logits(w, logits)
        b0 = None if bias is None else torch.from_numpy(bias).to(dev)
        args = mr.make_route_args(w.T, w.E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                                  n_group=w.n_group, topk_group=w.topk_group,
                                  group_topn=w.group_topn, renorm=w.renorm, scale=w.scale,
                                  logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)
        with_scores = w.aux_coeff is not None
        o0 = mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile, scores=with_scores)
        sb = x0.numel() * x0.element_size() + sum(
            t.numel() * t.element_size() for t in vars(o0).values() if isinstance(t, torch.Tensor))
        R = n_sets(sb, rotate_mb)
        sets = [(x0 if r == 0 else x0.clone(),
                 o0 if r == 0 else mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile,
                                                          scores=with_scores))
                for r in range(R)]

        def step(i, scores=False):
            x, o = sets[i % R]
            sc = o.scores
            o.scores = o.scores if scores else None
            mr.route_permute(args, x, b0, tile=w.tile, out=o)
            o.scores = sc

        ms = graph_ms(torch, step, K)
        total = int(o0.total_num_padded_tokens.item())
        ntiles = int(o0.num_non_exiting_ctas.item())
        nbytes = route_permute_bytes(w, w.T, total, ntiles)
        entry = {"workload": w.description, "us_per_call": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3),
                 "algorithmic_bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9, "buffer_sets": R}
        if with_scores:
            ms_s = graph_ms(torch, lambda i: step(i, True), K)
            sbytes = nbytes + w.T * w.E * 4
            entry["with_scores"] = {"us_per_call": ms_s * 1e3, "algorithmic_bytes": sbytes,
                                    "gbs": sbytes / (ms_s * 1e-3) / 1e9}
            # aux loss forward (reads probs) and backward (writes the gradient)
            probs = [o.scores for _, o in sets]
            counts = o0.expert_counts
            loss = torch.empty(1, dtype=torch.float32, device=dev)
            wsa = torch.zeros(max(mr.moe_aux_loss_workspace_size(w.T, w.E), 1), dtype=torch.uint8,
                              device=dev)
            grads = [torch.empty((w.T, w.E), dtype=torch.float32, device=dev) for _ in range(R)]
            fwd = graph_ms(torch, lambda i: mr.moe_aux_loss(probs[i % R], counts, w.T, w.T, w.E, w.k,
                                                            w.aux_coeff, loss=loss, workspace=wsa), K)
            bwd = graph_ms(torch, lambda i: mr.moe_aux_loss(None, counts, w.T, w.T, w.E, w.k,
                                                            w.aux_coeff, grad_probs=grads[i % R]), K)
            ab = w.T * w.E * 4 + w.E * 4
            del grads, probs
            shape = (w.T, w.E)
            entry["aux_forward"] = {
                "us_per_call": fwd * 1e3, "gbs": ab / (fwd * 1e-3) / 1e9,
                "plain_torch_op": plain_op_entry(
                    torch, rotate_mb, K, "row maximum of a [T,E] f32 tensor (amax over E)",
                    w.T * w.E * 4 + w.T * 4,
                    lambda: (torch.randn(shape, device=dev), torch.empty(w.T, device=dev)),
                    lambda p, m: torch.amax(p, dim=1, out=m))}
            entry["aux_backward"] = {
                "us_per_call": bwd * 1e3, "gbs": ab / (bwd * 1e-3) / 1e9,
                "plain_torch_op": plain_op_entry(
                    torch, rotate_mb, K, "fill of a [T,E] f32 tensor", w.T * w.E * 4,
                    lambda: (torch.empty(shape, device=dev),), lambda g: g.fill_(0.5))}
        if cpu_seconds:
            entry["near_ties"] = near_tie_entry(w, logits, bias, o0.topk_ids.cpu().numpy())
            entry["cpu_baseline"] = cpu_baseline_entry(w, cpu_seconds, max_T=8192)
        res[name] = entry
        del sets, o0

    # backward of the routing outputs (DeepSeek-V3-like: weights gradient;
    # Qwen-like: weights and full-E scores gradients), cold like the rest
    for name, with_s in (("deepseek_v3_like", False), ("qwen_moe_like", True)):
        if not want(name + "_backward"):
            continue
        w = WORKLOADS[name]
        logits, _ = route_inputs(w)
        x0 = dev_logits(w, logits)
        args = mr.make_route_args(w.T, w.E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                                  renorm=w.renorm, scale=w.scale, logits_dtype=w.logits_dtype)
        gen = torch.Generator(device="cpu").manual_seed(w.seed + 1)
        ids0 = torch.randint(0, w.E, (w.T, w.k), generator=gen, dtype=torch.int32).to(dev)
        gw0 = torch.randn((w.T, w.k), generator=gen, dtype=torch.float32).to(dev)
        gs0 = torch.randn((w.T, w.E), generator=gen, dtype=torch.float32).to(dev) if with_s else None
        set_b = (x0.numel() * x0.element_size() + ids0.numel() * 4 + gw0.numel() * 4 +
                 (gs0.numel() * 4 if with_s else 0) + w.T * w.E * 4)
        R = n_sets(set_b, rotate_mb)
        # algorithmic bytes: the sigmoid weights read only the k chosen logits
        # of a token, the softmax-before-top-k and score gradients the whole row
        alg_b = set_b if with_s else set_b - x0.numel() * x0.element_size() + ids0.numel() * x0.element_size()
        bsets = [(x0.clone(), ids0.clone(), gw0.clone(), None if gs0 is None else gs0.clone(),
                  torch.empty((w.T, w.E), dtype=torch.float32, device=dev)) for _ in range(R)]
        ms = graph_ms(torch, lambda i: mr.moe_route_backward(args, *bsets[i % R]), K)
        del bsets
        shape = (w.T, w.E)
        if with_s:
            plain = plain_op_entry(
                torch, rotate_mb, K, "f32 [T,E] + bf16 [T,E] -> f32 [T,E] (torch.add)",
                w.T * w.E * 10,
                lambda: (torch.randn(shape, device=dev), x0.clone(), torch.empty(shape, device=dev)),
                lambda a, b, c: torch.add(a, b, out=c))
        else:
            plain = plain_op_entry(
                torch, rotate_mb, K, "fill of a f32 [T,E] tensor", w.T * w.E * 4,
                lambda: (torch.empty(shape, device=dev),), lambda b: b.fill_(1.0))
        res[name + "_backward"] = {
            "workload": w.description + ("; grad of weights and scores" if with_s else
                                         "; grad of weights") + " -> grad of logits",
            "us_per_call": ms * 1e3, "algorithmic_bytes": alg_b,
            "gbs": alg_b / (ms * 1e-3) / 1e9, "buffer_sets": R, "plain_torch_op": plain}

    if want("deepseek_v3_like_dense_outputs"):
        # dense [T, E] probs + routing map from the DeepSeek-V3-like top-k outputs
        w = WORKLOADS["deepseek_v3_like"]
        gen = torch.Generator(device="cpu").manual_seed(w.seed + 3)
        ids0 = torch.argsort(torch.rand((w.T, w.E), generator=gen), dim=1)[:, :w.k].to(torch.int32).to(dev)
        wts0 = torch.rand((w.T, w.k), generator=gen).to(dev)
        x_bytes = w.T * w.k * 8 + w.T * w.E * 5
        R = n_sets(x_bytes, rotate_mb)
        xsets = [(ids0.clone(), wts0.clone(), torch.empty((w.T, w.E), dtype=torch.float32, device=dev),
                  torch.empty((w.T, w.E), dtype=torch.uint8, device=dev)) for _ in range(R)]
        ms_x = graph_ms(torch, lambda i: mr.moe_topk_to_dense(w.T, w.E, w.k, xsets[i % R][0], xsets[i % R][1],
                                                              mr.MOE_F32, xsets[i % R][2], xsets[i % R][3]), K)
        del xsets
        res["deepseek_v3_like_dense_outputs"] = {
            "workload": f"{w.description}; top-k ids/weights -> dense probs [T,E] f32 + routing map [T,E] u8",
            "us_per_call": ms_x * 1e3, "algorithmic_bytes": x_bytes, "gbs": x_bytes / (ms_x * 1e-3) / 1e9,
            "buffer_sets": R,
            "plain_torch_op": plain_op_entry(
                torch, rotate_mb, K, "fill of a u8 tensor of T*E*5 bytes", w.T * w.E * 5,
                lambda: (torch.empty(w.T * w.E * 5, dtype=torch.uint8, device=dev),),
                lambda b: b.fill_(1))}

    if want("deepseek_v3_like_T262144"):
        # the headline method at 16x the tokens (T = 262144, 134 MB of logits): how
        # close the same kernels come to the HBM roofline once a launch is long
        # enough to hide its cold reads and its drain
        w = with_overrides(WORKLOADS["deepseek_v3_like"], T=262144)
        logits, bias = route_inputs(w)
        x0 = dev_logits(w, logits)
        b0 = torch.from_numpy(bias).to(dev)
        del logits
        args = mr.make_route_args(w.T, w.E, w.k, score_fn=w.score_fn, n_group=w.n_group,
                                  topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                                  scale=w.scale, logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)
        o0 = mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile)
        sb = x0.numel() * x0.element_size() + sum(
            t.numel() * t.element_size() for t in vars(o0).values() if isinstance(t, torch.Tensor))
        R = n_sets(sb, rotate_mb)
        lsets = [(x0 if r == 0 else x0.clone(),
                  o0 if r == 0 else mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile))
                 for r in range(R)]

        def lstep(i):
            mr.route_permute(args, lsets[i % R][0], b0, tile=w.tile, out=lsets[i % R][1])

        ms = graph_ms(torch, lstep, K)
        torch.cuda._sleep(int(2.4e9 * 0.05))      # queued work ahead of the stamped launches
        mr.moe_profile_begin()
        for i in range(min(K, 50)):
            lstep(i)
        mr.moe_profile_end()
        torch.cuda.synchronize()
        rms, rn = mr.moe_profile_read(mr.MOE_KERNEL_ROUTE)
        route_us = rms / rn * 1000.0 if rn else None
        route_b = w.T * w.E * 2 + w.E * 4 + 2 * w.T * w.k * 4
        total = int(o0.total_num_padded_tokens.item())
        ntiles = int(o0.num_non_exiting_ctas.item())
        nbytes = route_permute_bytes(w, w.T, total, ntiles)
        res["deepseek_v3_like_T262144"] = {
            "workload": w.description.replace("T=16384", "T=262144"),
            "us_per_call": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "gbs": nbytes / (ms * 1e-3) / 1e9, "buffer_sets": R,
            "route_kernel_us": route_us, "route_kernel_algorithmic_bytes": route_b,
            "route_kernel_gbs": route_b / (route_us * 1e-6) / 1e9 if route_us else None,
            "route_kernel_frac_of_peak": route_b / (route_us * 1e-6) / 1e9 / HBM_PEAK_GBS if route_us else None}
        del lsets, x0, o0

    if want("deepseek_v3_like_bf16_weights"):
        # the headline method with bfloat16 routing weights (FlashInfer's
        # topk_weights dtype): the same step, 2-byte weights
        w = WORKLOADS["deepseek_v3_like"]
        logits, bias = route_inputs(w)
        x0 = dev_logits(w, logits)
        b0 = torch.from_numpy(bias).to(dev)
        args = mr.make_route_args(w.T, w.E, w.k, score_fn=w.score_fn, n_group=w.n_group,
                                  topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                                  scale=w.scale, logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype,
                                  weights_dtype="bf16")
        o0 = mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile)
        sb = x0.numel() * x0.element_size() + sum(
            t.numel() * t.element_size() for t in vars(o0).values() if isinstance(t, torch.Tensor))
        R = n_sets(sb, rotate_mb)
        hsets = [(x0 if r == 0 else x0.clone(),
                  o0 if r == 0 else mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile))
                 for r in range(R)]
        ms = graph_ms(torch, lambda i: mr.route_permute(args, hsets[i % R][0], b0, tile=w.tile,
                                                        out=hsets[i % R][1]), K)
        total = int(o0.total_num_padded_tokens.item())
        ntiles = int(o0.num_non_exiting_ctas.item())
        nbytes = route_permute_bytes(w, w.T, total, ntiles) - w.T * w.k * 2
        res["deepseek_v3_like_bf16_weights"] = {
            "workload": w.description + "; bf16 topk_weights",
            "us_per_call": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "gbs": nbytes / (ms * 1e-3) / 1e9, "buffer_sets": R}
        del hsets, x0, o0

    if want("deepseek_v3_like_dispatch") or want("deepseek_v3_like_combine"):
        # token dispatch and combine around the expert GEMM, DeepSeek-V3-like route
        # at the front end's hidden size (7168, bf16), rows of synthetic N(0,1)
        w = WORKLOADS["deepseek_v3_like"]
        logits, bias = route_inputs(w)
        x0 = dev_logits(w, logits)
        b0 = torch.from_numpy(bias).to(dev)
        args = mr.make_route_args(w.T, w.E, w.k, score_fn=w.score_fn, n_group=w.n_group,
                                  topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                                  scale=w.scale, logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)
        o = mr.alloc_route_outputs(args, dev, permute=True, tile=w.tile)
        mr.route_permute(args, x0, b0, tile=w.tile, out=o)
        torch.cuda.synchronize()
        H = FRONT_END.H
        total = int(o.total_num_padded_tokens.item())
        max_rows = o.permuted_idx_to_token_idx.numel()
        gen = torch.Generator(device="cpu").manual_seed(w.seed + 2)
        hid0 = torch.randn((w.T, H), generator=gen).to(torch.bfloat16).to(dev)
        d_bytes = total * H * 2 + w.T * w.k * H * 2 + total * 4          # rows written + read, p2t
        c_bytes = w.T * w.k * H * 2 + w.T * H * 2 + w.T * w.k * 8        # rows read + written, maps
        R = n_sets(max_rows * H * 2 + w.T * H * 2, rotate_mb)
        dsets = [(hid0 if r == 0 else hid0.clone(),
                  torch.empty((max_rows, H), dtype=torch.bfloat16, device=dev)) for r in range(R)]
        ms_d = graph_ms(torch, lambda i: mr.moe_dispatch(
            dsets[i % R][0], mr.MOE_BF16, w.T, H, o.permuted_idx_to_token_idx,
            o.total_num_padded_tokens, max_rows, dsets[i % R][1]), K)
        csets = [(ds[1], torch.empty((w.T, H), dtype=torch.bfloat16, device=dev)) for ds in dsets]
        ms_c = graph_ms(torch, lambda i: mr.moe_combine(
            csets[i % R][0], mr.MOE_BF16, w.T, H, w.k, o.expanded_idx_to_permuted_idx, o.topk_weights,
            mr.MOE_F32, csets[i % R][1]), K)
        del dsets, csets, o
        res["deepseek_v3_like_dispatch"] = {
            "workload": f"{w.description}; hidden [{w.T},{H}] bf16 rows into {total} permuted rows",
            "us_per_call": ms_d * 1e3, "algorithmic_bytes": d_bytes, "gbs": d_bytes / (ms_d * 1e-3) / 1e9,
            "buffer_sets": R,
            "plain_torch_op": plain_op_entry(
                torch, rotate_mb, K, f"copy of a [{total},{H}] bf16 tensor (copy_)", total * H * 4,
                lambda: (torch.empty((total, H), dtype=torch.bfloat16, device=dev),
                         torch.empty((total, H), dtype=torch.bfloat16, device=dev)),
                lambda a, b: b.copy_(a))}
        res["deepseek_v3_like_combine"] = {
            "workload": f"{w.description}; {w.k} weighted expert rows per token back to [{w.T},{H}] bf16",
            "us_per_call": ms_c * 1e3, "algorithmic_bytes": c_bytes, "gbs": c_bytes / (ms_c * 1e-3) / 1e9,
            "buffer_sets": R,
            "plain_torch_op": plain_op_entry(
                torch, rotate_mb, K, f"sum over k of a [{w.T},{w.k},{H}] bf16 tensor (torch.sum)",
                w.T * w.k * H * 2 + w.T * H * 2,
                lambda: (torch.empty((w.T, w.k, H), dtype=torch.bfloat16, device=dev),
                         torch.empty((w.T, H), dtype=torch.bfloat16, device=dev)),
                lambda a, b: torch.sum(a, dim=1, out=b))}

    if want("decode_front_end"):
        res["decode_front_end"] = front_end_bench(mr, torch, np, dev, rotate_mb, K, cpu_seconds)
    return res


def front_end_bench(mr, torch, np, dev, rotate_mb, K, cpu_seconds=None):
    """The decode front end (RMSNorm -> projection -> top-k), cold (rotating sets):
    microseconds per call, algorithmic GB/s and projection TFLOP/s; with
    cpu_seconds, the near-tie count of its output under the float32-summation
    rule and the oracle timed on the host (BLAS threads pinned to the CPUs this
    process may use)."""
    from workloads import FRONT_END, front_end_inputs
    f = FRONT_END
    hidden, gamma, W, _ = front_end_inputs(f)
    def bf(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    h0, g0, w0 = bf(hidden), bf(gamma), bf(W)
    set_b = (2 * f.T * f.H + f.H * f.E) * 2 + f.T * f.k * 4 + f.T * f.E * 2
    R = n_sets(set_b, rotate_mb)
    fsets = []
    for r in range(R):
        fsets.append((h0.clone(), w0.clone(), torch.empty((f.T, f.H), dtype=torch.bfloat16, device=dev),
                      torch.empty((f.T, f.k), dtype=torch.int32, device=dev),
                      torch.empty((f.T, f.E), dtype=torch.bfloat16, device=dev)))
    wsf = torch.zeros(max(mr.rmsnorm_gate_route_workspace_size(f.T, f.H, f.E), 1), dtype=torch.uint8,
                      device=dev)

    def fstep(i):
        h, wt, nm, ids, aff = fsets[i % R]
        mr.rmsnorm_gate_route(h, g0, wt, None, mr.MOE_BF16, f.T, f.H, f.E, f.eps, f.k,
                              mr.MOE_SIGMOID, nm, ids, aff, workspace=wsf)

    ms = graph_ms(torch, fstep, K)
    # both launches of a call under the library's event brackets, queue backlogged
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.02))
    mr.moe_profile_begin()
    for i in range(min(K, 100)):
        fstep(i)
    mr.moe_profile_end()
    torch.cuda.synchronize()
    pms, pn = mr.moe_profile_read(mr.MOE_KERNEL_FRONT_END)
    kernel_us = pms / pn * 1e3 if pn else None
    fb = 2 * f.T * f.H * 2 + f.H * 2 + f.H * f.E * 2 + f.T * f.k * 4 + f.T * f.E * 2
    flops = 2 * f.T * f.H * f.E
    entry = {"workload": f.description, "us_per_call": ms * 1e3,
             "tokens_per_s": f.T / (ms * 1e-3), "algorithmic_bytes": fb,
             "gbs": fb / (ms * 1e-3) / 1e9, "mfma_tflops": flops / (ms * 1e-3) / 1e12,
             "kernel_us_per_call": kernel_us, "buffer_sets": R}
    if cpu_seconds:
        import oracle
        from threadpoolctl import threadpool_limits
        h, _, nm, ids, _ = fsets[0]
        normed_bits = nm.view(torch.int16).cpu().numpy().view(np.uint16)
        depth = mr.rmsnorm_gate_route_sum_depth(f.H)
        ncpu = len(os.sched_getaffinity(0))
        with threadpool_limits(limits=ncpu):
            res = oracle.front_end_route(normed_bits, W, f.k, act=f.act)
            ex, *_ = oracle.fp32_sum_near_ties(res, f.k, depth)
            differ = np.any(ids.cpu().numpy() != res.ids, axis=1)
            entry["near_ties"] = {
                "rule": f"deciding logit gap below the float32 summation bound, depth {depth}",
                "near_tie_tokens": int(ex.sum()), "ids_differ_from_oracle": int(differ.sum()),
                "differing_outside_near_ties": int(np.sum(differ & ~ex)), "tokens": f.T}
            times = []
            while sum(times) < cpu_seconds or not times:
                t0 = time.perf_counter()
                _, nb = oracle.rmsnorm(hidden, gamma, f.eps)
                oracle.front_end_route(nb, W, f.k, act=f.act)
                times.append(time.perf_counter() - t0)
        med = sorted(times)[len(times) // 2]
        entry["cpu_baseline"] = {
            "value": f.T * len(times) / sum(times), "unit": "tokens/s", "cores": ncpu,
            "kind": "oracle",
            "sample": f"all {f.T} tokens, oracle RMSNorm + float64 projection + top-k, "
                      f"{len(times)} repetitions in {sum(times):.1f} s (median {med * 1e3:.1f} ms); "
                      f"BLAS limited to the {ncpu} CPUs of this process's affinity",
            "median_tokens_per_s": f.T / med}
    return entry


def copy_calibration(torch, dev, mb):
    """Three plain device copies of mb MiB: the kernel of known size whose
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings scale other kernels' readings."""
    n = mb * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 3,
            "op": "torch copy_ of a float32 tensor"}


def cpu_baseline(w, sample_T: int, seconds: float):
    """The oracle (route + permute) on a bounded sample of the same workload."""
    import numpy as np  # noqa: F401
    import oracle
    from workloads import route_inputs
    logits, bias = route_inputs(w, T=sample_T)
    times = []
    while sum(times) < seconds or not times:
        t0 = time.perf_counter()
        r = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn,
                         pre_softmax=w.pre_softmax, n_group=w.n_group,
                         topk_group=w.topk_group, group_topn=w.group_topn, renorm=w.renorm,
                         scale=w.scale, bias=bias, bias_dtype=w.bias_dtype)
        oracle.permute(r.ids, w.tile, num_experts=w.E)
        times.append(time.perf_counter() - t0)
    t_total = sum(times)
    return sample_T * len(times) / t_total, len(times), t_total, sorted(times)[len(times) // 2]


def cpu_baseline_entry(w, seconds: float, max_T: int = 4096):
    """cpu_baseline object for a routing workload: the oracle timed on the host."""
    sample_T = min(w.T, max_T)
    tps, reps, secs, med = cpu_baseline(w, sample_T, seconds)
    return {"value": tps, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample_T} of {w.T} tokens of the same workload, oracle route + "
                      f"permute, {reps} repetitions in {secs:.1f} s (median "
                      f"{med * 1e3:.1f} ms each); NumPy elementwise work on one core",
            "median_tokens_per_s": sample_T / med}


def near_tie_entry(w, logits, bias, ids_gpu):
    """Near-tie tokens of a workload by the oracle's rule (a deciding exact-key
    gap in (0, 1e-6) relative), and how many tokens' ids the GPU returned
    differently from the oracle (each of them must be a near-tie token)."""
    import numpy as np
    import oracle
    ref = oracle.route(logits, w.logits_dtype, w.k, score_fn=w.score_fn,
                       pre_softmax=w.pre_softmax, n_group=w.n_group, topk_group=w.topk_group,
                       group_topn=w.group_topn, renorm=w.renorm, scale=w.scale, bias=bias,
                       bias_dtype=w.bias_dtype)
    differ = np.any(ids_gpu != ref.ids, axis=1)
    return {"near_tie_tokens": int(ref.exempt.sum()), "ids_differ_from_oracle": int(differ.sum()),
            "differing_outside_near_ties": int(np.sum(differ & ~ref.exempt)), "tokens": int(w.T)}


def host_info():
    """The host the CPU baseline ran on: CPU model, CPUs, affinity, BLAS threads."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")}
                for d in threadpool_info()]
    except Exception:                                   # threadpoolctl absent or failing
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "blas": blas}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this routing path runs on one GPU; --gpus {a.gpus} is not supported "
              "(tokens shard independently: each GPU routes its own rows with replicated router state)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import top_expert_routing_amd as mr
    from workloads import WORKLOADS, route_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.workload == "decode_front_end":
        # the decode front end alone (for counter passes over its two kernels)
        fe = {"workload": "decode_front_end", "steps": a.steps,
              **front_end_bench(mr, torch, np, dev, a.rotate_mb, a.steps)}
        if a.copy_calibration_mb:
            fe["copy_calibration"] = copy_calibration(torch, dev, a.copy_calibration_mb)
        print(json.dumps(fe), flush=True)
        return
    w = WORKLOADS[a.workload]
    T, E, k, tile = w.T, w.E, w.k, w.tile

    logits_np, bias_np = route_inputs(w)
    if w.logits_dtype == "bf16":
        x0 = torch.from_numpy(logits_np.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        x0 = torch.from_numpy(logits_np).to(dev)
    b0 = None
    if bias_np is not None:
        b0 = torch.from_numpy(bias_np).to(dev) if w.bias_dtype == "f32" else \
            torch.from_numpy(bias_np.view(np.int16)).to(dev).view(torch.bfloat16)
    args = mr.make_route_args(T, E, k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                              n_group=w.n_group, topk_group=w.topk_group,
                              group_topn=w.group_topn, renorm=w.renorm, scale=w.scale,
                              logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)

    # rotating sets: inputs and outputs of a step, repeated past 2x the MALL
    probe = mr.alloc_route_outputs(args, dev, permute=True, tile=tile)
    out_bytes = sum(t.numel() * t.element_size() for t in vars(probe).values()
                    if isinstance(t, torch.Tensor))
    set_bytes = x0.numel() * x0.element_size() + out_bytes
    R = max(2, math.ceil(max(a.rotate_mb * 2 ** 20, 2 * MALL_BYTES + 1) / set_bytes))
    sets = []
    for r in range(R):
        x = x0.clone()
        o = probe if r == 0 else mr.alloc_route_outputs(args, dev, permute=True, tile=tile)
        sets.append((x, o))

    def step(i):
        x, o = sets[i % R]
        mr.route_permute(args, x, b0, tile=tile, out=o)

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: a HIP graph of exactly K steps --------------------------------
    K = a.steps
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for i in range(K):
            step(i)
    g.replay()                      # first replay uploads the graph
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / K

    # ---- per-kernel durations: library event brackets, backlogged queue -------------
    nprof = min(K, 200)
    torch.cuda._sleep(int(2.4e9 * 0.05))      # ~50 ms of queued work ahead of the brackets
    mr.moe_profile_begin()
    for i in range(nprof):
        step(i)
    mr.moe_profile_end()
    torch.cuda.synchronize()
    kt = {}
    for name, kind in (("route_kernel", mr.MOE_KERNEL_ROUTE),
                       ("scatter_kernel", mr.MOE_KERNEL_SCATTER)):
        ms, n = mr.moe_profile_read(kind)
        kt[name] = (ms / n * 1000.0) if n else None      # microseconds

    # ---- algorithmic bytes --------------------------------------------------------------
    o = sets[0][1]
    total = int(o.total_num_padded_tokens.item())
    ntiles = int(o.num_non_exiting_ctas.item())
    lsz = 2 if w.logits_dtype == "bf16" else 4
    route_bytes = T * E * lsz + (E * 4 if w.has_bias else 0) + T * k * 4 + T * k * 4
    step_bytes = (route_bytes + T * k * 4 + total * 4 + 2 * ntiles * 4 + E * 4 + (E + 1) * 4 + 8)
    route_us = kt["route_kernel"]
    achieved = route_bytes / (route_us * 1e-6) / 1e9 if route_us else None
    traffic = load_traffic(a.workload)

    warm = None
    if not a.no_warm:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=cap):
            for i in range(K):
                x, o0 = sets[0]
                mr.route_permute(args, x, b0, tile=tile, out=o0)
        gw.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gw.replay()
        e1.record()
        torch.cuda.synchronize()
        warm = e0.elapsed_time(e1) / K

    others = None
    if not a.no_other_configs and a.workload == "deepseek_v3_like":
        others = other_configs(mr, torch, np, dev, a.rotate_mb, min(K, 50),
                               cpu_seconds=None if a.no_cpu_baseline else a.cpu_seconds_other,
                               only=None if a.only_other is None else set(a.only_other.split(",")))

    cpu = None
    near = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline_entry(w, a.cpu_seconds)
        cpu["host"] = host_info()
        near = near_tie_entry(w, logits_np, bias_np, sets[0][1].topk_ids.cpu().numpy())

    line = {
        "metric": "routed tokens/sec + achieved HBM GB/s, T=16384 E=256 k=8 grouped sigmoid",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "T": T, "E": E, "k": k, "tile_tokens_dim": tile,
            "logits_dtype": w.logits_dtype,
            "step": "moe_route_permute (route + scatter kernels)",
            "timing": f"HIP graph of {K} steps, {R} rotating buffer sets "
                      f"({R * set_bytes / 2**20:.0f} MiB, cold in L2 and MALL)",
        },
        "step_hbm_gbs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_algorithmic_bytes": step_bytes,
        "kernel_us": kt,
        "roofline": {
            "kernel": "route_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": route_bytes,
        },
        "cpu_baseline": cpu,
        "near_ties": near,
        "wall_s_timed_region": wall,
    }
    if warm is not None:
        line["warm_single_set_ms_per_step"] = warm
    if others is not None:
        line["other_configs"] = others
    if a.copy_calibration_mb:
        line["copy_calibration"] = copy_calibration(torch, dev, a.copy_calibration_mb)
    s = json.dumps(line)
    print(s, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
