"""Python binding of libmoe_route.so, the gfx950 MoE top-k routing library.

Argument marshalling only: each function below has the name of a C entry
point declared in include/moe_route.h, takes torch tensors (device memory) or
None for its pointer arguments, passes their data pointers and torch's current
HIP stream, and raises ``MoeError`` on a non-zero status.  Every step of the
routing runs in the library's HIP kernels; there is no Python or CPU fallback,
and importing this package fails if the library has not been built
(``python top_expert_routing_amd/_build.py``).

``alloc_*`` helpers allocate correctly shaped output tensors; ``route`` and
``route_permute`` combine allocation and the call for convenience.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

from . import _lib
from ._lib import (MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP,
                   MOE_F32, MOE_BF16, MOE_F16, MOE_SOFTMAX, MOE_SIGMOID, MoeError,
                   moe_route_args, LIB_PATH, MOE_KERNEL_ROUTE, MOE_KERNEL_COUNTS,
                   MOE_KERNEL_SCATTER, MOE_KERNEL_AUX_FWD, MOE_KERNEL_AUX_BWD,
                   MOE_KERNEL_FRONT_END, MOE_KERNEL_ROUTE_BWD,
                   MOE_KERNEL_DISPATCH, MOE_KERNEL_COMBINE, MOE_KERNEL_DENSE)

__all__ = [
    "moe_route", "moe_route_permute", "moe_aux_loss", "rmsnorm_gate_route", "moe_route_backward",
    "moe_dispatch", "moe_combine", "moe_topk_to_dense",
    "moe_route_workspace_size", "moe_route_count_region_bytes", "moe_aux_loss_workspace_size",
    "moe_aux_loss_sync_region_bytes", "moe_profile_begin", "moe_profile_end", "moe_profile_read",
    "rmsnorm_gate_route_workspace_size", "rmsnorm_gate_route_sync_region_bytes",
    "rmsnorm_gate_route_sum_depth",
    "moe_max_padded_tokens", "moe_max_tiles",
    "make_route_args", "route", "route_permute", "MoeError", "moe_route_args", "LIB_PATH",
    "moe_route_permute_noalloc", "moe_route_permute_noalloc_max_scratch_bytes",
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_EHIP",
    "MOE_F32", "MOE_BF16", "MOE_F16", "MOE_SOFTMAX", "MOE_SIGMOID",
]

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "f16": MOE_F16}
_SF = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}


_ESZ = {MOE_F32: 4, MOE_BF16: 2, MOE_F16: 2}


def _esz(dtype: int) -> int:
    return _ESZ.get(int(dtype), 0)


def _ptr(t, need: int = 0, name: str = "tensor"):
    """Device pointer of a contiguous tensor.  `need`: the bytes the call reads
    or writes there, from the call's own sizes (0: not checked); a smaller
    tensor is refused before anything is launched."""
    if t is None:
        return None
    have = t.numel() * t.element_size()
    if need > 0 and have < need:
        raise ValueError(f"{name}: {have} bytes, the call needs {need}")
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be device tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, _lib.last_error_message())


def make_route_args(T: int, E: int, k: int, score_fn: str = "softmax", pre_softmax: bool = True,
                    n_group: int = 0, topk_group: int = 0, group_topn: int = 2,
                    renorm: bool = True, scale: float = 1.0, logits_dtype: str = "f32",
                    bias_dtype: str = "f32", weights_dtype: str = "f32") -> moe_route_args:
    return moe_route_args(
        num_tokens=T, num_experts=E, top_k=k, score_fn=_SF[score_fn],
        use_pre_softmax=int(bool(pre_softmax)), n_group=n_group, topk_group=topk_group,
        group_score_topn=group_topn, renormalize=int(bool(renorm)),
        routed_scaling_factor=float(scale), logits_dtype=_DT[logits_dtype],
        bias_dtype=_DT[bias_dtype], weights_dtype=_DT[weights_dtype])


# ---- the C entry points ---------------------------------------------------------------

def _route_sizes(args: moe_route_args):
    """Bytes of the [T, E] logits, the [E] bias, the [T, k] ids and weights and
    the [T, E] scores that a routing call touches (0 where a size is invalid:
    the library then reports it)."""
    T, E, k = args.num_tokens, args.num_experts, args.top_k
    if T <= 0 or E <= 0 or k <= 0:
        return dict(logits=0, bias=0, ids=0, weights=0, scores=0, counts=0)
    return dict(logits=T * E * _esz(args.logits_dtype), bias=E * _esz(args.bias_dtype),
                ids=T * k * 4, weights=T * k * _esz(args.weights_dtype), scores=T * E * 4,
                counts=E * 4)


def moe_route(args: moe_route_args, logits, bias, topk_ids, topk_weights, scores=None,
              expert_counts=None, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    n = _route_sizes(args)
    _check(_lib.lib.moe_route(ctypes.byref(args), _ptr(logits, n["logits"], "logits"),
                              _ptr(bias, n["bias"], "bias"), _ptr(topk_ids, n["ids"], "topk_ids"),
                              _ptr(topk_weights, n["weights"], "topk_weights"),
                              _ptr(scores, n["scores"], "scores"),
                              _ptr(expert_counts, n["counts"], "expert_counts"),
                              _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream)))


def _permute_ptrs(args, tile, n_loc, logits, bias, topk_ids, topk_weights, scores,
                  expert_counts, padded_offsets, total, nctas, e2p, p2t, batch_idx, mn_limit):
    n = _route_sizes(args)
    T, k = args.num_tokens, args.top_k
    mp = mt = 0
    if T > 0 and k > 0 and n_loc > 0 and tile > 0:
        mp = max(0, int(_lib.lib.moe_max_padded_tokens(T, k, n_loc, tile)))
        mt = max(0, int(_lib.lib.moe_max_tiles(T, k, n_loc, tile)))
    loc = max(0, n_loc)
    return (_ptr(logits, n["logits"], "logits"), _ptr(bias, n["bias"], "bias"),
            _ptr(topk_ids, n["ids"], "topk_ids"), _ptr(topk_weights, n["weights"], "topk_weights"),
            _ptr(scores, n["scores"], "scores"), _ptr(expert_counts, loc * 4, "expert_counts"),
            _ptr(padded_offsets, (loc + 1) * 4 if loc else 0, "padded_offsets"),
            _ptr(total, 4, "total_num_padded_tokens"), _ptr(nctas, 4, "num_non_exiting_ctas"),
            _ptr(e2p, n["ids"], "expanded_idx_to_permuted_idx"),
            _ptr(p2t, mp * 4, "permuted_idx_to_token_idx"),
            _ptr(batch_idx, mt * 4, "cta_idx_xy_to_batch_idx"),
            _ptr(mn_limit, mt * 4, "cta_idx_xy_to_mn_limit"))


def moe_route_permute(args: moe_route_args, tile_tokens_dim: int, local_expert_offset: int,
                      local_num_experts: int, logits, bias, topk_ids, topk_weights, scores,
                      expert_counts, padded_offsets, total_num_padded_tokens,
                      num_non_exiting_ctas, expanded_idx_to_permuted_idx,
                      permuted_idx_to_token_idx, cta_idx_xy_to_batch_idx,
                      cta_idx_xy_to_mn_limit, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p = _permute_ptrs(args, tile_tokens_dim, local_num_experts, logits, bias, topk_ids,
                      topk_weights, scores, expert_counts, padded_offsets,
                      total_num_padded_tokens, num_non_exiting_ctas,
                      expanded_idx_to_permuted_idx, permuted_idx_to_token_idx,
                      cta_idx_xy_to_batch_idx, cta_idx_xy_to_mn_limit)
    _check(_lib.lib.moe_route_permute(
        ctypes.byref(args), tile_tokens_dim, local_expert_offset, local_num_experts, *p,
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream)))


def moe_route_permute_noalloc(args: moe_route_args, tile_tokens_dim: int,
                              local_expert_offset: int, local_num_experts: int, logits, bias,
                              topk_ids, topk_weights, scores, expert_counts, padded_offsets,
                              total_num_padded_tokens, num_non_exiting_ctas,
                              expanded_idx_to_permuted_idx, permuted_idx_to_token_idx,
                              cta_idx_xy_to_batch_idx, cta_idx_xy_to_mn_limit,
                              stream=None) -> None:
    p = _permute_ptrs(args, tile_tokens_dim, local_num_experts, logits, bias, topk_ids,
                      topk_weights, scores, expert_counts, padded_offsets,
                      total_num_padded_tokens, num_non_exiting_ctas,
                      expanded_idx_to_permuted_idx, permuted_idx_to_token_idx,
                      cta_idx_xy_to_batch_idx, cta_idx_xy_to_mn_limit)
    _check(_lib.lib.moe_route_permute_noalloc(
        ctypes.byref(args), tile_tokens_dim, local_expert_offset, local_num_experts, *p,
        _stream(stream)))


def moe_route_permute_noalloc_max_scratch_bytes() -> int:
    return int(_lib.lib.moe_route_permute_noalloc_max_scratch_bytes())


def moe_aux_loss(probs, tokens_per_expert, rows: int, total_num_tokens: int, num_experts: int,
                 top_k: int, coeff: float, loss=None, grad_loss=None, grad_probs=None,
                 workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    re = rows * num_experts * 4 if rows > 0 and num_experts > 0 else 0
    _check(_lib.lib.moe_aux_loss(
        _ptr(probs, re, "probs"), _ptr(tokens_per_expert, max(0, num_experts) * 4, "tokens_per_expert"),
        ctypes.c_int64(rows), ctypes.c_int64(total_num_tokens), num_experts, top_k,
        ctypes.c_float(coeff), _ptr(loss, 4, "loss"), _ptr(grad_loss, 4, "grad_loss"),
        _ptr(grad_probs, re, "grad_probs"), _ptr(workspace), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def moe_route_backward(args: moe_route_args, logits, topk_ids, grad_weights, grad_scores,
                       grad_logits, stream=None) -> None:
    n = _route_sizes(args)
    _check(_lib.lib.moe_route_backward(ctypes.byref(args), _ptr(logits, n["logits"], "logits"),
                                       _ptr(topk_ids, n["ids"], "topk_ids"),
                                       _ptr(grad_weights, n["ids"], "grad_weights"),
                                       _ptr(grad_scores, n["scores"], "grad_scores"),
                                       _ptr(grad_logits, n["scores"], "grad_logits"),
                                       _stream(stream)))


def moe_topk_to_dense(T: int, E: int, top_k: int, topk_ids, topk_weights, weights_dtype: int,
                      probs=None, routing_map=None, stream=None) -> None:
    tk = T * top_k if T > 0 and top_k > 0 else 0
    te = T * E if T > 0 and E > 0 else 0
    _check(_lib.lib.moe_topk_to_dense(T, E, top_k, _ptr(topk_ids, tk * 4, "topk_ids"),
                                      _ptr(topk_weights, tk * _esz(weights_dtype), "topk_weights"),
                                      weights_dtype, _ptr(probs, te * 4, "probs"),
                                      _ptr(routing_map, te, "routing_map"), _stream(stream)))


def moe_dispatch(hidden, dtype: int, T: int, H: int, permuted_idx_to_token_idx,
                 total_num_padded_tokens, max_padded_tokens: int, permuted_hidden,
                 stream=None) -> None:
    th = T * H * _esz(dtype) if T > 0 and H > 0 else 0
    mp = max(0, max_padded_tokens)
    _check(_lib.lib.moe_dispatch(_ptr(hidden, th, "hidden"), dtype, T, H,
                                 _ptr(permuted_idx_to_token_idx, mp * 4, "permuted_idx_to_token_idx"),
                                 _ptr(total_num_padded_tokens, 4, "total_num_padded_tokens"),
                                 ctypes.c_int64(max_padded_tokens),
                                 _ptr(permuted_hidden, mp * max(0, H) * _esz(dtype), "permuted_hidden"),
                                 _stream(stream)))


def moe_combine(expert_out, dtype: int, T: int, H: int, top_k: int, expanded_idx_to_permuted_idx,
                topk_weights, weights_dtype: int, out, stream=None) -> None:
    tk = T * top_k if T > 0 and top_k > 0 else 0
    th = T * H * _esz(dtype) if T > 0 and H > 0 else 0
    _check(_lib.lib.moe_combine(_ptr(expert_out), dtype, T, H, top_k,
                                _ptr(expanded_idx_to_permuted_idx, tk * 4, "expanded_idx_to_permuted_idx"),
                                _ptr(topk_weights, tk * _esz(weights_dtype), "topk_weights"),
                                weights_dtype, _ptr(out, th, "out"), _stream(stream)))


def rmsnorm_gate_route(hidden, gamma, router_weights, router_bias, dtype: int, T: int, H: int,
                       E: int, eps: float, top_k: int, act_fn: int, normed, topk_ids,
                       affinities, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    es = 2 if int(dtype) in (MOE_BF16, MOE_F16) else 0   # else the library reports the dtype
    ok = T > 0 and H > 0 and E > 0 and top_k > 0 and es > 0
    _check(_lib.lib.rmsnorm_gate_route(
        _ptr(hidden, T * H * es if ok else 0, "hidden"), _ptr(gamma, H * es if ok else 0, "gamma"),
        _ptr(router_weights, H * E * es if ok else 0, "router_weights"),
        _ptr(router_bias, E * es if ok else 0, "router_bias"), dtype, T, H, E,
        ctypes.c_float(eps), top_k, act_fn, _ptr(normed, T * H * es if ok else 0, "normed"),
        _ptr(topk_ids, T * top_k * 4 if ok else 0, "topk_ids"),
        _ptr(affinities, T * E * 2 if ok else 0, "affinities"),
        _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream(stream)))


def moe_route_workspace_size(args: moe_route_args, tile_tokens_dim: int,
                             local_num_experts: int) -> int:
    return int(_lib.lib.moe_route_workspace_size(ctypes.byref(args), tile_tokens_dim,
                                                 local_num_experts))


def moe_route_count_region_bytes() -> int:
    return int(_lib.lib.moe_route_count_region_bytes())


def moe_aux_loss_workspace_size(rows: int, num_experts: int) -> int:
    return int(_lib.lib.moe_aux_loss_workspace_size(ctypes.c_int64(rows), num_experts))


def moe_aux_loss_sync_region_bytes() -> int:
    return int(_lib.lib.moe_aux_loss_sync_region_bytes())


def rmsnorm_gate_route_workspace_size(T: int, H: int, E: int) -> int:
    return int(_lib.lib.rmsnorm_gate_route_workspace_size(T, H, E))


def rmsnorm_gate_route_sync_region_bytes() -> int:
    return int(_lib.lib.rmsnorm_gate_route_sync_region_bytes())


def rmsnorm_gate_route_sum_depth(H: int) -> int:
    return int(_lib.lib.rmsnorm_gate_route_sum_depth(H))


def moe_max_padded_tokens(T: int, k: int, local_num_experts: int, tile: int) -> int:
    return int(_lib.lib.moe_max_padded_tokens(T, k, local_num_experts, tile))


def moe_max_tiles(T: int, k: int, local_num_experts: int, tile: int) -> int:
    return int(_lib.lib.moe_max_tiles(T, k, local_num_experts, tile))


def moe_profile_begin() -> None:
    _check(_lib.lib.moe_profile_begin())


def moe_profile_end() -> None:
    _check(_lib.lib.moe_profile_end())


def moe_profile_read(kernel_kind: int):
    """(total milliseconds, launches) of one kernel kind since moe_profile_begin."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(_lib.lib.moe_profile_read(kernel_kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---- allocation conveniences ------------------------------------------------------------

@dataclass
class RouteOutputs:
    topk_ids: "torch.Tensor"
    topk_weights: "torch.Tensor"
    scores: Optional["torch.Tensor"] = None
    expert_counts: Optional["torch.Tensor"] = None
    padded_offsets: Optional["torch.Tensor"] = None
    total_num_padded_tokens: Optional["torch.Tensor"] = None
    num_non_exiting_ctas: Optional["torch.Tensor"] = None
    expanded_idx_to_permuted_idx: Optional["torch.Tensor"] = None
    permuted_idx_to_token_idx: Optional["torch.Tensor"] = None
    cta_idx_xy_to_batch_idx: Optional["torch.Tensor"] = None
    cta_idx_xy_to_mn_limit: Optional["torch.Tensor"] = None
    workspace: Optional["torch.Tensor"] = None


def alloc_route_outputs(args: moe_route_args, device, scores: bool = False,
                        counts: bool = False, permute: bool = False, tile: int = 8,
                        local_num_experts: Optional[int] = None) -> RouteOutputs:
    import torch
    T, E, k = args.num_tokens, args.num_experts, args.top_k
    wdt = torch.bfloat16 if args.weights_dtype == MOE_BF16 else torch.float32
    out = RouteOutputs(
        topk_ids=torch.empty((T, k), dtype=torch.int32, device=device),
        topk_weights=torch.empty((T, k), dtype=wdt, device=device))
    if scores:
        out.scores = torch.empty((T, E), dtype=torch.float32, device=device)
    n_loc = E if local_num_experts is None else local_num_experts
    if counts or permute:
        out.expert_counts = torch.empty(n_loc, dtype=torch.int32, device=device)
        ws = moe_route_workspace_size(args, tile, n_loc)
        # the counting region must start zero-filled; the library keeps it so
        out.workspace = torch.zeros(max(ws, 1), dtype=torch.uint8, device=device)
    if permute:
        mp = moe_max_padded_tokens(T, k, n_loc, tile)
        mt = moe_max_tiles(T, k, n_loc, tile)
        out.padded_offsets = torch.empty(n_loc + 1, dtype=torch.int32, device=device)
        out.total_num_padded_tokens = torch.empty(1, dtype=torch.int32, device=device)
        out.num_non_exiting_ctas = torch.empty(1, dtype=torch.int32, device=device)
        out.expanded_idx_to_permuted_idx = torch.empty(T * k, dtype=torch.int32, device=device)
        out.permuted_idx_to_token_idx = torch.empty(max(mp, 1), dtype=torch.int32, device=device)
        out.cta_idx_xy_to_batch_idx = torch.empty(max(mt, 1), dtype=torch.int32, device=device)
        out.cta_idx_xy_to_mn_limit = torch.empty(max(mt, 1), dtype=torch.int32, device=device)
    return out


def route(args: moe_route_args, logits, bias=None, scores: bool = False, counts: bool = False,
          out: Optional[RouteOutputs] = None, stream=None) -> RouteOutputs:
    if out is None:
        out = alloc_route_outputs(args, logits.device, scores=scores, counts=counts)
    moe_route(args, logits, bias, out.topk_ids, out.topk_weights, out.scores,
              out.expert_counts, out.workspace, stream)
    return out


def route_permute(args: moe_route_args, logits, bias=None, tile: int = 8,
                  local_expert_offset: int = 0, local_num_experts: Optional[int] = None,
                  scores: bool = False, out: Optional[RouteOutputs] = None,
                  stream=None) -> RouteOutputs:
    n_loc = args.num_experts - local_expert_offset if local_num_experts is None \
        else local_num_experts
    if out is None:
        out = alloc_route_outputs(args, logits.device, scores=scores, permute=True, tile=tile,
                                  local_num_experts=n_loc)
    moe_route_permute(args, tile, local_expert_offset, n_loc, logits, bias, out.topk_ids,
                      out.topk_weights, out.scores, out.expert_counts, out.padded_offsets,
                      out.total_num_padded_tokens, out.num_non_exiting_ctas,
                      out.expanded_idx_to_permuted_idx, out.permuted_idx_to_token_idx,
                      out.cta_idx_xy_to_batch_idx, out.cta_idx_xy_to_mn_limit,
                      out.workspace, stream)
    return out
