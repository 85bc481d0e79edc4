"""moe_route_permute_noalloc (the entry point that allocates nothing) against
moe_route_permute, through the C ABI: every output identical, on calls in a
row that share the library's static scratch (the second and third smaller
than the first).  Sizes beyond the static scratch are refused on the host."""
import ctypes

import pytest

from gpu_helpers import log, to_dev
from workloads import WORKLOADS, route_inputs, with_overrides

torch = pytest.importorskip("torch")
mr = pytest.importorskip("top_expert_routing_amd")

FIELDS = ("topk_ids", "topk_weights", "expert_counts", "padded_offsets",
          "total_num_padded_tokens", "num_non_exiting_ctas", "expanded_idx_to_permuted_idx",
          "permuted_idx_to_token_idx", "cta_idx_xy_to_batch_idx", "cta_idx_xy_to_mn_limit")


def _args(w, T):
    return mr.make_route_args(T, w.E, w.k, score_fn=w.score_fn, pre_softmax=w.pre_softmax,
                              n_group=w.n_group, topk_group=w.topk_group,
                              group_topn=w.group_topn, renorm=w.renorm, scale=w.scale,
                              logits_dtype=w.logits_dtype, bias_dtype=w.bias_dtype)


def _noalloc(args, x, b, tile, o):
    mr.moe_route_permute_noalloc(
        args, tile, 0, args.num_experts, x, b, o.topk_ids, o.topk_weights, None,
        o.expert_counts, o.padded_offsets, o.total_num_padded_tokens, o.num_non_exiting_ctas,
        o.expanded_idx_to_permuted_idx, o.permuted_idx_to_token_idx, o.cta_idx_xy_to_batch_idx,
        o.cta_idx_xy_to_mn_limit)


def test_noalloc_oversize_refused_on_host():
    # refused before anything touches a device: no GPU needed
    w = WORKLOADS["deepseek_v3_like"]
    T = 1 << 20                                  # 16384 blocks x 256 experts of counts
    args = _args(w, T)
    need = mr.moe_route_workspace_size(args, w.tile, w.E)
    assert need > mr.moe_route_permute_noalloc_max_scratch_bytes() == 8 << 20
    from top_expert_routing_amd import _lib
    fake = ctypes.c_void_p(0x1000)             # never dereferenced: refused first
    st = _lib.lib.moe_route_permute_noalloc(ctypes.byref(args), w.tile, 0, w.E,
                                            *([fake] * 13), None)
    assert st == mr.MOE_EUNSUPPORTED
    assert b"scratch" in _lib.lib.moe_last_error_message()


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    calls = [(WORKLOADS["deepseek_v3_like"], 16384),
             (WORKLOADS["deepseek_v3_like"], 4097),
             (WORKLOADS["qwen_moe_like"], 1000),
             (WORKLOADS["qwen_moe_like"], 65536 + 5)]   # scatter blocks of two route blocks
    for i, (w, T) in enumerate(calls):
        label = f"noalloc call {i}: {w.name} T={T}"
        log(f"[gpu] {label}")
        logits, bias = route_inputs(w, T=T, seed=7000 + i)
        x = to_dev(logits, w.logits_dtype)
        b = to_dev(bias, w.bias_dtype) if bias is not None else None
        args = _args(w, T)
        ref = mr.route_permute(args, x, b, tile=w.tile)
        got = mr.alloc_route_outputs(args, "cuda:0", permute=True, tile=w.tile)
        for f in FIELDS:                          # poison every output first
            getattr(got, f).fill_(-7)
        _noalloc(args, x, b, w.tile, got)
        torch.cuda.synchronize()
        total = int(ref.total_num_padded_tokens.item())
        ntiles = int(ref.num_non_exiting_ctas.item())
        for f in FIELDS:
            a, c = getattr(ref, f), getattr(got, f)
            if f == "permuted_idx_to_token_idx":
                a, c = a[:total], c[:total]
            elif f.startswith("cta_idx"):
                a, c = a[:ntiles], c[:ntiles]
            assert torch.equal(a, c), f"{label}: {f} differs"
        log(f"[gpu] {label}: identical to moe_route_permute")
