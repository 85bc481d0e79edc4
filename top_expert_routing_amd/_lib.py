"""ctypes declarations of the C ABI in include/moe_route.h.

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_ROUTE_LIB", os.path.join(HERE, "lib", "libmoe_route.so"))

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
MOE_SOFTMAX, MOE_SIGMOID = 0, 1

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE",
                4: "MOE_EHIP"}

# Every symbol the header declares.
EXPORTED = [
    "moe_route", "moe_route_permute", "moe_route_permute_noalloc",
    "moe_route_permute_noalloc_max_scratch_bytes", "moe_aux_loss", "rmsnorm_gate_route", "moe_route_backward",
    "moe_dispatch", "moe_combine", "moe_topk_to_dense",
    "moe_route_workspace_size", "moe_route_count_region_bytes", "moe_aux_loss_workspace_size",
    "moe_aux_loss_sync_region_bytes",
    "rmsnorm_gate_route_workspace_size", "rmsnorm_gate_route_sync_region_bytes",
    "rmsnorm_gate_route_sum_depth",
    "moe_max_padded_tokens", "moe_max_tiles",
    "moe_status_string", "moe_last_error_message", "moe_last_hip_error",
    "moe_profile_begin", "moe_profile_end", "moe_profile_read",
]

MOE_KERNEL_ROUTE, MOE_KERNEL_COUNTS, MOE_KERNEL_SCATTER = 0, 1, 2
MOE_KERNEL_AUX_FWD, MOE_KERNEL_AUX_BWD, MOE_KERNEL_FRONT_END = 3, 4, 5
MOE_KERNEL_ROUTE_BWD, MOE_KERNEL_DISPATCH, MOE_KERNEL_COMBINE, MOE_KERNEL_DENSE = 6, 7, 8, 9


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class moe_route_args(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("score_fn", ctypes.c_int32),
        ("use_pre_softmax", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("group_score_topn", ctypes.c_int32),
        ("renormalize", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("logits_dtype", ctypes.c_int32),
        ("bias_dtype", ctypes.c_int32),
        ("weights_dtype", ctypes.c_int32),
    ]


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return set()
    return {os.path.realpath(p) for p in paths}


def _load():
    # torch supplies device memory and streams; it ships its own HIP runtime.
    # Import it first so that the library's libamdhip64.so.7 dependency binds
    # to that same runtime (matching SONAME): one process, one HIP runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python top_expert_routing_amd/_build.py` "
            "(the routing path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (" +
                          ", ".join(sorted(runtimes)) + "); import torch before anything "
                          "that loads /opt/rocm's libamdhip64")
    vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_float)
    args_p = ctypes.POINTER(moe_route_args)
    lib.moe_route.argtypes = [args_p, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route.restype = i32
    lib.moe_route_permute.argtypes = [args_p, i32, i32, i32] + [vp] * 14 + [sz, vp]
    lib.moe_route_permute.restype = i32
    lib.moe_route_permute_noalloc.argtypes = [args_p, i32, i32, i32] + [vp] * 13 + [vp]
    lib.moe_route_permute_noalloc.restype = i32
    lib.moe_route_permute_noalloc_max_scratch_bytes.argtypes = []
    lib.moe_route_permute_noalloc_max_scratch_bytes.restype = sz
    lib.moe_aux_loss.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.moe_aux_loss.restype = i32
    lib.moe_route_backward.argtypes = [args_p, vp, vp, vp, vp, vp, vp]
    lib.moe_route_backward.restype = i32
    lib.moe_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, i64, vp, vp]
    lib.moe_dispatch.restype = i32
    lib.moe_combine.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, vp, vp]
    lib.moe_combine.restype = i32
    lib.moe_topk_to_dense.argtypes = [i32, i32, i32, vp, vp, i32, vp, vp, vp]
    lib.moe_topk_to_dense.restype = i32
    lib.rmsnorm_gate_route.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp, vp,
                                       vp, vp, sz, vp]
    lib.rmsnorm_gate_route.restype = i32
    lib.moe_route_workspace_size.argtypes = [args_p, i32, i32]
    lib.moe_route_workspace_size.restype = sz
    lib.moe_route_count_region_bytes.argtypes = []
    lib.moe_route_count_region_bytes.restype = sz
    lib.moe_aux_loss_workspace_size.argtypes = [i64, i32]
    lib.moe_aux_loss_workspace_size.restype = sz
    lib.moe_aux_loss_sync_region_bytes.argtypes = []
    lib.moe_aux_loss_sync_region_bytes.restype = sz
    lib.rmsnorm_gate_route_workspace_size.argtypes = [i32, i32, i32]
    lib.rmsnorm_gate_route_workspace_size.restype = sz
    lib.rmsnorm_gate_route_sync_region_bytes.argtypes = []
    lib.rmsnorm_gate_route_sync_region_bytes.restype = sz
    lib.rmsnorm_gate_route_sum_depth.argtypes = [i32]
    lib.rmsnorm_gate_route_sum_depth.restype = i32
    lib.moe_max_padded_tokens.argtypes = [i32, i32, i32, i32]
    lib.moe_max_padded_tokens.restype = i64
    lib.moe_max_tiles.argtypes = [i32, i32, i32, i32]
    lib.moe_max_tiles.restype = i64
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error_message.argtypes = []
    lib.moe_last_error_message.restype = ctypes.c_char_p
    lib.moe_last_hip_error.argtypes = []
    lib.moe_last_hip_error.restype = i32
    lib.moe_profile_begin.argtypes = []
    lib.moe_profile_begin.restype = i32
    lib.moe_profile_end.argtypes = []
    lib.moe_profile_end.restype = i32
    lib.moe_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.moe_profile_read.restype = i32
    return lib


lib = _load()


def last_error_message() -> str:
    return lib.moe_last_error_message().decode()
