"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol include/moe_route.h declares, and rejects invalid arguments with the
documented status before enqueueing anything.

Every call here fails validation, so no kernel is ever launched; the non-NULL
pointer values are never dereferenced."""
import ctypes
import os
import re
import subprocess

import pytest

import top_expert_routing_amd as mr
from top_expert_routing_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "while", "for", "sizeof", "return"})


def test_header_symbols_exported():
    names = _declared_functions()
    assert "moe_route" in names and "rmsnorm_gate_route" in names
    for n in names:
        assert hasattr(_lib.lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", mr.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def _route(args, **kw):
    p = dict(logits=FAKE, bias=None, ids=FAKE, weights=FAKE, scores=None, counts=None,
             ws=None, ws_bytes=0)
    p.update(kw)
    return _lib.lib.moe_route(ctypes.byref(args), p["logits"], p["bias"], p["ids"], p["weights"],
                              p["scores"], p["counts"], p["ws"], p["ws_bytes"], None)


def _permute(args, tile=8, off=0, n_loc=None, **kw):
    n_loc = args.num_experts if n_loc is None else n_loc
    p = dict(ws=FAKE, ws_bytes=1 << 30, counts=FAKE, p2t=FAKE)
    p.update(kw)
    return _lib.lib.moe_route_permute(
        ctypes.byref(args), tile, off, n_loc, FAKE, None, FAKE, FAKE, None, p["counts"], FAKE,
        FAKE, FAKE, FAKE, p["p2t"], FAKE, FAKE, p["ws"], p["ws_bytes"], None)


BAD_ROUTE = [
    (dict(T=-1, E=8, k=2), mr.MOE_EINVAL),
    (dict(T=4, E=0, k=1), mr.MOE_EINVAL),
    (dict(T=4, E=8, k=0), mr.MOE_EINVAL),
    (dict(T=4, E=8, k=9), mr.MOE_EINVAL),
    (dict(T=4, E=4096, k=8), mr.MOE_EUNSUPPORTED),
    (dict(T=4, E=256, k=65), mr.MOE_EUNSUPPORTED),
    (dict(T=4, E=8, k=2, n_group=3, topk_group=1), mr.MOE_EINVAL),        # E % n_group
    (dict(T=4, E=8, k=5, n_group=4, topk_group=2), mr.MOE_EINVAL),        # k > kept experts
    (dict(T=4, E=8, k=2, n_group=2, topk_group=3), mr.MOE_EINVAL),        # topk_group > n_group
    (dict(T=4, E=8, k=2, n_group=2, topk_group=1, group_topn=5), mr.MOE_EINVAL),
    (dict(T=4, E=16, k=2, n_group=2, topk_group=1, group_topn=3), mr.MOE_EUNSUPPORTED),
    (dict(T=4, E=60, k=4, n_group=4, topk_group=2), mr.MOE_EUNSUPPORTED),  # group of 15
    (dict(T=4, E=96, k=4, n_group=4, topk_group=2), mr.MOE_EUNSUPPORTED),  # group of 24 = 8 x 3
    (dict(T=4, E=260, k=4, n_group=65, topk_group=8), mr.MOE_EUNSUPPORTED),  # 65 lanes of 4
    (dict(T=4, E=8, k=2, n_group=-1), mr.MOE_EINVAL),
    (dict(T=4, E=8, k=2, scale=float("inf")), mr.MOE_EINVAL),
    (dict(T=4, E=8, k=2, logits_dtype="f16"), mr.MOE_EINVAL),
]


@pytest.mark.parametrize("kw,status", BAD_ROUTE)
def test_route_validation(kw, status):
    kw = dict(kw)
    args = mr.make_route_args(kw.pop("T"), kw.pop("E"), kw.pop("k"), **kw)
    assert _route(args) == status, _lib.last_error_message()
    assert _lib.last_error_message()
    assert _permute(args) == status


def test_route_null_pointers_and_workspace():
    args = mr.make_route_args(100, 8, 2)
    assert _route(args, logits=None) == mr.MOE_EINVAL
    assert _route(args, ids=None) == mr.MOE_EINVAL
    # counts requested without enough workspace
    assert _route(args, counts=FAKE, ws=FAKE, ws_bytes=4) == mr.MOE_EWORKSPACE
    assert _route(args, counts=FAKE, ws=None, ws_bytes=0) == mr.MOE_EWORKSPACE
    assert _permute(args, ws_bytes=4) == mr.MOE_EWORKSPACE
    # the routing workspace must be 256-byte aligned (its counting region is reused)
    assert _permute(args, ws=ctypes.c_void_p(0x1010)) == mr.MOE_EINVAL
    assert _route(args, counts=FAKE, ws=ctypes.c_void_p(0x1010), ws_bytes=1 << 30) == mr.MOE_EINVAL
    assert _permute(args, counts=None) == mr.MOE_EINVAL
    assert _permute(args, p2t=None) == mr.MOE_EINVAL
    w = ctypes.c_void_p(0x1002)     # misaligned float32 weights
    assert _lib.lib.moe_route(ctypes.byref(args), FAKE, None, FAKE, w, None, None, None, 0,
                              None) == mr.MOE_EINVAL


@pytest.mark.parametrize("tile,off,n_loc,status", [
    (6, 0, 8, mr.MOE_EINVAL), (0, 0, 8, mr.MOE_EINVAL), (2048, 0, 8, mr.MOE_EINVAL),
    (8, -1, 8, mr.MOE_EINVAL), (8, 4, 8, mr.MOE_EINVAL), (8, 0, 0, mr.MOE_EINVAL)])
def test_permute_validation(tile, off, n_loc, status):
    args = mr.make_route_args(100, 8, 2)
    assert _permute(args, tile=tile, off=off, n_loc=n_loc) == status


def test_aux_loss_validation():
    L = _lib.lib.moe_aux_loss
    f = ctypes.c_float
    assert L(FAKE, FAKE, -1, 10, 8, 2, f(0.01), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(FAKE, FAKE, 10, 0, 8, 2, f(0.01), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(FAKE, FAKE, 10, 10, 8, 9, f(0.01), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(FAKE, FAKE, 10, 10, 8, 2, f(0.01), None, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(FAKE, None, 10, 10, 8, 2, f(0.01), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(None, FAKE, 10, 10, 8, 2, f(0.01), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL
    assert L(FAKE, FAKE, 10, 10, 8, 2, f(0.01), FAKE, None, None, FAKE, 0, None) == mr.MOE_EWORKSPACE
    assert L(FAKE, FAKE, 10, 10, 8, 2, f(float("nan")), FAKE, None, None, FAKE, 1 << 20, None) == mr.MOE_EINVAL


def test_size_helpers():
    assert mr.moe_max_padded_tokens(16384, 8, 256, 8) == 16384 * 8 + 256 * 7
    assert mr.moe_max_tiles(16384, 8, 256, 8) == (16384 * 8 + 256 * 7) // 8
    assert mr.moe_max_padded_tokens(10, 2, 8, 3) == -1
    assert mr.moe_max_tiles(-1, 2, 8, 4) == -1
    args = mr.make_route_args(16384, 256, 8)
    region = mr.moe_route_count_region_bytes()
    assert region == 2 * 64 * 2048 * 4 + 256      # fixed: independent of the sizes
    assert mr.moe_route_workspace_size(args, 8, 256) == region + 256 * 256 * 4
    assert mr.moe_route_workspace_size(mr.make_route_args(1, 8, 2), 8, 8) == region + 256
    assert mr.moe_route_workspace_size(args, 8, 256) % 256 == 0
    # the aux forward's workspace is one sync region: a 64-bit partial slot for
    # each of at most 2048 blocks, whatever the sizes
    assert mr.moe_aux_loss_sync_region_bytes() == 2048 * 8
    for rows, E in ((65536, 128), (0, 8), (10 ** 7, 128), (1, 2048)):
        assert mr.moe_aux_loss_workspace_size(rows, E) == 2048 * 8


def test_status_strings():
    for s in range(5):
        assert _lib.lib.moe_status_string(s).decode().startswith(_lib.STATUS_NAMES[s])
    assert b"unknown" in _lib.lib.moe_status_string(99)


def _front(T=128, H=7168, E=256, k=8, dtype=None, act=None, eps=1e-6, ws=FAKE, ws_bytes=1 << 30,
           hidden=FAKE, ids=FAKE):
    dtype = mr.MOE_BF16 if dtype is None else dtype
    act = mr.MOE_SIGMOID if act is None else act
    return _lib.lib.rmsnorm_gate_route(hidden, FAKE, FAKE, None, dtype, T, H, E,
                                       ctypes.c_float(eps), k, act, FAKE, ids, FAKE, ws,
                                       ctypes.c_size_t(ws_bytes), None)


def test_front_end_validation():
    # every call below fails on the host, before anything is launched
    assert _front(T=0) == mr.MOE_EINVAL
    assert _front(T=129) == mr.MOE_EINVAL              # single-tile decode: T <= 128
    assert _front(H=7000) == mr.MOE_EINVAL             # H % 128 != 0
    assert _front(E=24) == mr.MOE_EUNSUPPORTED         # E % 16 != 0
    assert _front(k=257) == mr.MOE_EINVAL              # k > E
    assert _front(k=0) == mr.MOE_EINVAL
    assert _front(dtype=mr.MOE_F32) == mr.MOE_EINVAL
    assert _front(act=7) == mr.MOE_EINVAL
    assert _front(eps=float("nan")) == mr.MOE_EINVAL
    assert _front(hidden=None) == mr.MOE_EINVAL
    assert _front(ids=None) == mr.MOE_EINVAL
    assert _front(ws_bytes=16) == mr.MOE_EWORKSPACE
    assert _front(ws=None) == mr.MOE_EWORKSPACE
    # the synchronisation region is reused across calls: 256-byte alignment
    assert _front(ws=ctypes.c_void_p(0x1010)) == mr.MOE_EINVAL


def test_front_end_workspace_size():
    region = mr.rmsnorm_gate_route_sync_region_bytes()
    assert region == 1024                              # fixed: independent of the sizes
    # sync region + float32 partials [H / 448, T, E]
    assert mr.rmsnorm_gate_route_workspace_size(128, 7168, 256) == region + 16 * 128 * 256 * 4
    for T, H, E in [(1, 128, 16), (37, 2048, 256), (128, 384, 32)]:
        n = mr.rmsnorm_gate_route_workspace_size(T, H, E)
        assert n % 256 == 0 and n >= region + T * E * 4
    assert mr.rmsnorm_gate_route_workspace_size(0, 7168, 256) == 0


def test_route_backward_validation():
    B = _lib.lib.moe_route_backward
    args = mr.make_route_args(64, 256, 8, score_fn="sigmoid", logits_dtype="bf16")
    ok = (ctypes.byref(args), FAKE, FAKE, FAKE, None, FAKE, None)
    # every call below fails on the host, before anything is launched
    assert B(None, *ok[1:]) == mr.MOE_EINVAL
    assert B(ctypes.byref(args), FAKE, FAKE, None, None, FAKE, None) == mr.MOE_EINVAL   # no gradient
    assert B(ctypes.byref(args), None, FAKE, FAKE, None, FAKE, None) == mr.MOE_EINVAL   # no logits
    assert B(ctypes.byref(args), FAKE, None, FAKE, None, FAKE, None) == mr.MOE_EINVAL   # ids needed
    assert B(ctypes.byref(args), FAKE, FAKE, FAKE, None, None, None) == mr.MOE_EINVAL   # no output
    assert B(ctypes.byref(args), FAKE, FAKE, ctypes.c_void_p(0x1002), None, FAKE, None) == mr.MOE_EINVAL
    big = mr.make_route_args(64, 4096, 8)
    assert B(ctypes.byref(big), *ok[1:]) == mr.MOE_EUNSUPPORTED
    bad_k = mr.make_route_args(64, 16, 17)
    assert B(ctypes.byref(bad_k), *ok[1:]) == mr.MOE_EINVAL
    bad_fn = mr.make_route_args(64, 16, 2)
    bad_fn.score_fn = 5
    assert B(ctypes.byref(bad_fn), *ok[1:]) == mr.MOE_EINVAL
    # T = 0 is valid and launches nothing, even with placeholder pointers
    empty = mr.make_route_args(0, 16, 2)
    assert B(ctypes.byref(empty), None, None, None, FAKE, None, None) == mr.MOE_OK


def test_dispatch_combine_validation():
    D, C = _lib.lib.moe_dispatch, _lib.lib.moe_combine
    i64 = ctypes.c_int64
    # every call below fails on the host, before anything is launched
    assert D(FAKE, mr.MOE_F16, 10, 64, FAKE, FAKE, i64(100), FAKE, None) == mr.MOE_EINVAL
    assert D(FAKE, mr.MOE_BF16, 10, 0, FAKE, FAKE, i64(100), FAKE, None) == mr.MOE_EINVAL
    assert D(None, mr.MOE_BF16, 10, 64, FAKE, FAKE, i64(100), FAKE, None) == mr.MOE_EINVAL
    assert D(FAKE, mr.MOE_BF16, 10, 64, FAKE, None, i64(100), FAKE, None) == mr.MOE_EINVAL
    assert D(ctypes.c_void_p(0x1001), mr.MOE_BF16, 10, 64, FAKE, FAKE, i64(100), FAKE, None) == mr.MOE_EINVAL
    assert D(FAKE, mr.MOE_BF16, 0, 64, None, None, i64(0), None, None) == mr.MOE_OK   # nothing to do
    assert C(FAKE, mr.MOE_BF16, 10, 64, 0, FAKE, FAKE, mr.MOE_F32, FAKE, None) == mr.MOE_EINVAL
    assert C(FAKE, mr.MOE_BF16, 10, 64, 65, FAKE, FAKE, mr.MOE_F32, FAKE, None) == mr.MOE_EUNSUPPORTED
    assert C(FAKE, mr.MOE_BF16, 10, 64, 8, FAKE, FAKE, mr.MOE_F16, FAKE, None) == mr.MOE_EINVAL
    assert C(FAKE, mr.MOE_BF16, 10, 64, 8, None, FAKE, mr.MOE_F32, FAKE, None) == mr.MOE_EINVAL
    assert C(FAKE, mr.MOE_F32, 10, 64, 8, FAKE, ctypes.c_void_p(0x1002), mr.MOE_F32, FAKE, None) == mr.MOE_EINVAL
    assert C(None, mr.MOE_BF16, 0, 64, 8, None, None, mr.MOE_F32, None, None) == mr.MOE_OK


def test_topk_to_dense_validation():
    X = _lib.lib.moe_topk_to_dense
    # every call below fails on the host, before anything is launched
    assert X(10, 8, 2, FAKE, FAKE, mr.MOE_F32, None, None, None) == mr.MOE_EINVAL    # no output
    assert X(10, 8, 9, FAKE, FAKE, mr.MOE_F32, FAKE, None, None) == mr.MOE_EINVAL    # k > E
    assert X(10, 4096, 8, FAKE, FAKE, mr.MOE_F32, FAKE, None, None) == mr.MOE_EUNSUPPORTED
    assert X(10, 8, 2, None, FAKE, mr.MOE_F32, FAKE, None, None) == mr.MOE_EINVAL
    assert X(10, 8, 2, FAKE, FAKE, mr.MOE_F16, FAKE, None, None) == mr.MOE_EINVAL
    assert X(10, 8, 2, FAKE, ctypes.c_void_p(0x1002), mr.MOE_F32, FAKE, None, None) == mr.MOE_EINVAL
    assert X(0, 8, 2, None, None, mr.MOE_F32, FAKE, None, None) == mr.MOE_OK         # nothing to do


def test_header_is_plain_c(tmp_path):
    # the boundary is a C ABI: a C11 translation unit that includes the header
    # and takes the address of every entry point compiles as C
    import shutil
    gcc = shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gcc is None or not os.path.isdir(rocm_inc):
        pytest.skip("gcc or the HIP runtime headers are not available")
    names = _declared_functions()
    assert names, "no entry points found in the header"
    src = tmp_path / "abi.c"
    src.write_text('#include "moe_route.h"\nint main(void) {\n  const void* fns[] = {' +
                   ", ".join(f"(const void*){n}" for n in names) +
                   "};\n  return fns[0] == 0;\n}\n")
    res = subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", f"-I{os.path.dirname(HEADER)}",
                          f"-I{rocm_inc}", str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]


def test_binding_refuses_short_tensors():
    # the binding derives each tensor's bytes from the call's own sizes and
    # refuses a shorter one before anything reaches the library (CPU tensors:
    # the size check of an argument comes before its device check, and the
    # arguments are taken in order)
    torch = pytest.importorskip("torch")
    args = mr.make_route_args(64, 256, 8, score_fn="sigmoid", logits_dtype="bf16",
                              weights_dtype="bf16")
    short = torch.empty(64 * 256 - 1, dtype=torch.bfloat16)
    full = torch.empty(64 * 256, dtype=torch.bfloat16)
    ids = torch.empty(64 * 8, dtype=torch.int32)
    w = torch.empty(64 * 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="logits: 32766 bytes, the call needs 32768"):
        mr.moe_route(args, short, None, ids, w)
    with pytest.raises(ValueError, match="device"):      # sizes right: the device check
        mr.moe_route(args, full, None, ids, w)
    with pytest.raises(ValueError, match="logits"):
        mr.moe_route_permute(args, 8, 0, 256, short, None, ids, w, None, None, None, None,
                             None, None, None, None, None, None)
    with pytest.raises(ValueError, match="logits"):
        mr.moe_route_backward(args, short, ids, w, None, None)
    with pytest.raises(ValueError, match="topk_ids"):
        mr.moe_topk_to_dense(64, 256, 8, ids[:-1], w, mr.MOE_BF16, None, None)
    with pytest.raises(ValueError, match="hidden"):
        mr.moe_dispatch(torch.empty(10, dtype=torch.bfloat16), mr.MOE_BF16, 4, 128, None, None,
                        16, None)
    with pytest.raises(ValueError, match="hidden"):
        mr.rmsnorm_gate_route(torch.empty(10, dtype=torch.bfloat16), None, None, None, mr.MOE_BF16,
                              4, 128, 16, 1e-6, 2, mr.MOE_SIGMOID, None, None, None)
    with pytest.raises(ValueError, match="probs"):
        mr.moe_aux_loss(torch.empty(7), None, 4, 4, 2, 1, 0.1)
    # the sizes the other arguments are held to, from their definitions
    n = mr._route_sizes(args)
    assert n == dict(logits=64 * 256 * 2, bias=256 * 4, ids=64 * 8 * 4, weights=64 * 8 * 2,
                     scores=64 * 256 * 4, counts=256 * 4)
    assert mr._route_sizes(mr.make_route_args(0, 256, 8))["logits"] == 0   # T = 0: nothing
