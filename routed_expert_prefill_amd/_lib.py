"""ctypes loader for libmoe_prefill.so (the C ABI in include/moe_prefill.h)."""
from __future__ import annotations

import ctypes
import os

# MOE_PREFILL_LIB names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree gfx950 build.
LIB_PATH = os.environ.get("MOE_PREFILL_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_prefill.so")

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EALIGN = -3
MOE_EWORKSPACE = -4
MOE_EHIP = -5
MOE_ETOOLARGE = -6
MOE_ROUTE_NOALLOC_MAX_ROUTES = 1 << 20

MOE_W_BF16 = 0
MOE_W_FP8_E4M3_B128 = 1
MOE_ACT_BF16 = 0
MOE_ACT_FP8_E4M3_ROW = 1

EXPORTED = [
    "moe_status_string", "moe_abi_version",
    "moe_route_build_workspace", "moe_route_build",
    "moe_grouped_ffn_workspace", "moe_grouped_ffn",
    "moe_ffn_plan", "moe_ffn_gate_up", "moe_ffn_down",
    "moe_combine", "moe_quant_rows_fp8", "moe_route_topk", "moe_combine_shared",
    "moe_route_build_noalloc",
]


class MoeFfnDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("k", ctypes.c_int32), ("E", ctypes.c_int32),
                ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32)]


_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load the HIP library; raises LibraryNotBuilt when it is missing (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing: build the gfx950 library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [i32]
    lib.moe_abi_version.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_route_build_workspace.restype = sz
    lib.moe_route_build_workspace.argtypes = [i32, i32, i32]
    lib.moe_route_build.restype = i32
    lib.moe_route_build.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_build_noalloc.restype = i32
    lib.moe_route_build_noalloc.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_grouped_ffn_workspace.restype = sz
    lib.moe_grouped_ffn_workspace.argtypes = [ctypes.POINTER(MoeFfnDesc)]
    lib.moe_grouped_ffn.restype = i32
    lib.moe_grouped_ffn.argtypes = [ctypes.POINTER(MoeFfnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, sz, vp]
    dp = ctypes.POINTER(MoeFfnDesc)
    lib.moe_ffn_plan.restype = i32
    lib.moe_ffn_plan.argtypes = [dp, vp, vp, vp, sz, vp]
    lib.moe_ffn_gate_up.restype = i32
    lib.moe_ffn_gate_up.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_ffn_down.restype = i32
    lib.moe_ffn_down.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine.restype = i32
    lib.moe_combine.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp]
    lib.moe_quant_rows_fp8.restype = i32
    lib.moe_quant_rows_fp8.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_combine_shared.restype = i32
    lib.moe_combine_shared.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.moe_route_topk.restype = i32
    lib.moe_route_topk.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().moe_status_string(code).decode()


def check(code: int, what: str) -> None:
    if code != MOE_OK:
        raise RuntimeError(f"{what} failed: {status_string(code)} ({code})")
