"""ctypes loader for the C ABI in include/nvfp4.h (libnvfp4.so, built in-tree).

The library must have been built (``python -m nvfp4_block_scaled_act_amd.build``
or ``__graft_entry__.build()``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
import re
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")
HEADER = os.path.join(HERE, "..", "include", "nvfp4.h")

_lock = threading.Lock()
_lib = None

P = C.c_void_p
I64 = C.c_int64
I32 = C.c_int
SZ = C.c_size_t

STATUS = {0: "ok", 1: "invalid argument", 2: "invalid shape", 3: "alignment", 4: "unsupported", 5: "workspace", 6: "hip"}
ROUTE_W4A16, ROUTE_W4A4 = 0, 1


LAYOUT_TILED = 1


class Weight(C.Structure):
    """Mirror of struct nvfp4_weight."""
    _fields_ = [("data", P), ("N", I64), ("K", I64), ("layout", C.c_int32), ("reserved", C.c_int32)]


class MoeLayout(C.Structure):
    """Mirror of struct nvfp4_moe_layout (byte offsets into the MoE workspace)."""
    _fields_ = [(n, I64) for n in ("x_codes", "x_scales", "counts", "offsets", "tiles", "sorted", "h_codes",
                                   "h_scales", "inv", "ys", "max_tiles", "total_bytes")]


class MoeW4A16Layout(C.Structure):
    """Mirror of struct nvfp4_moe_w4a16_layout (byte offsets into the W4A16 MoE workspace)."""
    _fields_ = [(n, I64) for n in ("counts", "offsets", "tiles", "sorted", "inv", "h", "ys", "max_tiles",
                                   "total_bytes")]


_SIGS = {
    "nvfp4_status_str": (C.c_char_p, [I32]),
    "nvfp4_version": (I32, []),
    "nvfp4_build_source_hash": (C.c_char_p, []),
    "nvfp4_quantize_act": (I32, [P, I64, I64, I64, P, P, P, P]),
    "nvfp4_global_scale": (I32, [P, I64, I64, I64, P, P]),
    "nvfp4_alpha": (I32, [P, P, P, P]),
    "nvfp4_prepared_weight_bytes": (SZ, [I64, I64]),
    "nvfp4_prepare_weight": (I32, [P, P, I64, I64, P, SZ, C.POINTER(Weight), P]),
    "nvfp4_swizzled_scales_bytes": (SZ, [I64, I64]),
    "nvfp4_fused_weight_global": (I32, [P, I64, P, P]),
    "nvfp4_quantize_act_swizzled": (I32, [P, I64, I64, I64, P, P, P, SZ, P]),
    "nvfp4_prepare_weight_swizzled": (I32, [P, P, SZ, I64, I64, P, SZ, C.POINTER(Weight), P]),
    "nvfp4_linear_w4a16": (I32, [P, I64, I64, C.POINTER(Weight), P, P, I64, P]),
    "nvfp4_linear_w4a16_ex": (I32, [P, I64, I64, C.POINTER(Weight), P, P, I64, I32, I32, I32, I32, P]),
    "nvfp4_linear_w4a4": (I32, [P, P, I64, C.POINTER(Weight), P, P, I64, P]),
    "nvfp4_linear_w4a4_ws": (I32, [P, P, I64, C.POINTER(Weight), P, P, I64, P, SZ, P]),
    "nvfp4_linear_w4a4_workspace_bytes": (SZ, [I64, I64, I64]),
    "nvfp4_route": (I32, [I64, I64, I64, I32]),
    "nvfp4_set_route_m_max": (None, [I64]),
    "nvfp4_get_route_m_max": (I64, []),
    "nvfp4_linear_workspace_bytes": (SZ, [I64, I64, I64]),
    "nvfp4_linear": (I32, [P, I64, I64, C.POINTER(Weight), P, P, P, P, I64, P, SZ, C.POINTER(I32), P]),
    "nvfp4_linear_noalloc": (I32, [P, I64, I64, C.POINTER(Weight), P, P, P, P, I64, C.POINTER(I32), P]),
    "nvfp4_stream_read": (I32, [P, SZ, P, P]),
    "nvfp4_gated_mlp_w4a4": (I32, [P, P, I64, C.POINTER(Weight), P, P, P, P, P, P]),
    "nvfp4_moe_route": (I32, [I64, I64, I64, I32]),
    "nvfp4_set_moe_route_tokens_per_expert": (None, [I64]),
    "nvfp4_get_moe_route_tokens_per_expert": (I64, []),
    "nvfp4_moe_dispatch_workspace_bytes": (SZ, [I64, I64, I64, I64, I64, I32]),
    "nvfp4_moe": (I32, [P, I64, I64, P, P, I64, I64, I64, C.POINTER(Weight), C.POINTER(Weight), P, P, P, P, P, P,
                        P, I64, P, SZ, C.POINTER(I32), P]),
    "nvfp4_moe_w4a16_workspace_bytes": (SZ, [I64, I64, I64, I64, I64]),
    "nvfp4_moe_w4a16_workspace_layout": (I32, [I64, I64, I64, I64, I64, C.POINTER(MoeW4A16Layout)]),
    "nvfp4_moe_w4a16": (I32, [P, I64, I64, P, P, I64, I64, I64, C.POINTER(Weight), C.POINTER(Weight), P, P, P,
                              I64, P, SZ, P]),
    "nvfp4_moe_workspace_bytes": (SZ, [I64, I64, I64, I64, I64]),
    "nvfp4_moe_workspace_layout": (I32, [I64, I64, I64, I64, I64, C.POINTER(MoeLayout)]),
    "nvfp4_moe_w4a4": (I32, [P, I64, I64, P, P, I64, I64, I64, C.POINTER(Weight), C.POINTER(Weight), P, P, P, P,
                             P, I64, P, SZ, P, P]),
}


def header_functions() -> list[str]:
    """Names of the functions include/nvfp4.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load libnvfp4.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m nvfp4_block_scaled_act_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            if hasattr(L, name):
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
        from . import build as _build

        want = _build.source_hash()
        got = L.nvfp4_build_source_hash().decode() if hasattr(L, "nvfp4_build_source_hash") else "none"
        if got != want:
            raise RuntimeError(f"{LIB_PATH} was built from other sources (hash {got}, tree {want}): rebuild it "
                               "with python -m nvfp4_block_scaled_act_amd.build")
        _lib = L
        return L


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {STATUS.get(code, code)} (status {code})")
        self.code = code


def check(fn: str, code: int) -> None:
    if code != 0:
        if code in (1, 2, 3, 4, 5):
            raise NVFP4ValueError(fn, code)
        raise NVFP4Error(fn, code)


class NVFP4ValueError(NVFP4Error, ValueError):
    pass
