"""CPU oracle for the NVFP4 quantized linear -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``nvfp4_oracle.cpp``: a plain, slow, obviously correct
C++ definition of activation quantization, the W4A16 and W4A4 linears and the
NVFP4 MoE expert layer (W4A4, and W4A16 for decode-sized batches).  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it, and the two share no code.

Functions whose parity is unpinned: none of the linear-path functions.  The
128x4 scale swizzle (``swizzle_scales_128x4``) is parity unpinned against the
pages, which name the layout without its index map: it follows the public
layout, and its tests pin it to that layout's closed-form byte offset.  The MoE
calibration of the second activation global (max |h| over a calibration batch)
follows a reading, not a passage of the pages, and is parity unpinned as a
choice of value (its arithmetic is the pinned global-scale formula).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.cpp")
_SO = os.path.join(_HERE, "_nvfp4_oracle.so")
_LOCK = threading.Lock()
_LIB = None

_P = C.c_void_p
_I64 = C.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (OpenMP, IEEE double, no fast-math)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
           "-shared", "-fPIC", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
                build(force=True)
            L = C.CDLL(_SO)
            L.orc_e2m1_value.restype = C.c_double
            L.orc_e2m1_value.argtypes = [C.c_int]
            L.orc_e4m3_value.restype = C.c_double
            L.orc_e4m3_value.argtypes = [C.c_int]
            L.orc_e4m3_round.restype = C.c_int
            L.orc_e4m3_round.argtypes = [C.c_double] * 3
            L.orc_e2m1_round.restype = C.c_int
            L.orc_e2m1_round.argtypes = [C.c_double] * 3
            L.orc_bf16_rne.restype = C.c_uint16
            L.orc_bf16_rne.argtypes = [C.c_double]
            L.orc_global_scale.restype = C.c_float
            L.orc_global_scale.argtypes = [_P, _I64, _I64, _I64]
            L.orc_global_scale_from_amax.restype = C.c_float
            L.orc_global_scale_from_amax.argtypes = [C.c_double]
            L.orc_alpha.restype = C.c_float
            L.orc_alpha.argtypes = [C.c_float, C.c_float]
            L.orc_quantize_bf16.restype = None
            L.orc_quantize_bf16.argtypes = [_P, _I64, _I64, _I64, C.c_float, _P, _P]
            L.orc_quantize_f64.restype = None
            L.orc_quantize_f64.argtypes = [_P, _I64, _I64, _I64, C.c_float, _P, _P]
            L.orc_dequant.restype = None
            L.orc_dequant.argtypes = [_P, _P, _I64, _I64, _P]
            L.orc_linear_w4a16.restype = None
            L.orc_linear_w4a16.argtypes = [_P, _I64, _P, _I64, _P, _P, _I64, _P, _I64, C.c_float, _P, _P, _P]
            L.orc_linear_w4a4.restype = None
            L.orc_linear_w4a4.argtypes = [_P, _P, _P, _I64, _P, _P, _I64, _P, _I64, C.c_float, _P, _P, _P]
            L.orc_moe_w4a4.restype = None
            L.orc_moe_w4a4.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P,
                                       C.c_float, C.c_float, _P, _P, _P, _I64,
                                       _P, _P, _P, _P, _P, _P, _P, _P]
            L.orc_moe_w4a16.restype = None
            L.orc_moe_w4a16.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P,
                                        _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P]
            _LIB = L
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(int(byte))


def e4m3_round(x: float, y: float, den: float) -> int:
    """Nearest E4M3 byte to the exact value x*y/den (RNE, saturating)."""
    return lib().orc_e4m3_round(float(x), float(y), float(den))


def e2m1_round(x: float, y: float, den: float) -> int:
    """Nearest e2m1 magnitude index to the exact value x*y/den (RNE, saturating)."""
    return lib().orc_e2m1_round(float(x), float(y), float(den))


def bf16_rne(r: float) -> int:
    return int(lib().orc_bf16_rne(float(r)))


# ---------------------------------------------------------------- scalars
def global_scale(x_bf16: np.ndarray) -> np.float32:
    x = _c(x_bf16, np.uint16)
    x2 = x.reshape(-1, x.shape[-1]) if x.ndim != 2 else x
    return np.float32(lib().orc_global_scale(_ptr(x2), x2.shape[0], x2.shape[1], x2.shape[1]))


def global_scale_from_amax(amax: float) -> np.float32:
    return np.float32(lib().orc_global_scale_from_amax(float(amax)))


def alpha(g_w, g_a=None) -> np.float32:
    return np.float32(lib().orc_alpha(float(g_w), float(g_a) if g_a is not None else 0.0))


# ---------------------------------------------------------------- quantizer
def quantize(x_bf16: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    """bf16 bits [rows, K] -> (codes uint8 [rows, K/2], scales uint8 [rows, K/16])."""
    x = _c(x_bf16, np.uint16)
    rows, K = x.shape
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    lib().orc_quantize_bf16(_ptr(x), rows, K, K, float(np.float32(g)), _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_f64(x: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    x = _c(x, np.float64)
    rows, K = x.shape
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    lib().orc_quantize_f64(_ptr(x), rows, K, K, float(np.float32(g)), _ptr(codes), _ptr(scales))
    return codes, scales


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = codes.shape
    K = 2 * half
    out = np.empty((rows, K), np.float64)
    lib().orc_dequant(_ptr(codes), _ptr(scales), rows, K, _ptr(out))
    return out


# ---------------------------------------------------------------- linears
def _idx(ix, n):
    if ix is None:
        return None, n
    ix = _c(ix, np.int64)
    return ix, len(ix)


def linear_w4a16(a_bf16, w_codes, w_scales, alpha_, rows=None, cols=None):
    """-> (out bf16 bits, ref fp64, sabs fp64), each [n_rows, n_cols]."""
    a = _c(a_bf16, np.uint16)
    wc = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.uint8)
    M, K = a.shape
    N = wc.shape[0]
    r, nr = _idx(rows, M)
    c, nc = _idx(cols, N)
    out = np.empty((nr, nc), np.uint16)
    ref = np.empty((nr, nc), np.float64)
    sabs = np.empty((nr, nc), np.float64)
    lib().orc_linear_w4a16(_ptr(a), K, _ptr(r), nr, _ptr(wc), _ptr(ws), K, _ptr(c), nc,
                           float(np.float32(alpha_)), _ptr(out), _ptr(ref), _ptr(sabs))
    return out, ref, sabs


def linear_w4a4(a_codes, a_scales, w_codes, w_scales, alpha_, rows=None, cols=None):
    ac = _c(a_codes, np.uint8)
    as_ = _c(a_scales, np.uint8)
    wc = _c(w_codes, np.uint8)
    ws = _c(w_scales, np.uint8)
    M = ac.shape[0]
    K = 2 * ac.shape[1]
    N = wc.shape[0]
    r, nr = _idx(rows, M)
    c, nc = _idx(cols, N)
    out = np.empty((nr, nc), np.uint16)
    ref = np.empty((nr, nc), np.float64)
    sabs = np.empty((nr, nc), np.float64)
    lib().orc_linear_w4a4(_ptr(ac), _ptr(as_), _ptr(r), nr, _ptr(wc), _ptr(ws), K, _ptr(c), nc,
                          float(np.float32(alpha_)), _ptr(out), _ptr(ref), _ptr(sabs))
    return out, ref, sabs


def moe_w4a4(x_bf16, ids, rw, gu_codes, gu_scales, dn_codes, dn_scales, g1, g2,
             alpha_gu, alpha_dn, tokens=None):
    """NVFP4 MoE layer on selected tokens.  Returns a dict with out/ref/sabs
    [n_tok, K], the oracle's h codes/scales [n_tok*top_k, I/2 | I/16], their
    boundary margins, and h_amax."""
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    ids = _c(ids, np.int32)
    rw = _c(rw, np.float32)
    top_k = ids.shape[1]
    guc = _c(gu_codes, np.uint8)
    gus = _c(gu_scales, np.uint8)
    dnc = _c(dn_codes, np.uint8)
    dns = _c(dn_scales, np.uint8)
    E, twoI = guc.shape[0], guc.shape[1]
    I = twoI // 2
    agu = _c(alpha_gu, np.float32)
    adn = _c(alpha_dn, np.float32)
    t, nt = _idx(tokens, T)
    P = nt * top_k
    res = {
        "h_codes": np.empty((P, I // 2), np.uint8),
        "h_scales": np.empty((P, I // 16), np.uint8),
        "h_code_margin": np.empty((P, I), np.float64),
        "h_scale_margin": np.empty((P, I // 16), np.float64),
        "out": np.empty((nt, K), np.uint16),
        "ref": np.empty((nt, K), np.float64),
        "sabs": np.empty((nt, K), np.float64),
    }
    amax = np.zeros(1, np.float64)
    lib().orc_moe_w4a4(_ptr(x), T, K, _ptr(ids), _ptr(rw), top_k, E, I, _ptr(guc), _ptr(gus),
                       _ptr(dnc), _ptr(dns), float(np.float32(g1)), float(np.float32(g2)),
                       _ptr(agu), _ptr(adn), _ptr(t), nt,
                       _ptr(res["h_codes"]), _ptr(res["h_scales"]), _ptr(res["h_code_margin"]),
                       _ptr(res["h_scale_margin"]), _ptr(amax), _ptr(res["out"]), _ptr(res["ref"]),
                       _ptr(res["sabs"]))
    res["h_amax"] = float(amax[0])
    return res


def moe_w4a16(x_bf16, ids, rw, gu_codes, gu_scales, dn_codes, dn_scales, alpha_gu, alpha_dn, tokens=None,
              h_in=None):
    """NVFP4 MoE layer with W4A16 on both GEMMs on selected tokens.  Returns a
    dict with out/ref/sabs [n_tok, K] and, per pair q = tt*top_k + r, the
    oracle's h as bf16 bits, in fp64 and its error scale ("h", "h_ref",
    "h_sabs", [n_tok*top_k, I]).  h_in (bf16 bits, same shape) replaces the
    oracle's own h in the down projection."""
    x = _c(x_bf16, np.uint16)
    T, K = x.shape
    ids = _c(ids, np.int32)
    rw = _c(rw, np.float32)
    top_k = ids.shape[1]
    guc = _c(gu_codes, np.uint8)
    gus = _c(gu_scales, np.uint8)
    dnc = _c(dn_codes, np.uint8)
    dns = _c(dn_scales, np.uint8)
    E, twoI = guc.shape[0], guc.shape[1]
    I = twoI // 2
    agu = _c(alpha_gu, np.float32)
    adn = _c(alpha_dn, np.float32)
    t, nt = _idx(tokens, T)
    P = nt * top_k
    hin = None if h_in is None else _c(h_in, np.uint16).reshape(P, I)
    res = {
        "h": np.empty((P, I), np.uint16),
        "h_ref": np.empty((P, I), np.float64),
        "h_sabs": np.empty((P, I), np.float64),
        "out": np.empty((nt, K), np.uint16),
        "ref": np.empty((nt, K), np.float64),
        "sabs": np.empty((nt, K), np.float64),
    }
    lib().orc_moe_w4a16(_ptr(x), T, K, _ptr(ids), _ptr(rw), top_k, E, I, _ptr(guc), _ptr(gus), _ptr(dnc),
                        _ptr(dns), _ptr(agu), _ptr(adn), _ptr(t), nt, _ptr(hin), _ptr(res["h"]),
                        _ptr(res["h_ref"]), _ptr(res["h_sabs"]), _ptr(res["out"]), _ptr(res["ref"]),
                        _ptr(res["sabs"]))
    return res


def swizzle_scales_128x4(scales: np.ndarray) -> np.ndarray:
    """Block scales [rows, K/16] in the 128x4-swizzled layout that the FreeToken
    PR #737 page (Changes) says checkpoints and the block-scaled GEMMs take.
    The page names the layout without its index map, so this follows the
    public one.  Pad with zeros to a multiple of 128 rows and 4 columns.  Split
    the rows into (block, 4 groups of 32) and the columns into (block, 4).
    Store block by block, and inside a block row r % 32 outermost, then the
    group (r / 32) % 4, then the column.  Returns a flat uint8 array."""
    rows, cols = scales.shape
    rp, cp = -(-rows // 128) * 128, -(-cols // 4) * 4
    pad = np.zeros((rp, cp), dtype=np.uint8)
    pad[:rows, :cols] = scales
    # axes: row block, row group of 32, row in group, column block, column in block
    t = pad.reshape(rp // 128, 4, 32, cp // 4, 4)
    return np.ascontiguousarray(t.transpose(0, 3, 2, 1, 4)).reshape(-1)


def unswizzle_scales_128x4(buf: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The inverse of swizzle_scales_128x4: the [rows, cols] scales back."""
    rp, cp = -(-rows // 128) * 128, -(-cols // 4) * 4
    t = np.asarray(buf, dtype=np.uint8)[:rp * cp].reshape(rp // 128, cp // 4, 32, 4, 4)
    return np.ascontiguousarray(t.transpose(0, 3, 2, 1, 4)).reshape(rp, cp)[:rows, :cols]
