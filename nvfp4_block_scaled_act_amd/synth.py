"""Seeded synthetic inputs for the NVFP4 quantized linear.

This module only draws random numbers and lays out the workloads' shapes; it
holds none of the quantization or GEMM arithmetic.  The same bytes feed the
GPU library and the CPU oracle.

Generator: numpy's PCG64 bit generator, standard normal fp32 draws, rounded to
bf16 (nearest, ties to even) to form bf16 tensors.  Large tensors are drawn in
fixed row chunks from one generator, so the bytes depend only on the seed and
the shape.

The workloads follow the pages' shapes: the W4A16 decode shapes and the large
fused shape are the ones the SM70 QPN2 pack change tests (1Cat-vLLM PR #611,
Test Plan); the MoE layer follows the expert-layer flow of FreeToken PR #736
(Changes) with random banks and a calibration batch for the static input
scales, as that page's Results section measures it.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# Workloads (shapes only)
# ----------------------------------------------------------------------------
W4A16_SMALL = dict(M=4, N=512, K=1024)
W4A16_DECODE_SHAPES = [(3584, 5120), (8704, 5120), (5120, 1536), (5120, 4352)]
W4A16_DECODE_M = [1, 2, 4, 8, 16]
W4A4_PREFILL = dict(N=8704, K=5120, M=[1024, 4096, 8192], calib_rows=512)
FUSED_LARGE = dict(N=62080, K=5120, M=[1, 8, 16, 64, 256, 1024, 4096, 8192], calib_rows=512)
MOE = dict(E=128, top_k=8, K=2048, I=768, T=8192, calib_rows=512)

# Roles of the tensors a workload draws (part of the seed).
ROLE_W, ROLE_A, ROLE_CAL, ROLE_LOGITS, ROLE_GATE_UP, ROLE_DOWN, ROLE_CAL_LOGITS = 1, 2, 3, 4, 5, 6, 7
WORKLOAD_ID = {"w4a16_small": 0, "w4a16_decode": 1, "w4a4_prefill": 2, "fused_large": 3, "moe": 4}


def seed_for(workload: str, role: int, shape_index: int = 0) -> int:
    return 1000003 * (WORKLOAD_ID[workload] + 1) + role + 16 * shape_index


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest, ties to even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_bf16(seed: int, rows: int, cols: int, chunk_rows: int = 4096) -> np.ndarray:
    """bf16 bits [rows, cols] of N(0, 1) draws."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = _bf16_bits(g.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def normal_f32(seed: int, rows: int, cols: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.standard_normal((rows, cols), dtype=np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def route_top_k(logits: np.ndarray, top_k: int) -> tuple[np.ndarray, np.ndarray]:
    """Router input: softmax over each row of fp32 logits (in fp64), the top_k
    experts by probability (ties to the lower expert id), and their
    probabilities as fp32 routing weights (not renormalised)."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :top_k]
    ids = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, w


def moe_inputs(T: int | None = None, E: int | None = None, K: int | None = None, I: int | None = None,
               top_k: int | None = None, calib_rows: int | None = None, seed_base: str = "moe"):
    """bf16 hidden states, routing, and bf16 expert banks of the MoE workload
    (defaults: E=128, top-8, K=2048, I=768, T=8192)."""
    T = MOE["T"] if T is None else T
    E = MOE["E"] if E is None else E
    K = MOE["K"] if K is None else K
    I = MOE["I"] if I is None else I
    top_k = MOE["top_k"] if top_k is None else top_k
    calib_rows = MOE["calib_rows"] if calib_rows is None else calib_rows
    x = normal_bf16(seed_for(seed_base, ROLE_A), T, K)
    logits = normal_f32(seed_for(seed_base, ROLE_LOGITS), T, E)
    ids, w = route_top_k(logits, top_k)
    cal = normal_bf16(seed_for(seed_base, ROLE_CAL), calib_rows, K)
    cal_logits = normal_f32(seed_for(seed_base, ROLE_CAL_LOGITS), calib_rows, E)
    cal_ids, cal_w = route_top_k(cal_logits, top_k)
    gate_up = normal_bf16(seed_for(seed_base, ROLE_GATE_UP), E * 2 * I, K).reshape(E, 2 * I, K)
    down = normal_bf16(seed_for(seed_base, ROLE_DOWN), E * K, I).reshape(E, K, I)
    return dict(x=x, ids=ids, w=w, cal=cal, cal_ids=cal_ids, cal_w=cal_w, gate_up=gate_up, down=down,
                T=T, E=E, K=K, I=I, top_k=top_k)
