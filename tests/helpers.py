"""Shared test helpers: the GEMM tolerance check and device plumbing."""
from __future__ import annotations

import numpy as np

from nvfp4_block_scaled_act_amd import synth


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(bits).astype(np.float64)


def gemm_check(gpu_bits: np.ndarray, ref_bits: np.ndarray, sabs: np.ndarray, max_ulp: float = 2.0,
               rel_l2_max: float = 1e-3) -> dict:
    """Compare bf16 GEMM outputs with the oracle's bf16-rounded fp64 result.

    Per element: |gpu - ref| <= max_ulp * ulp_bf16(max(|ref|, 2^-13 * Sabs)),
    ulp_bf16(y) = 2^(floor(log2 y) - 7), where Sabs = alpha * sum |a * w| is the
    magnitude scale of the fp32 accumulation error (the floor only governs
    outputs that cancel to far below their terms).  Whole output: relative L2
    error <= rel_l2_max.  Returns the statistics; raises AssertionError on a
    violation.
    """
    g = bf16_f64(gpu_bits)
    r = bf16_f64(ref_bits)
    assert np.isfinite(g).all(), "non-finite GPU output"
    y = np.maximum(np.abs(r), 2.0 ** -13 * np.asarray(sabs, np.float64))
    err = np.abs(g - r)
    zero = y == 0
    ulp = np.where(zero, 0.0, np.exp2(np.floor(np.log2(np.where(zero, 1.0, y))) - 7))
    bad = err > max_ulp * ulp
    nr = np.linalg.norm(r)
    rel_l2 = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g))
    stats = dict(n=int(g.size), bad=int(bad.sum()), rel_l2=rel_l2,
                 max_err_ulp=float(np.max(np.where(zero, 0, err / np.where(ulp == 0, 1, ulp)))) if g.size else 0.0,
                 floor_governs=int((np.abs(r) < 2.0 ** -13 * sabs).sum()),
                 exact=int((err == 0).sum()))
    assert stats["bad"] == 0, f"{stats['bad']} elements beyond {max_ulp} bf16 ulp: {stats}"
    assert rel_l2 <= rel_l2_max, f"rel-L2 {rel_l2} > {rel_l2_max}: {stats}"
    return stats


def to_dev(x: np.ndarray, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray):
    import torch

    return to_dev(bits.view(np.int16), None).view(torch.bfloat16)


def bf16_host(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8_host(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def f32_dev(v) -> "torch.Tensor":
    import torch

    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device="cuda")


# W4A16 schedules (schedule, ksplit, chunk_steps) that parity tests run besides
# the default (0, 0, 0); schedules_for keeps the ones valid at (M, K).
SCHEDULES = ([(1, ks, 0) for ks in (1, 2, 3, 7, 16)] + [(2, 0, kc) for kc in (1, 2, 3, 4, 17)]
             + [(3, ks, 0) for ks in (1, 3, 7, 16)] + [(3, ks, 2) for ks in (1, 3, 7, 8)]
             + [(3, ks, 3) for ks in (3, 5, 8)]
             + [(4, ks, 0) for ks in (1, 3, 7, 16)])


def _schedule_valid(sch, M, K):
    steps = K // 256
    if sch[0] == 2:  # LDS rows: M for one token group, else M padded to 16-row groups
        rows = M if M <= 16 else 16 * -(-M // 16)
        return rows * min(sch[2], steps) <= 64
    if sch[0] == 3:  # chunk_steps 2: two tiles per workgroup, at most 8 waves; 3: 2-3 tiles, 3-8 waves
        ks = min(sch[1], steps)
        per = -(-steps // ks)
        waves = -(-steps // per)
        return per <= 8 and (sch[2] < 2 or waves <= 8) and (sch[2] < 3 or waves >= 3)
    if sch[0] == 4:  # dot: M <= 4, <= 8 steps per wave
        ks = min(sch[1], steps)
        return M <= 4 and -(-steps // ks) <= 8
    return True


def schedules_for(M, K):
    return [(0, 0, 0)] + [sch for sch in SCHEDULES if _schedule_valid(sch, M, K)]
