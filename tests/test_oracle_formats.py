"""Pins of the oracle's number formats against facts outside the oracle.

* e2m1: the 16-entry value table of the FP4 E2M1 format ({0, .5, 1, 1.5, 2, 3,
  4, 6} x sign), with the sign in bit 3 and the magnitude index in the low three
  bits (FlashInfer PR #3597, review thread: the E2M1 nibble table).
* E4M3: all 256 bytes against PyTorch's own float8_e4m3fn decode (a library
  routine), and the E4M3 largest value 448 of the (448 * 6) global of
  FlashInfer PR #3597, API example.
* rounding: against PyTorch's fp32 -> float8_e4m3fn and fp32 -> bf16 casts
  (round to nearest even) where those apply, and closed forms at every
  midpoint, one double ulp either side, and past the largest value.
"""
import math

import numpy as np
import pytest
import torch

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table(orc):
    for i, v in enumerate(E2M1_TABLE):
        assert orc.e2m1_value(i) == v
        neg = orc.e2m1_value(8 | i)
        assert neg == -v and math.copysign(1.0, neg) == -1.0


def test_e4m3_decode_all_bytes_vs_torch(orc):
    lib_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        ours = orc.e4m3_value(b)
        if b in (0x7F, 0xFF):
            assert math.isnan(ours) and math.isnan(lib_vals[b])
        else:
            assert ours == lib_vals[b], hex(b)
            assert math.copysign(1.0, ours) == (-1.0 if b & 0x80 else 1.0)


def test_e4m3_landmarks(orc):
    assert orc.e4m3_value(0x7E) == 448.0          # largest finite (the 448 of 448*6)
    assert orc.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert orc.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    vals = [orc.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # strictly increasing 0x00..0x7E


def test_e4m3_encode_roundtrip(orc):
    for b in range(0x7F):
        v = orc.e4m3_value(b)
        assert orc.e4m3_round(v, 1.0, 1.0) == b


def _e4m3_candidates():
    """fp32 values at, and one fp32 ulp around, every E4M3 value and midpoint
    below 448, plus random values."""
    vals = [float(torch.tensor(b, dtype=torch.uint8).view(torch.float8_e4m3fn).float()) for b in range(0x7F)]
    pts = set()
    for a, b in zip(vals, vals[1:]):
        for p in (a, 0.5 * (a + b)):
            f = np.float32(p)
            pts.update([f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))])
    rng = np.random.default_rng(7)
    pts.update(np.float32(v) for v in rng.uniform(0, 448, 2000))
    pts.update(np.float32(v) for v in np.exp2(rng.uniform(-12, 8.8, 2000)))
    return sorted(float(p) for p in pts if 0 <= p <= 448)


def test_e4m3_rounding_vs_torch(orc):
    pts = _e4m3_candidates()
    lib = torch.tensor(pts, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_round(p, 1.0, 1.0) for p in pts])
    assert (ours == lib).all()


def test_e4m3_saturation(orc):
    # Past the largest value every real rounds to 0x7E (the format has no inf;
    # 0x7F is NaN).
    for t in (448.0, 448.0 * (1 + 2 ** -40), 463.999, 464.0, 480.0, 1e6, 1e30):
        assert orc.e4m3_round(t, 1.0, 1.0) == 0x7E
    # Below half the smallest subnormal -> 0; exactly half -> tie to even 0x00.
    assert orc.e4m3_round(2.0 ** -10, 1.0, 1.0) == 0
    assert orc.e4m3_round(math.nextafter(2.0 ** -10, 1), 1.0, 1.0) == 1


def test_e2m1_rounding_midpoints(orc):
    # grid 0, .5, 1, 1.5, 2, 3, 4, 6; midpoints and their even-index winner.
    mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for m, even in mids:
        assert orc.e2m1_round(m, 1.0, 1.0) == even
        lo = [i for i, v in enumerate(E2M1_TABLE) if v < m][-1]
        hi = lo + 1
        assert orc.e2m1_round(math.nextafter(m, 0), 1.0, 1.0) == lo
        assert orc.e2m1_round(math.nextafter(m, 10), 1.0, 1.0) == hi
    for v in (6.0, 6.5, 7.0, 1e9):
        assert orc.e2m1_round(v, 1.0, 1.0) == 7
    for i, v in enumerate(E2M1_TABLE):
        assert orc.e2m1_round(v, 1.0, 1.0) == i


def test_e2m1_rounding_brute_force(orc):
    # Exact ratios x*y/den against an exhaustive nearest-value search done in
    # exact rational arithmetic.
    from fractions import Fraction

    rng = np.random.default_rng(11)
    for _ in range(3000):
        x = float(np.float32(rng.uniform(0, 8)))
        y = float(np.float32(rng.uniform(0.5, 2)))
        den = float(torch.tensor(int(rng.integers(0x20, 0x48)), dtype=torch.uint8).view(torch.float8_e4m3fn).float())
        v = Fraction(x) * Fraction(y) / Fraction(den)
        dist = [abs(v - Fraction(t)) for t in E2M1_TABLE]
        best = min(dist)
        cands = [i for i, d in enumerate(dist) if d == best]
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert orc.e2m1_round(x, y, den) == want, (x, y, den)


def test_bf16_rne_vs_torch(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(5000) * 1e30).astype(np.float32)])
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([orc.bf16_rne(float(v)) for v in x], np.uint16)
    assert (ours == lib).all()


def test_bf16_rne_no_double_rounding(orc):
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7; a double just
    # above it must round up, although its fp32 rounding lands on the midpoint
    # (which would then tie to even 1.0).
    r = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(r) == np.float32(1.0 + 2.0 ** -8)
    assert orc.bf16_rne(r) == 0x3F81
    assert orc.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80       # exact tie -> even
    assert orc.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82   # tie -> even (up)
    assert orc.bf16_rne(-0.0) == 0x8000
    assert orc.bf16_rne(1e300) == 0x7F80
