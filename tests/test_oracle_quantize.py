"""Pins of the oracle's NVFP4 quantizer.

The quantizer follows the per-16-element FP8-E4M3 block scale of FlashInfer PR
#3597 (Description) under the global (448 * 6) / max|w| of its API example:
scale = E4M3(amax * g / 6), code = sign | e2m1(|x| * g / scale), two codes per
byte with even k in the low nibble.

Pins: hand-worked blocks (tests/golden/worked_blocks.json), an exhaustive
brute-force quantizer in exact rational arithmetic on random tiny blocks, the
quantization error bound and other invariants, and the global scale against
fp32 division done by numpy.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_act_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.json")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3 = [float(v) for v in torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double()]


def unpack(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def test_golden_blocks(orc):
    d = json.load(open(GOLDEN))
    for b in d["blocks"]:
        x = np.array(b["x"], np.float32).reshape(1, 16)
        bits = synth._bf16_bits(x)
        assert (synth.bf16_to_f32(bits) == x).all()
        codes, scales = orc.quantize(bits, b["g"])
        assert int(scales[0, 0]) == b["scale"], b["why"]
        assert unpack(codes)[0].tolist() == b["codes"], b["why"]


def _nearest(v, grid):
    dist = [abs(v - Fraction(t)) for t in grid]
    best = min(dist)
    c = [i for i, d in enumerate(dist) if d == best]
    return c[0] if len(c) == 1 else [i for i in c if i % 2 == 0][0]


def brute_block(x, g):
    """Exhaustive nearest search in exact rationals: the scale over all 127
    finite non-negative E4M3 values, each code over the 8 e2m1 magnitudes."""
    xs = [Fraction(float(v)) for v in x]
    G = Fraction(float(g))
    amax = max(abs(v) for v in xs)
    s = _nearest(amax * G / 6, E4M3)
    S = Fraction(E4M3[s])
    codes = []
    for v, f in zip(xs, x):
        sign = 8 if np.signbit(f) else 0
        mag = 0 if S == 0 else _nearest(abs(v) * G / S, E2M1)
        codes.append(sign | mag)
    return s, codes


def test_brute_force_random_blocks(orc):
    rng = np.random.default_rng(5)
    blocks, gs = [], []
    for i in range(400):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(16)
        elif kind == 1:   # wide dynamic range inside a block
            x = rng.standard_normal(16) * np.exp2(rng.integers(-12, 6, 16))
        elif kind == 2:   # values placed on e2m1 midpoints of a power-of-two scale
            x = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], 16) * rng.choice([-1, 1], 16)
        else:             # outliers past the calibration range
            x = rng.standard_normal(16) * 20
        blocks.append(x.astype(np.float32))
        gs.append(np.float32(rng.choice([1.0, 0.5, 3.0, rng.uniform(50, 1000)])))
    for x, g in zip(blocks, gs):
        bits = synth._bf16_bits(x.reshape(1, 16))
        xb = synth.bf16_to_f32(bits)[0]
        codes, scales = orc.quantize(bits, g)
        s, want = brute_block(xb, g)
        assert int(scales[0, 0]) == s, (xb, g)
        assert unpack(codes)[0].tolist() == want, (xb, g)


@pytest.fixture(scope="module")
def normal_quant(orc):
    x = synth.normal_bf16(1234, 256, 1024)
    g = orc.global_scale(x)
    codes, scales = orc.quantize(x, g)
    return x, g, codes, scales


def test_scale_invariants(normal_quant, orc):
    x, g, codes, scales = normal_quant
    assert scales.max() <= 0x7E
    xf = synth.bf16_to_f32(x).astype(np.float64).reshape(x.shape[0], -1, 16)
    amax = np.abs(xf).max(axis=2)
    S = np.array([orc.e4m3_value(b) for b in range(256)])[scales]
    t = amax * float(g) / 6
    # the chosen scale is within half an E4M3 step of t (relative 2^-4)
    normal = S >= 2 ** -6
    assert (np.abs(S - t)[normal] <= S[normal] * 2 ** -4 + 1e-30).all()
    # global's own block maps to the largest finite scale (448 at max|x|)
    r, b = np.unravel_index(np.argmax(amax), amax.shape)
    assert scales[r, b] == 0x7E


def test_code_invariants(normal_quant, orc):
    x, g, codes, scales = normal_quant
    c = unpack(codes).reshape(x.shape[0], -1, 16)
    mag = c & 7
    xf = synth.bf16_to_f32(x).astype(np.float64).reshape(x.shape[0], -1, 16)
    S = np.array([orc.e4m3_value(b) for b in range(256)])[scales][..., None]
    deq = np.array(E2M1)[mag] * np.where(c & 8, -1.0, 1.0) * S / float(g)
    err = np.abs(xf - deq)
    # error bound |x - deq| <= S/g everywhere, <= S/(4g) where |x| g / S < 2
    assert (err <= S / float(g) * (1 + 1e-12)).all()
    small = np.abs(xf) * float(g) / S < 2
    assert (err <= np.where(small, 0.25, 1.0) * S / float(g) * (1 + 1e-12)).all()
    # sign bit follows the input's sign
    assert ((c >> 3).astype(bool) == np.signbit(xf)).all()
    # block maxima get magnitude 6 when the block scale is a normal, unsaturated E4M3
    arg = np.abs(xf).argmax(axis=2)
    top = np.take_along_axis(mag, arg[..., None], axis=2)[..., 0]
    normal = (S[..., 0] >= 2 ** -6) & (scales < 0x7E)
    assert (top[normal] == 7).all()
    # monotone within a block
    order = np.argsort(np.abs(xf), axis=2, kind="stable")
    ms = np.take_along_axis(mag, order, axis=2)
    assert (np.diff(ms.astype(int), axis=2) >= 0).all()


def test_global_scale_is_fp32_division(orc):
    for seed in range(5):
        x = synth.normal_bf16(seed, 64, 256)
        amax = np.abs(synth.bf16_to_f32(x)).max()
        want = np.float32(2688.0) / np.float32(amax)   # IEEE fp32 division
        assert orc.global_scale(x) == want


def test_alpha_definition(orc):
    rng = np.random.default_rng(0)
    for _ in range(200):
        gw = np.float32(rng.uniform(10, 2000))
        ga = np.float32(rng.uniform(10, 2000))
        assert orc.alpha(gw) == np.float32(1.0 / float(gw))
        assert orc.alpha(gw, ga) == np.float32(1.0 / (float(gw) * float(ga)))


def test_quantize_rows_independent(orc):
    # Row stride and row selection do not change a row's result.
    x = synth.normal_bf16(9, 8, 64)
    c_all, s_all = orc.quantize(x, 100.0)
    for r in range(8):
        c, s = orc.quantize(x[r:r + 1], 100.0)
        assert (c[0] == c_all[r]).all() and (s[0] == s_all[r]).all()


def test_quantize_f64_matches_bf16_path(orc):
    x = synth.normal_bf16(21, 16, 128)
    c1, s1 = orc.quantize(x, 321.5)
    c2, s2 = orc.quantize_f64(synth.bf16_to_f32(x).astype(np.float64), 321.5)
    assert (c1 == c2).all() and (s1 == s2).all()
