"""Pins of the oracle's W4A16 and W4A4 linears.

W4A16 is out = (a @ dequant(W, W_sf).T) * alpha (FlashInfer PR #3597,
Description); W4A4 runs the same product on NVFP4-quantized activations with
alpha = 1 / (g_w * g_a) (FreeToken PR #737, Changes).

Pins: one-hot activations (fix nibble order, scale indexing and the row /
column map independently of accumulation order), unit scales (reduces W4A16 to
a plain matmul, checked with numpy), exact rational brute force on tiny shapes,
and the page's own sanity bound against the unquantized weight (FlashInfer PR
#3597, API example: rel_l2 < 0.15 and cos > 0.99 at M, N, K = 128, 4096, 4096).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_act_amd import synth

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decode(codes, scales):
    """Test-side dequantization from the pinned tables: low nibble = even k."""
    c = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    v = E2M1[c & 7] * np.where(c & 8, -1.0, 1.0)
    return v * np.repeat(E4M3[scales], 16, axis=1)


def bf16_nearest(fr: Fraction) -> int:
    """Nearest bf16 to an exact rational (ties to even), by comparing the
    exact distances to neighbouring bf16 values."""
    f = float(fr)
    base = int(torch.tensor(f, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    best = None
    for b in (base - 1, base, base + 1):
        if not (0 <= b <= 0xFFFF) or (b & 0x7F80) == 0x7F80:
            continue
        v = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        d = abs(Fraction(v) - fr)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1]


@pytest.fixture(scope="module")
def small_weight(orc):
    w = synth.normal_bf16(77, 24, 256)
    g = orc.global_scale(w)
    codes, scales = orc.quantize(w, g)
    return w, g, codes, scales


def test_w4a16_one_hot(small_weight, orc):
    w, g, codes, scales = small_weight
    K = 256
    ks = [0, 1, 15, 16, 17, 130, 255]
    a = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        a[i, k] = 1.0
    al = orc.alpha(g)
    out, ref, _ = orc.linear_w4a16(synth._bf16_bits(a), codes, scales, al)
    deq = decode(codes, scales)
    for i, k in enumerate(ks):
        want = float(al) * deq[:, k]
        assert np.array_equal(ref[i], want)
        assert [bf16_nearest(Fraction(v)) for v in want] == out[i].tolist()


def test_w4a16_unit_scales_is_matmul(orc):
    rng = np.random.default_rng(1)
    N, K, M = 16, 128, 5
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)          # every scale = 1.0
    a = synth.normal_bf16(3, M, K)
    _, ref, _ = orc.linear_w4a16(a, codes, scales, 1.0)
    wv = np.empty((N, K))
    wv[:, 0::2] = E2M1[codes & 7] * np.where(codes & 8, -1, 1)
    wv[:, 1::2] = E2M1[(codes >> 4) & 7] * np.where(codes & 0x80, -1, 1)
    want = synth.bf16_to_f32(a).astype(np.float64) @ wv.T
    np.testing.assert_allclose(ref, want, rtol=1e-13, atol=1e-13)


def test_w4a16_exact_brute_force(small_weight, orc):
    w, g, codes, scales = small_weight
    a = synth.normal_bf16(5, 3, 256)
    al = orc.alpha(g)
    out, ref, sabs = orc.linear_w4a16(a, codes, scales, al)
    deq = decode(codes, scales)
    af = synth.bf16_to_f32(a).astype(np.float64)
    for m in range(3):
        for n in range(24):
            s = sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(af[m], deq[n])), Fraction(0))
            exact = Fraction(float(al)) * s
            assert abs(Fraction(ref[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)
            assert out[m, n] == bf16_nearest(exact)
            assert sabs[m, n] == pytest.approx(float(al) * np.abs(af[m] * deq[n]).sum(), rel=1e-12)


def test_w4a4_one_hot(small_weight, orc):
    w, g, codes, scales = small_weight
    K = 256
    ks = [0, 3, 16, 100, 255]
    vals = [1.0, -2.5, 0.375, 7.0, -0.0078125]
    a = np.zeros((len(ks), K), np.float32)
    for i, (k, v) in enumerate(zip(ks, vals)):
        a[i, k] = v
    abits = synth._bf16_bits(a)
    ga = np.float32(500.0)
    ac, as_ = orc.quantize(abits, ga)
    al = orc.alpha(g, ga)
    out, ref, _ = orc.linear_w4a4(ac, as_, codes, scales, al)
    deq = decode(codes, scales)
    for i, (k, v) in enumerate(zip(ks, vals)):
        sa = E4M3[as_[i, k // 16]]
        # the lone element is its block's max: code magnitude 6 at scale sa
        assert decode(ac[i:i + 1], as_[i:i + 1])[0, k] == np.sign(v) * 6 * sa
        want = float(al) * (np.sign(v) * 6 * sa) * deq[:, k]
        assert np.array_equal(ref[i], want)
        assert [bf16_nearest(Fraction(x)) for x in want] == out[i].tolist()


def test_w4a4_exact_brute_force(small_weight, orc):
    w, g, codes, scales = small_weight
    a = synth.normal_bf16(8, 4, 256)
    ga = orc.global_scale(a)
    ac, as_ = orc.quantize(a, ga)
    al = orc.alpha(g, ga)
    out, ref, _ = orc.linear_w4a4(ac, as_, codes, scales, al)
    da, dw = decode(ac, as_), decode(codes, scales)
    for m in range(4):
        for n in range(24):
            s = sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(da[m], dw[n])), Fraction(0))
            exact = Fraction(float(al)) * s
            assert abs(Fraction(ref[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 52)
            assert out[m, n] == bf16_nearest(exact)


def test_w4a4_equals_w4a16_on_dequantized_activations(small_weight, orc):
    # dequantized NVFP4 values are exact in bf16, so W4A4(A) = W4A16(deq(A)).
    w, g, codes, scales = small_weight
    a = synth.normal_bf16(10, 6, 256)
    ga = orc.global_scale(a)
    ac, as_ = orc.quantize(a, ga)
    al = orc.alpha(g, ga)
    out4, ref4, _ = orc.linear_w4a4(ac, as_, codes, scales, al)
    da = decode(ac, as_).astype(np.float32)
    assert (synth.bf16_to_f32(synth._bf16_bits(da)) == da).all()
    out16, ref16, _ = orc.linear_w4a16(synth._bf16_bits(da), codes, scales, al)
    np.testing.assert_allclose(ref16, ref4, rtol=1e-13, atol=1e-13 * np.abs(ref4).max())


def test_row_col_selection(small_weight, orc):
    w, g, codes, scales = small_weight
    a = synth.normal_bf16(12, 9, 256)
    al = orc.alpha(g)
    full, _, _ = orc.linear_w4a16(a, codes, scales, al)
    rows, cols = np.array([8, 0, 3]), np.array([23, 1, 1, 7])
    sel, _, _ = orc.linear_w4a16(a, codes, scales, al, rows=rows, cols=cols)
    assert (sel == full[np.ix_(rows, cols)]).all()
    ga = orc.global_scale(a)
    ac, as_ = orc.quantize(a, ga)
    full4, _, _ = orc.linear_w4a4(ac, as_, codes, scales, orc.alpha(g, ga))
    sel4, _, _ = orc.linear_w4a4(ac, as_, codes, scales, orc.alpha(g, ga), rows=rows, cols=cols)
    assert (sel4 == full4[np.ix_(rows, cols)]).all()


@pytest.mark.slow
def test_page_sanity_bound_vs_unquantized_weight(orc):
    # FlashInfer PR #3597, API example: rel_l2 < 0.15 and cos > 0.99 against
    # (a.float() @ w.float().T).to(bf16) at M, N, K = 128, 4096, 4096.
    M, N, K = 128, 4096, 4096
    w = synth.normal_bf16(100, N, K)
    a = synth.normal_bf16(101, M, K)
    g = orc.global_scale(w)
    codes, scales = orc.quantize(w, g)
    out, _, _ = orc.linear_w4a16(a, codes, scales, orc.alpha(g))
    ref = (torch.from_numpy(synth.bf16_to_f32(a)) @ torch.from_numpy(synth.bf16_to_f32(w)).T).to(torch.bfloat16).float()
    o = torch.from_numpy(synth.bf16_to_f32(out))
    rel_l2 = float((o - ref).norm() / ref.norm())
    cos = float(torch.nn.functional.cosine_similarity(o.flatten(), ref.flatten(), dim=0))
    assert rel_l2 < 0.15 and cos > 0.99
