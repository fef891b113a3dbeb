"""GEMM parity on the edge data of the NVFP4 format, against the oracle.

The other GEMM tests draw N(0,1) weights and activations, whose quantized
scales are all normal E4M3 values well inside the range.  Here the weight is
built directly from bytes, as a checkpoint could hold it (the format's block
scales are FP8-E4M3 per 16 elements, FlashInfer PR #3597, Description), with:
  * zero scale bytes (0x00), subnormal ones (0x01..0x07), the largest finite
    one (0x7E = 448) and normal ones across the whole range;
  * every code nibble, including -0 (0x8) and +-6 (0x7, 0xF); whole rows of
    -0 codes, of the largest magnitude, of scale 0x7E and of scale 0.
The activations hold x20 outlier channels, exact zeros, -0.0 and rows scaled
by 1e-4 and 1e-6.  Quantized under a global calibrated on a batch without the
outliers, their outlier blocks saturate the scale at 448 and clip codes at 6,
and the tiny rows get subnormal or zero scales; the codes are checked bit for
bit against the oracle's first.  Every W4A16 schedule and the W4A4 linear then
meet the bar (2 bf16 ulp with the Sabs floor, rel-L2 <= 1e-3).
"""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_host, f32_dev, gemm_check, schedules_for, to_dev, u8_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


def edge_weight(seed, N, K):
    """Codes [N, K/2] and E4M3 scales [N, K/16] with the format's edge values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    kind = rng.integers(0, 10, (N, K // 16))
    scales = np.select(
        [kind == 0, kind == 1, kind == 2, kind < 6],
        [np.zeros_like(kind), rng.integers(1, 8, kind.shape), np.full_like(kind, 0x7E),
         rng.integers(0x08, 0x7F, kind.shape)],
        rng.integers(0x30, 0x48, kind.shape)).astype(np.uint8)
    codes[0::17] = 0x88   # every code -0
    codes[1::17] = 0x7F   # +6 (low nibble) and -6 (high nibble)
    scales[2::17] = 0x7E  # the largest scale
    scales[3::17] = 0x00  # a zero row
    return codes, scales


def edge_activations(seed, M, K):
    """bf16 [M, K]: N(0,1) with x20 outlier channels, exact zeros, -0.0, and
    rows scaled by 1e-4 and 1e-6."""
    x = synth.bf16_to_f32(synth.normal_bf16(seed, M, K)).astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    outlier = rng.choice(K, K // 64, replace=False)
    x[:, outlier] *= 20.0
    x[:, ::37] = 0.0
    x[:, 5::41] = -0.0
    if M > 2:
        x[1] *= 1e-4
        x[2] *= 1e-6
    if M > 3:
        x[3] = -0.0
    return synth._bf16_bits(x)


def check_codes(ops, orc, a_bits, g):
    """GPU quantization of a under g equals the oracle's; returns both."""
    ac, as_ = ops.quantize_act(bf16_dev(a_bits), f32_dev(g))
    oc, os_ = orc.quantize(a_bits, g)
    assert (u8_host(ac) == oc).all(), "activation codes"
    assert (u8_host(as_) == os_).all(), "activation scales"
    return ac, as_, oc, os_


@pytest.mark.parametrize("M,N,K", [(7, 1000, 4352), (16, 300, 1024), (4, 4096, 2048)])
def test_w4a16_edge_data_every_schedule(ops, orc, M, N, K):
    codes, scales = edge_weight(100 + N, N, K)
    w = ops.prepare_weight(to_dev(codes), to_dev(scales))
    a = edge_activations(200 + M, M, K)
    alpha = np.float32(1.0 / 384.0)
    ref, _, sabs = orc.linear_w4a16(a, codes, scales, alpha)
    ad = bf16_dev(a)
    al = f32_dev(alpha)
    for sch, ks, kc in schedules_for(M, K):
        out = ops.linear_w4a16(ad, w, al, schedule=sch, ksplit=ks, chunk_steps=kc)
        gemm_check(bf16_host(out), ref, sabs)
    for m in range(1, M + 1):  # the default at every token count
        out = ops.linear_w4a16(ad[:m], w, al)
        gemm_check(bf16_host(out), ref[:m], sabs[:m])


# M = 20 and 100 run the few-rows kernel (one and four 32-row groups, N not a
# multiple of 256); 300 and 1100 the 256 x 256 tiles
@pytest.mark.parametrize("M,N,K", [(20, 4104, 768), (100, 1000, 1024), (300, 1000, 1024), (1100, 520, 2048)])
def test_w4a4_edge_data(ops, orc, M, N, K):
    codes, scales = edge_weight(300 + N, N, K)
    w = ops.prepare_weight(to_dev(codes), to_dev(scales))
    a = edge_activations(400 + M, M, K)
    # the activation global from a calibration batch without outliers: the
    # outlier blocks then saturate (scale 448, codes clipped at 6)
    g = orc.global_scale(synth.normal_bf16(500 + M, 64, K))
    ac, as_, oc, os_ = check_codes(ops, orc, a, g)
    assert (os_ == 0x7E).any(), "no saturated activation scale"
    assert (os_[1] < 0x08).any() or (os_[2] == 0).any(), "no subnormal or zero activation scale"
    alpha = np.float32(1.0 / (float(g) * 384.0))
    ref, _, sabs = orc.linear_w4a4(oc, os_, codes, scales, alpha)
    out = ops.linear_w4a4(ac, as_, w, f32_dev(alpha))
    stats = gemm_check(bf16_host(out), ref, sabs)
    print(stats)


def test_dispatch_edge_data(ops, orc):
    # both routes of the dispatched linear on the same edge data
    M, N, K = 40, 700, 1536
    codes, scales = edge_weight(600, N, K)
    w = ops.prepare_weight(to_dev(codes), to_dev(scales))
    a = edge_activations(601, M, K)
    g = orc.global_scale(synth.normal_bf16(602, 64, K))
    oc, os_ = orc.quantize(a, g)
    a16, a4 = np.float32(1.0 / 384.0), np.float32(1.0 / (float(g) * 384.0))
    ad = bf16_dev(a)
    ops.set_route_m_max(16)
    for m in (1, 16, 17, 40):
        out, route = ops.linear(ad[:m], w, f32_dev(g), f32_dev(a16), f32_dev(a4))
        if route == 0:
            ref, _, sabs = orc.linear_w4a16(a[:m], codes, scales, a16)
        else:
            ref, _, sabs = orc.linear_w4a4(oc[:m], os_[:m], codes, scales, a4)
        assert route == (1 if m > 16 else 0)
        gemm_check(bf16_host(out), ref, sabs)
