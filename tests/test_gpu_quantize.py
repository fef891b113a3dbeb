"""GPU parity of the quantizer and calibration helpers against the oracle:
codes and scales bit-exact, global scale and alpha bit-exact."""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, f32_dev, u8_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


def _quant_both(ops, orc, x_bits, g, lda=None):
    M, K = x_bits.shape
    if lda is None:
        xd = bf16_dev(x_bits)
    else:
        pad = np.full((M, lda), 0x7F7F, np.uint16)  # padding holds large finite values
        pad[:, :K] = x_bits
        xd = bf16_dev(pad)[:, :K]
    gd = f32_dev(g)
    c, s = ops.quantize_act(xd, gd)
    oc, os_ = orc.quantize(x_bits, g)
    return u8_host(c), u8_host(s), oc, os_


def _assert_same(gc, gs, oc, os_, what):
    bad_s = np.argwhere(gs != os_)
    bad_c = np.argwhere(gc != oc)
    assert len(bad_s) == 0, f"{what}: {len(bad_s)} scale mismatches, first {bad_s[:5].tolist()}"
    assert len(bad_c) == 0, f"{what}: {len(bad_c)} code-byte mismatches, first {bad_c[:5].tolist()}"


def test_global_scale_and_alpha(ops, orc):
    import torch

    for seed, (r, c) in enumerate([(512, 5120), (512, 1024), (7, 48), (1, 8)]):
        x = synth.normal_bf16(500 + seed, r, c)
        g = ops.global_scale(bf16_dev(x))
        assert g.item() == orc.global_scale(x), (r, c)
    gw = torch.tensor([917.25], dtype=torch.float32, device="cuda")
    ga = torch.tensor([471.0625], dtype=torch.float32, device="cuda")
    assert ops.alpha(gw).item() == orc.alpha(917.25)
    assert ops.alpha(gw, ga).item() == orc.alpha(917.25, 471.0625)
    rng = np.random.default_rng(1)
    for _ in range(50):
        a, b = np.float32(rng.uniform(1, 5000)), np.float32(rng.uniform(1, 5000))
        assert ops.alpha(f32_dev(a), f32_dev(b)).item() == orc.alpha(a, b)
    z = np.zeros((4, 16), np.uint16)
    assert ops.global_scale(bf16_dev(z)).item() == 0.0


def test_prefill_activations(ops, orc):
    # W4A4 prefill workload: N(0,1) activations [1024, 5120] under the static
    # global of a 512-row calibration batch.
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, 5120)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 1024, 5120)
    g = orc.global_scale(cal)
    assert ops.global_scale(bf16_dev(cal)).item() == g
    _assert_same(*_quant_both(ops, orc, a, g), "prefill activations")


def test_moe_activations(ops, orc):
    a = synth.normal_bf16(synth.seed_for("moe", synth.ROLE_A), 8192, 2048)
    g = orc.global_scale(synth.normal_bf16(synth.seed_for("moe", synth.ROLE_CAL), 512, 2048))
    _assert_same(*_quant_both(ops, orc, a, g), "moe activations")


def test_weights_small_config(ops, orc):
    w = synth.normal_bf16(synth.seed_for("w4a16_small", synth.ROLE_W), 512, 1024)
    g = orc.global_scale(w)
    _assert_same(*_quant_both(ops, orc, w, g), "weights 512x1024")


@pytest.mark.parametrize("M,K,lda", [(1, 16, None), (5, 48, None), (7, 272, 280), (3, 1024, 1032), (130, 4352, None)])
def test_ragged_and_strided(ops, orc, M, K, lda):
    x = synth.normal_bf16(900 + M + K, M, K)
    g = np.float32(391.7)
    _assert_same(*_quant_both(ops, orc, x, g, lda=lda), f"M={M} K={K} lda={lda}")


def _tie_blocks(rng, nblocks):
    """bf16 blocks whose |x|*1/S hit the e2m1 midpoints exactly at g = 1."""
    thr = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 0.0]
    blocks = []
    for _ in range(nblocks):
        sb = int(rng.integers(0x18, 0x70))   # a normal E4M3 scale byte
        e, m = sb >> 3, sb & 7
        S = (1 + m / 8) * 2.0 ** (e - 7)
        vals = [6.0 * S] + [t * S * rng.choice([-1, 1]) for t in rng.choice(thr, 15)]
        blocks.append(vals)
    x = np.array(blocks, np.float32)
    bits = synth._bf16_bits(x)
    assert (synth.bf16_to_f32(bits) == x).all()
    return bits


def test_exact_ties_and_near_ties(ops, orc):
    rng = np.random.default_rng(42)
    x = _tie_blocks(rng, 4096).reshape(256, 256)
    one = np.float32(1.0)
    for g in [one, np.nextafter(one, np.float32(2)), np.nextafter(one, np.float32(0)), np.float32(2.0),
              np.float32(0.5), np.nextafter(np.float32(0.5), np.float32(1)), np.float32(3.0)]:
        _assert_same(*_quant_both(ops, orc, x, g), f"ties at g={g!r}")


def _tie_blocks_at(rng, nblocks, g):
    """bf16 blocks whose |x|*g/S hit e2m1 midpoints (and codes) exactly under
    the global g, with a block max that makes S the block's scale."""
    thr = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 0.0]
    blocks = []
    while len(blocks) < nblocks:
        sb = int(rng.integers(0x10, 0x78))
        e, m = sb >> 3, sb & 7
        S = (1 + m / 8) * 2.0 ** (e - 7)
        vals = np.array([6.0 * S / g] + [t * S / g * rng.choice([-1, 1]) for t in rng.choice(thr, 15)], np.float32)
        if (synth.bf16_to_f32(synth._bf16_bits(vals)) == vals).all():
            blocks.append(vals)
    return synth._bf16_bits(np.array(blocks, np.float32))


@pytest.mark.parametrize("g", [512.0, 384.0, 96.0, 3.0, 0.75, 1.5 * 2 ** 20])
def test_small_mantissa_global(ops, orc, g):
    # a global of at most 8 significant bits takes the tie-snapping path (the
    # prefill workload's g = 2688/5.25 = 512 is one): exact ties at every
    # midpoint, and N(0,1) rows spread over 40 binades
    rng = np.random.default_rng(int(g * 7) % 1000)
    g = np.float32(g)
    ties = _tie_blocks_at(rng, 4096, float(g)).reshape(256, 256)
    _assert_same(*_quant_both(ops, orc, ties, g), f"ties at g={g}")
    x = (rng.standard_normal((512, 1024)) * np.exp(rng.uniform(-14, 14, (512, 1)))).astype(np.float32) / g
    _assert_same(*_quant_both(ops, orc, synth._bf16_bits(x), g), f"wide rows at g={g}")


def test_special_values(ops, orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, ::2] = -0.0
    x[3] *= 1e-39                 # fp32/bf16 subnormals
    x[4] *= 1e4                   # saturates the scale (448) and codes (6)
    x[5, :16] = [1e-30] * 15 + [3.0]
    x[6] = np.where(rng.random(512) < 0.7, 0.0, x[6])  # sparse blocks
    x[7, :16] = 0.0
    x[7, 3] = -1e-38
    bits = synth._bf16_bits(x)
    for g in [np.float32(200.0), np.float32(1.0), np.float32(1e-3), np.float32(6e4)]:
        _assert_same(*_quant_both(ops, orc, bits, g), f"special values g={g}")


def test_deterministic(ops):
    x = synth.normal_bf16(3, 64, 1024)
    xd = bf16_dev(x)
    g = f32_dev(300.0)
    c1, s1 = ops.quantize_act(xd, g)
    c2, s2 = ops.quantize_act(xd, g)
    assert (u8_host(c1) == u8_host(c2)).all() and (u8_host(s1) == u8_host(s2)).all()


# ------------------------------------------------------------------ 128x4-swizzled scales

@pytest.mark.parametrize("M,K", [(300, 272), (1, 16), (128, 4096), (513, 1024)])
def test_quantize_swizzled(ops, orc, M, K):
    # codes as the row-major call, scales in the 128x4 layout with zero padding,
    # bit for bit against the oracle's quantization and swizzle
    import torch

    a = synth.normal_bf16(41 + M, M, K)
    g = orc.global_scale(a)
    oc, os_ = orc.quantize(a, g)
    ad, gd = bf16_dev(a), f32_dev(g)
    torch.empty(1 << 24, dtype=torch.uint8, device="cuda").fill_(0xFF)  # leave non-zero bytes in the allocator
    c, s = ops.quantize_act_swizzled(ad, gd)
    assert (u8_host(c) == oc).all()
    assert (u8_host(s) == orc.swizzle_scales_128x4(os_)).all()


def test_prepare_weight_swizzled(ops, orc):
    # the prepared weight from swizzled scales equals the one from row-major
    # scales byte for byte (ragged N: the last 16-row tile and 128-row block)
    import torch

    N, K = 300, 512
    W = synth.normal_bf16(43, N, K)
    wd = bf16_dev(W)
    gd = ops.global_scale(wd)
    c, s = ops.quantize_act(wd, gd)
    w_row = ops.prepare_weight(c, s)
    sw = torch.from_numpy(orc.swizzle_scales_128x4(u8_host(s))).cuda()
    w_swz = ops.prepare_weight_swizzled(c, sw)
    assert (u8_host(w_swz.data) == u8_host(w_row.data)).all()
    _, s2 = ops.quantize_act_swizzled(wd, gd)
    assert (u8_host(ops.prepare_weight_swizzled(c, s2).data) == u8_host(w_row.data)).all()
