"""Structural pins of the oracle's NVFP4 MoE expert layer.

The layer follows FreeToken PR #736 (Changes): gate_up on NVFP4 activations,
the gated activation and NVFP4 quantization of its output, then down with the
routing weight and a sum over the top-k routes.  With one expert and one route
of weight 1 it reduces to the dense chain quantize -> W4A4 -> SiLU(gate)*up ->
quantize -> W4A4, built here from the separately pinned linear functions; the
route sum is checked for linearity.
"""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth


def _bank(orc, seed, E, rows, K):
    w = synth.normal_bf16(seed, E * rows, K).reshape(E, rows, K)
    codes = np.empty((E, rows, K // 2), np.uint8)
    scales = np.empty((E, rows, K // 16), np.uint8)
    gs = np.empty(E, np.float32)
    for e in range(E):
        gs[e] = orc.global_scale(w[e])
        codes[e], scales[e] = orc.quantize(w[e], gs[e])
    return codes, scales, gs


def _chain(orc, x, e, guc, gus, dnc, dns, g1, g2, agu, adn):
    """Dense reference for one token row x through expert e -> y (fp64)."""
    I = guc.shape[1] // 2
    xc, xs = orc.quantize(x, g1)
    _, z, _ = orc.linear_w4a4(xc, xs, guc[e], gus[e], agu[e])
    h = z[:, :I] / (1 + np.exp(-z[:, :I])) * z[:, I:]
    hc, hs = orc.quantize_f64(h, g2)
    _, y, _ = orc.linear_w4a4(hc, hs, dnc[e], dns[e], adn[e])
    return y, hc, hs, h


@pytest.fixture(scope="module")
def tiny_moe(orc):
    E, K, I, T = 3, 64, 32, 5
    guc, gus, ggu = _bank(orc, 31, E, 2 * I, K)
    dnc, dns, gdn = _bank(orc, 32, E, K, I)
    x = synth.normal_bf16(33, T, K)
    g1 = orc.global_scale(x)
    g2 = np.float32(40.0)
    agu = np.array([orc.alpha(ggu[e], g1) for e in range(E)], np.float32)
    adn = np.array([orc.alpha(gdn[e], g2) for e in range(E)], np.float32)
    return dict(E=E, K=K, I=I, T=T, guc=guc, gus=gus, dnc=dnc, dns=dns, x=x, g1=g1, g2=g2, agu=agu, adn=adn)


def test_single_route_reduces_to_dense_chain(tiny_moe, orc):
    m = tiny_moe
    ids = np.array([[t % m["E"]] for t in range(m["T"])], np.int32)
    w = np.ones((m["T"], 1), np.float32)
    res = orc.moe_w4a4(m["x"], ids, w, m["guc"], m["gus"], m["dnc"], m["dns"], m["g1"], m["g2"],
                       m["agu"], m["adn"])
    for t in range(m["T"]):
        y, hc, hs, h = _chain(orc, m["x"][t:t + 1], ids[t, 0], m["guc"], m["gus"], m["dnc"], m["dns"],
                              m["g1"], m["g2"], m["agu"], m["adn"])
        assert (res["h_codes"][t] == hc[0]).all() and (res["h_scales"][t] == hs[0]).all()
        np.testing.assert_allclose(res["ref"][t], y[0], rtol=1e-12, atol=1e-15)
    assert res["h_amax"] > 0


def test_route_sum_is_linear(tiny_moe, orc):
    m = tiny_moe
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(m["E"])[:2] for _ in range(m["T"])]).astype(np.int32)
    w = rng.uniform(0.05, 0.6, (m["T"], 2)).astype(np.float32)
    res = orc.moe_w4a4(m["x"], ids, w, m["guc"], m["gus"], m["dnc"], m["dns"], m["g1"], m["g2"],
                       m["agu"], m["adn"])
    for t in range(m["T"]):
        want = 0
        for r in range(2):
            y, *_ = _chain(orc, m["x"][t:t + 1], ids[t, r], m["guc"], m["gus"], m["dnc"], m["dns"],
                           m["g1"], m["g2"], m["agu"], m["adn"])
            want = want + float(w[t, r]) * y[0]
        np.testing.assert_allclose(res["ref"][t], want, rtol=1e-12, atol=1e-15)


def test_token_selection(tiny_moe, orc):
    m = tiny_moe
    rng = np.random.default_rng(6)
    ids = np.stack([rng.permutation(m["E"])[:2] for _ in range(m["T"])]).astype(np.int32)
    w = rng.uniform(0.05, 0.6, (m["T"], 2)).astype(np.float32)
    args = (m["x"], ids, w, m["guc"], m["gus"], m["dnc"], m["dns"], m["g1"], m["g2"], m["agu"], m["adn"])
    full = orc.moe_w4a4(*args)
    sel = orc.moe_w4a4(*args, tokens=np.array([4, 1]))
    assert (sel["out"] == full["out"][[4, 1]]).all()
    assert (sel["h_codes"][0:2] == full["h_codes"][8:10]).all()

