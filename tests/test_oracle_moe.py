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


def test_skipped_ids(tiny_moe, orc):
    # an id outside [0, E) adds nothing: the same sum as that route with
    # weight 0, no h for the pair (zero codes and scales, infinite margins),
    # and the other pairs' h unchanged
    m = tiny_moe
    rng = np.random.default_rng(8)
    ids = np.stack([rng.permutation(m["E"])[:2] for _ in range(m["T"])]).astype(np.int32)
    w = rng.uniform(0.05, 0.6, (m["T"], 2)).astype(np.float32)
    args = (m["guc"], m["gus"], m["dnc"], m["dns"], m["g1"], m["g2"], m["agu"], m["adn"])
    ids2 = ids.copy()
    ids2[1, 0], ids2[3, 1] = -1, m["E"]
    w0 = w.copy()
    w0[1, 0] = w0[3, 1] = 0.0
    skipped = orc.moe_w4a4(m["x"], ids2, w, *args)
    zero_w = orc.moe_w4a4(m["x"], ids, w0, *args)
    np.testing.assert_array_equal(skipped["ref"], zero_w["ref"])
    np.testing.assert_array_equal(skipped["out"], zero_w["out"])
    for p in (1 * 2 + 0, 3 * 2 + 1):
        assert (skipped["h_codes"][p] == 0).all() and (skipped["h_scales"][p] == 0).all()
        assert np.isinf(skipped["h_code_margin"][p]).all() and np.isinf(skipped["h_scale_margin"][p]).all()
    kept = [p for p in range(2 * m["T"]) if p not in (2, 7)]
    assert (skipped["h_codes"][kept] == zero_w["h_codes"][kept]).all()



# ------------------------------------------------------------ W4A16 layer
# The W4A16 layer keeps x and h in bf16 (no activation globals): with one
# expert and one route of weight 1 it reduces to the dense chain W4A16 ->
# SiLU(gate)*up -> bf16 -> W4A16, built from the separately pinned linear.

def _chain16(orc, x, e, guc, gus, dnc, dns, agu, adn):
    I = guc.shape[1] // 2
    _, z, zs = orc.linear_w4a16(x, guc[e], gus[e], agu[e])
    h = z[:, :I] / (1 + np.exp(-z[:, :I])) * z[:, I:]
    hb = np.array([[orc.bf16_rne(v) for v in row] for row in h], np.uint16)
    _, y, _ = orc.linear_w4a16(hb, dnc[e], dns[e], adn[e])
    return y, hb, h


@pytest.fixture(scope="module")
def tiny_moe16(orc):
    E, K, I, T = 3, 64, 32, 5
    guc, gus, ggu = _bank(orc, 41, E, 2 * I, K)
    dnc, dns, gdn = _bank(orc, 42, E, K, I)
    x = synth.normal_bf16(43, T, K)
    agu = np.array([orc.alpha(g, np.float32(1.0)) for g in ggu], np.float32)
    adn = np.array([orc.alpha(g, np.float32(1.0)) for g in gdn], np.float32)
    return dict(E=E, K=K, I=I, T=T, guc=guc, gus=gus, dnc=dnc, dns=dns, x=x, agu=agu, adn=adn)


def test_w4a16_single_route_reduces_to_dense_chain(tiny_moe16, orc):
    m = tiny_moe16
    ids = np.array([[t % m["E"]] for t in range(m["T"])], np.int32)
    w = np.ones((m["T"], 1), np.float32)
    res = orc.moe_w4a16(m["x"], ids, w, m["guc"], m["gus"], m["dnc"], m["dns"], m["agu"], m["adn"])
    for t in range(m["T"]):
        y, hb, h = _chain16(orc, m["x"][t:t + 1], ids[t, 0], m["guc"], m["gus"], m["dnc"], m["dns"],
                            m["agu"], m["adn"])
        assert (res["h"][t] == hb[0]).all()
        np.testing.assert_allclose(res["h_ref"][t], h[0], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(res["ref"][t], y[0], rtol=1e-12, atol=1e-15)
        assert (res["out"][t] == np.array([orc.bf16_rne(v) for v in res["ref"][t]], np.uint16)).all()


def test_w4a16_route_sum_linear_and_skipped_ids(tiny_moe16, orc):
    m = tiny_moe16
    rng = np.random.default_rng(5)
    ids = np.stack([rng.permutation(m["E"])[:2] for _ in range(m["T"])]).astype(np.int32)
    w = rng.uniform(0.05, 0.6, (m["T"], 2)).astype(np.float32)
    args = (m["guc"], m["gus"], m["dnc"], m["dns"], m["agu"], m["adn"])
    res = orc.moe_w4a16(m["x"], ids, w, *args)
    for t in range(m["T"]):
        want = 0
        for r in range(2):
            y, *_ = _chain16(orc, m["x"][t:t + 1], ids[t, r], *args)
            want = want + float(w[t, r]) * y[0]
        np.testing.assert_allclose(res["ref"][t], want, rtol=1e-12, atol=1e-15)
    # an id outside [0, E) adds nothing: the same as that route with weight 0
    ids2 = ids.copy()
    ids2[1, 0], ids2[3, 1] = -1, m["E"]
    w0 = w.copy()
    w0[1, 0] = w0[3, 1] = 0.0
    skipped = orc.moe_w4a16(m["x"], ids2, w, *args)
    zero_w = orc.moe_w4a16(m["x"], ids, w0, *args)
    np.testing.assert_array_equal(skipped["ref"], zero_w["ref"])
    assert (skipped["h"][1 * 2 + 0] == 0).all() and (skipped["h_sabs"][3 * 2 + 1] == 0).all()


def test_w4a16_h_in_and_token_selection(tiny_moe16, orc):
    m = tiny_moe16
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]], np.int32)
    w = np.full((m["T"], 2), 0.5, np.float32)
    args = (m["guc"], m["gus"], m["dnc"], m["dns"], m["agu"], m["adn"])
    res = orc.moe_w4a16(m["x"], ids, w, *args)
    # feeding the oracle its own h back changes nothing
    again = orc.moe_w4a16(m["x"], ids, w, *args, h_in=res["h"])
    np.testing.assert_array_equal(again["ref"], res["ref"])
    # a selected token subset gives the same rows
    sel = orc.moe_w4a16(m["x"], ids, w, *args, tokens=[3, 1])
    np.testing.assert_array_equal(sel["ref"], res["ref"][[3, 1]])
    np.testing.assert_array_equal(sel["h"], res["h"].reshape(m["T"], 2, -1)[[3, 1]].reshape(4, -1))
    # the error scale of h bounds h's sensitivity: zero only where h is zero
    assert (res["h_sabs"] > 0).all()
