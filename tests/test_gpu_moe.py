"""GPU parity of the NVFP4 MoE expert layer against the oracle.

Stage-wise check (the GPU's h is fp32, the oracle's fp64, so h's NVFP4 codes
may legitimately differ where h sits on a rounding boundary):
  align    bit-exact: pairs grouped by expert in pair order (a stable sort of
           the expert ids), expert offsets, tile table
  h        codes and scales per pair equal the oracle's, except benign flips:
           the oracle's exact value within a small relative margin of the
           boundary it straddles (scale flips may change the whole block)
  out      rel-L2 <= 1e-3 over all checked tokens, and the per-element bar
           (2 bf16 ulp with the Sabs floor) on every token whose h has no flip
"""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_host, f32_dev, gemm_check, to_dev, u8_host

pytestmark = pytest.mark.gpu

# A flip of an h code or scale is benign when the oracle's exact |h|*g2/S (or
# amax*g2/6) lies within this relative distance of the boundary it straddles.
BENIGN_MARGIN = 2.0 ** -14


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


class Banks:
    """Expert banks quantized per expert on the GPU (one global per expert
    tensor) and prepared as one stacked weight each; the oracle quantizes the
    same bf16 banks itself, and the two are compared on `check_experts`.
    Without g2, g2 is calibrated by the oracle on `cal` = (x, ids, w):
    g2 = fp32(2688 / max |h|) over the calibration batch's routed pairs."""

    def __init__(self, ops, orc, gate_up, down, g1, g2=None, cal=None, check_experts=None):
        import torch

        E, twoI, K = gate_up.shape
        I = twoI // 2
        self.E, self.K, self.I = E, K, I
        g1 = np.float32(g1)
        og_gu = [orc.global_scale(gate_up[e]) for e in range(E)]
        og_dn = [orc.global_scale(down[e]) for e in range(E)]
        self.o_gu = (np.empty((E, twoI, K // 2), np.uint8), np.empty((E, twoI, K // 16), np.uint8))
        self.o_dn = (np.empty((E, K, I // 2), np.uint8), np.empty((E, K, I // 16), np.uint8))
        for e in range(E):
            self.o_gu[0][e], self.o_gu[1][e] = orc.quantize(gate_up[e], og_gu[e])
            self.o_dn[0][e], self.o_dn[1][e] = orc.quantize(down[e], og_dn[e])
        self.o_alpha_gu = np.array([orc.alpha(g, g1) for g in og_gu], np.float32)
        if g2 is None:
            a_dn1 = np.array([orc.alpha(g, np.float32(1.0)) for g in og_dn], np.float32)
            xc, ic, wc = cal
            res = orc.moe_w4a4(xc, ic, wc, self.o_gu[0], self.o_gu[1], self.o_dn[0], self.o_dn[1], g1,
                               np.float32(1.0), self.o_alpha_gu, a_dn1)
            g2 = orc.global_scale_from_amax(res["h_amax"])
        g2 = np.float32(g2)
        self.g1, self.g2 = g1, g2
        self.o_alpha_dn = np.array([orc.alpha(g, g2) for g in og_dn], np.float32)

        g1d, g2d = f32_dev(g1), f32_dev(g2)
        self.alpha_gu = torch.empty(E, dtype=torch.float32, device="cuda")
        self.alpha_dn = torch.empty(E, dtype=torch.float32, device="cuda")
        check = range(E) if check_experts is None else check_experts
        prepared = []
        for bank, g_in_dev, alphas, o_codes in ((gate_up, g1d, self.alpha_gu, self.o_gu),
                                                (down, g2d, self.alpha_dn, self.o_dn)):
            rows = bank.shape[1]
            dev = bf16_dev(bank.reshape(E * rows, bank.shape[2]))
            codes = torch.empty((E * rows, bank.shape[2] // 2), dtype=torch.uint8, device="cuda")
            scales = torch.empty((E * rows, bank.shape[2] // 16), dtype=torch.uint8, device="cuda")
            for e in range(E):
                sl = slice(e * rows, (e + 1) * rows)
                g = ops.global_scale(dev[sl])
                ops.quantize_act(dev[sl], g, codes=codes[sl], scales=scales[sl])
                ops.alpha(g, g_in_dev, out=alphas[e:e + 1])
            hc, hs = u8_host(codes), u8_host(scales)
            for e in check:
                sl = slice(e * rows, (e + 1) * rows)
                assert (hc[sl] == o_codes[0][e]).all(), f"weight codes of expert {e}"
                assert (hs[sl] == o_codes[1][e]).all(), f"weight scales of expert {e}"
            del dev
            prepared.append(ops.prepare_weight(codes, scales))
        assert (self.alpha_gu.cpu().numpy() == self.o_alpha_gu).all()
        assert (self.alpha_dn.cpu().numpy() == self.o_alpha_dn).all()
        self.w_gu, self.w_dn = prepared

    def run(self, ops, x, ids, w, h_amax=None, workspace=None):
        import torch

        T = x.shape[0]
        top_k = ids.shape[1]
        if workspace is None:
            workspace = torch.empty(max(1, ops.moe_workspace_bytes(T, top_k, self.E, self.K, self.I)),
                                    dtype=torch.uint8, device="cuda")
        out = ops.moe_w4a4(bf16_dev(x), to_dev(ids), to_dev(w), self.w_gu, self.w_dn, self.E, f32_dev(self.g1),
                           f32_dev(self.g2), self.alpha_gu, self.alpha_dn, workspace=workspace, h_amax=h_amax)
        torch.cuda.synchronize()
        return out, workspace

    def oracle(self, orc, x, ids, w, tokens=None):
        return orc.moe_w4a4(x, ids, w, self.o_gu[0], self.o_gu[1], self.o_dn[0], self.o_dn[1], self.g1, self.g2,
                            self.o_alpha_gu, self.o_alpha_dn, tokens=tokens)


def expected_align(ids, E, rows=256):
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    idx = np.nonzero(valid)[0]
    order = idx[np.argsort(flat[idx], kind="stable")]
    counts = np.bincount(flat[idx], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    tiles = []
    for e in range(E):
        for j in range(0, counts[e], rows):
            tiles.append((e, offsets[e] + j, min(rows, counts[e] - j), 0))
    return order, offsets, tiles


def check_align(views, ids, E, rows=256):
    order, offsets, tiles = expected_align(ids, E, rows)
    n = len(order)
    got_sorted = views["sorted"].cpu().numpy()
    assert (got_sorted[:n] == order).all(), "sorted pairs differ from a stable sort by expert"
    assert (views["offsets"].cpu().numpy() == offsets).all(), "expert offsets"
    tt = views["tiles"].cpu().numpy()
    assert len(tiles) <= tt.shape[0]
    assert (tt[:len(tiles)] == np.array(tiles, np.int64).reshape(-1, 4)).all(), "tile table"
    assert (tt[len(tiles):, 2] == 0).all(), "entries past the last tile must be empty"
    inv = np.full(ids.size, -1, np.int64)
    inv[order] = np.arange(n)
    assert (views["inv"].cpu().numpy() == inv).all(), "slot of each pair (inverse of sorted)"
    return inv


def check_h(views, inv, res, tokens, top_k, I):
    """h codes/scales of the tokens' pairs; returns the set of tokens with a
    (benign) flip.  Any flip outside the margin fails."""
    tokens = np.asarray(tokens, np.int64)
    p = (tokens[:, None] * top_k + np.arange(top_k)[None, :]).reshape(-1)  # pair of each oracle row q
    slot = inv[p]
    kept = np.nonzero(slot >= 0)[0]
    if len(kept) == 0:
        return set(), 0, 0
    hc = views["h_codes"].cpu().numpy()[slot[kept]]
    hs = views["h_scales"].cpu().numpy()[slot[kept]]
    o_hc, o_hs = res["h_codes"][kept], res["h_scales"][kept]
    scale_bad = hs != o_hs
    if scale_bad.any():
        m = res["h_scale_margin"][kept][scale_bad]
        assert (m <= BENIGN_MARGIN).all(), f"h scale mismatch with margin {m.max()}"
    def nibbles(c):
        return np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1)
    code_bad = (nibbles(hc) != nibbles(o_hc)) & ~np.repeat(scale_bad, 16, axis=1)
    if code_bad.any():
        m = res["h_code_margin"][kept][code_bad]
        where = np.argwhere(code_bad)[:4]
        assert (m <= BENIGN_MARGIN).all(), f"h code mismatch at (row, i) {where.tolist()}, margin {m.max()}"
    rows = np.nonzero(scale_bad.any(1) | code_bad.any(1))[0]
    flipped = {int(tokens[kept[r] // top_k]) for r in rows}
    return flipped, int(code_bad.sum()), int(scale_bad.sum())


def check_out(out_bits, res, tokens, flipped):
    keep = np.array([i for i, t in enumerate(tokens) if t not in flipped], np.int64)
    g = out_bits[tokens]
    ref = res["out"]
    # rel-L2 over every checked token
    stats = gemm_check(g, ref, res["sabs"], max_ulp=float("inf"))
    if len(keep):
        stats = gemm_check(g[keep], ref[keep], res["sabs"][keep])
    return stats


def _small_case(seed, T, E, top_k, K, I, bias=None, calib_rows=64):
    x = synth.normal_bf16(seed, T, K)
    logits = synth.normal_f32(seed + 1, T, E)
    cal = synth.normal_bf16(seed + 2, calib_rows, K)
    cal_logits = synth.normal_f32(seed + 3, calib_rows, E)
    if bias is not None:
        logits = logits + bias
        cal_logits = cal_logits + bias
    ids, w = synth.route_top_k(logits, top_k)
    cids, cw = synth.route_top_k(cal_logits, top_k)
    gate_up = synth.normal_bf16(seed + 4, E * 2 * I, K).reshape(E, 2 * I, K)
    down = synth.normal_bf16(seed + 5, E * K, I).reshape(E, K, I)
    return x, ids, w, cal, cids, cw, gate_up, down


def test_moe_small_multi_tile(ops, orc):
    # 8 experts, top-2, K=512, I=256, T=700: expert 0 draws most tokens (3
    # tiles, the last ragged), expert 7 none; every other expert one ragged tile
    E, top_k, K, I, T = 8, 2, 512, 256, 700
    bias = np.zeros(E, np.float32)
    bias[0], bias[7] = 2.5, -30.0
    x, ids, w, cal, cids, cw, gate_up, down = _small_case(101, T, E, top_k, K, I, bias)
    banks = Banks(ops, orc, gate_up, down, orc.global_scale(cal), cal=(cal, cids, cw))
    import torch

    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out, ws = banks.run(ops, x, ids, w, h_amax=h_amax)
    views = ops.moe_workspace_views(ws, T, top_k, E, K, I)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert counts[0] > 512 and counts[7] == 0
    inv = check_align(views, ids, E)
    tokens = np.arange(T)
    res = banks.oracle(orc, x, ids, w)
    flipped, ncf, nsf = check_h(views, inv, res, tokens, top_k, I)
    stats = check_out(bf16_host(out), res, tokens, flipped)
    assert abs(h_amax.item() - res["h_amax"]) <= 1e-5 * res["h_amax"]
    print(f"flipped tokens {len(flipped)}/{T}, code flips {ncf}, scale flips {nsf}, {stats}")


@pytest.mark.parametrize("K,I", [(768, 512), (256, 256)])
def test_moe_few_rows_tiles(ops, orc, K, I):
    # expert tiles of at most 128 pairs run the few-rows GEMM loop with 1, 2
    # or 4 groups of 32 rows: 8 experts, top-2, T=160, routed so that the
    # tiles hold 108, 85, 53, 37, 23, 12, 2 and 0 pairs (every group count,
    # ragged); K=768 and I=512 take 3 and 2 units of 256 k, K=I=256 one unit
    # each (the prefetch ring re-reads the only unit)
    E, top_k, T = 8, 2, 160
    bias = np.array([1.2, 0.9, 0.5, 0.2, 0.0, -0.6, -1.2, -30.0], np.float32)
    x, ids, w, cal, cids, cw, gate_up, down = _small_case(303, T, E, top_k, K, I, bias)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert (counts > 64).any() and ((counts > 32) & (counts <= 64)).any() and ((counts > 0) & (counts <= 32)).any()
    assert counts.max() <= 128
    banks = Banks(ops, orc, gate_up, down, orc.global_scale(cal), cal=(cal, cids, cw))
    import torch

    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out, ws = banks.run(ops, x, ids, w, h_amax=h_amax)
    views = ops.moe_workspace_views(ws, T, top_k, E, K, I)
    inv = check_align(views, ids, E)
    tokens = np.arange(T)
    res = banks.oracle(orc, x, ids, w)
    flipped, ncf, nsf = check_h(views, inv, res, tokens, top_k, I)
    stats = check_out(bf16_host(out), res, tokens, flipped)
    assert abs(h_amax.item() - res["h_amax"]) <= 1e-5 * res["h_amax"]
    print(f"counts {counts.tolist()}: flipped tokens {len(flipped)}/{T}, code flips {ncf}, scale flips {nsf}, {stats}")


def test_moe_skipped_ids_and_repeat(ops, orc):
    # ids outside [0, E) add nothing; a second call on the same workspace gives
    # the same h and the same output bits (the route sum has a fixed order)
    E, top_k, K, I, T = 4, 3, 256, 256, 130
    x, ids, w, cal, cids, cw, gate_up, down = _small_case(202, T, E, top_k, K, I)
    ids = ids.copy()
    ids[::7, 0] = -1
    ids[3::11, 2] = E
    banks = Banks(ops, orc, gate_up, down, orc.global_scale(cal), cal=(cal, cids, cw))
    out1, ws = banks.run(ops, x, ids, w)
    views = ops.moe_workspace_views(ws, T, top_k, E, K, I)
    inv = check_align(views, ids, E)
    h1 = views["h_codes"].cpu().numpy().copy()
    out2, _ = banks.run(ops, x, ids, w, workspace=ws)
    n = int(views["offsets"].cpu().numpy()[E])
    assert (views["h_codes"].cpu().numpy()[:n] == h1[:n]).all()
    assert (bf16_host(out1) == bf16_host(out2)).all(), "route sum must be deterministic"
    # the oracle skips the same pairs (ids outside [0, E) add nothing)
    res = banks.oracle(orc, x, ids, w)
    flipped, _, _ = check_h(views, inv, res, np.arange(T), top_k, I)
    for out in (out1, out2):
        check_out(bf16_host(out), res, np.arange(T), flipped)


def test_moe_empty(ops, orc):
    import torch

    E, top_k, K, I = 2, 2, 256, 256
    gate_up = synth.normal_bf16(5, E * 2 * I, K).reshape(E, 2 * I, K)
    down = synth.normal_bf16(6, E * K, I).reshape(E, K, I)
    banks = Banks(ops, orc, gate_up, down, 1.0, 1.0)
    x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((0, top_k), dtype=torch.float32, device="cuda")
    out = ops.moe_w4a4(x, ids, w, banks.w_gu, banks.w_dn, E, f32_dev(1.0), f32_dev(1.0), banks.alpha_gu,
                       banks.alpha_dn)
    assert out.shape == (0, K)


def test_moe_full_size(ops, orc):
    # the MoE workload (E=128, top-8, K=2048, I=768, T=8192), every output:
    # align checked on all 65536 pairs, h on every pair, out on every token;
    # g2 calibrated by the oracle on all 512 rows of the calibration batch
    import torch

    m = synth.MOE
    d = synth.moe_inputs()
    E, top_k, K, I, T = m["E"], m["top_k"], m["K"], m["I"], m["T"]
    banks = Banks(ops, orc, d["gate_up"], d["down"], orc.global_scale(d["cal"]),
                  cal=(d["cal"], d["cal_ids"], d["cal_w"]))
    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    out, ws = banks.run(ops, d["x"], d["ids"], d["w"], h_amax=h_amax)
    views = ops.moe_workspace_views(ws, T, top_k, E, K, I)
    inv = check_align(views, d["ids"], E)
    tokens = np.arange(T)
    res = banks.oracle(orc, d["x"], d["ids"], d["w"])
    flipped, ncf, nsf = check_h(views, inv, res, tokens, top_k, I)
    stats = check_out(bf16_host(out), res, tokens, flipped)
    assert abs(h_amax.item() - res["h_amax"]) <= 1e-5 * res["h_amax"]
    print(f"g2 {banks.g2}, flipped tokens {len(flipped)}/{T}, code flips {ncf}, scale flips {nsf}, {stats}")


# ------------------------------------------------------------ W4A16 layer
# Stage-wise, as the GPU's z is an fp32 sum: h (bf16 by slot) within 2 bf16
# ulp of the oracle's bf16(h), with the floor set by h's error scale and an
# absolute floor of 2^-100 (an fp32 SiLU underflows to 0 for a gate below
# about -87, where |h| < 2^-110; such an h moves no output by a measurable
# amount); then the output against the oracle's down + route sum fed the
# GPU's own h, to the linears' bar (2 bf16 ulp with the Sabs floor, rel-L2
# <= 1e-3).
H_ABS_FLOOR = 2.0 ** -100

def banks16(ops, orc, gate_up, down, check_experts=None):
    """Banks for the W4A16 layer: alpha_e = 1/g_e (no activation global)."""
    return Banks(ops, orc, gate_up, down, 1.0, 1.0, check_experts=check_experts)


def run16(ops, banks, x, ids, w, workspace=None):
    import torch

    T, top_k = ids.shape
    if workspace is None:
        workspace = torch.empty(max(1, ops.moe_w4a16_workspace_bytes(T, top_k, banks.E, banks.K, banks.I)),
                                dtype=torch.uint8, device="cuda")
    out = ops.moe_w4a16(bf16_dev(x), to_dev(ids), to_dev(w), banks.w_gu, banks.w_dn, banks.E, banks.alpha_gu,
                        banks.alpha_dn, workspace=workspace)
    torch.cuda.synchronize()
    return out, workspace


def check16(ops, orc, banks, x, ids, w, out, ws, tokens=None):
    T, top_k = ids.shape
    E, K, I = banks.E, banks.K, banks.I
    views = ops.moe_w4a16_workspace_views(ws, T, top_k, E, K, I)
    if T * top_k <= ops.MOE_W4A16_DIRECT_PAIRS and top_k <= 16 and I <= 2048:
        # the direct path: no align, h at the pair index (skipped pairs unwritten)
        valid = ((ids >= 0) & (ids < E)).reshape(-1)
        inv = np.where(valid, np.arange(T * top_k), -1)
    else:
        inv = check_align(views, ids, E, rows=16)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    args = (banks.o_gu[0], banks.o_gu[1], banks.o_dn[0], banks.o_dn[1], banks.o_alpha_gu, banks.o_alpha_dn)
    res = orc.moe_w4a16(x, ids, w, *args, tokens=tokens)
    hv = views["h"].cpu().numpy().view(np.uint16)
    pairs = (tokens[:, None] * top_k + np.arange(top_k)[None, :]).reshape(-1)
    slots = inv[pairs]
    live = slots >= 0
    h_gpu = np.zeros((len(pairs), I), np.uint16)
    h_gpu[live] = hv[slots[live]]
    hstats = gemm_check(h_gpu[live], res["h"][live], np.maximum(res["h_sabs"][live], 2.0 ** 13 * H_ABS_FLOOR))
    fed = orc.moe_w4a16(x, ids, w, *args, tokens=tokens, h_in=h_gpu)
    ostats = gemm_check(bf16_host(out)[tokens], fed["out"], fed["sabs"])
    return hstats, ostats


@pytest.fixture(scope="module")
def full_banks16(ops, orc):
    m = synth.MOE
    d = synth.moe_inputs()
    banks = banks16(ops, orc, d["gate_up"], d["down"], check_experts=[0, 1, m["E"] - 1])
    return banks, d


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_moe_w4a16_decode(ops, orc, full_banks16, T):
    # the MoE workload's banks (E=128, top-8, K=2048, I=768) at decode batch
    # sizes: the first T tokens of its inputs and routing
    banks, d = full_banks16
    x, ids, w = d["x"][:T], d["ids"][:T], d["w"][:T]
    out, ws = run16(ops, banks, x, ids, w)
    hstats, ostats = check16(ops, orc, banks, x, ids, w, out, ws)
    print(f"T={T}: h {hstats}, out {ostats}")


def test_moe_w4a16_entries_skips_and_repeat(ops, orc):
    # 8 experts, top-2, K=512, I=256, T=90: expert 0 draws most tokens (several
    # 16-pair entries, the last ragged), expert 7 none, some ids skipped; a
    # second call on the same workspace gives the same bits
    E, top_k, K, I, T = 8, 2, 512, 256, 90
    bias = np.zeros(E, np.float32)
    bias[0], bias[7] = 2.5, -30.0
    x, ids, w, _, _, _, gate_up, down = _small_case(303, T, E, top_k, K, I, bias)
    ids = ids.copy()
    ids[::9, 1] = -1
    ids[4::13, 0] = E
    banks = banks16(ops, orc, gate_up, down)
    out1, ws = run16(ops, banks, x, ids, w)
    counts = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
    assert counts[0] > 48 and counts[7] == 0
    check16(ops, orc, banks, x, ids, w, out1, ws)
    out2, _ = run16(ops, banks, x, ids, w, workspace=ws)
    assert (bf16_host(out1) == bf16_host(out2)).all(), "W4A16 MoE must be deterministic"


def test_moe_w4a16_direct_skips_and_repeat(ops, orc):
    # few pairs (the direct path: no align, down and the route sum in one
    # launch): top-3 over 8 experts, T = 7 (21 pairs), ids outside [0, E)
    # skipped, a token with every route skipped; a second call on the same
    # workspace gives the same bits
    E, top_k, K, I, T = 8, 3, 512, 256, 7
    x, ids, w, _, _, _, gate_up, down = _small_case(707, T, E, top_k, K, I)
    ids = ids.copy()
    ids[1, 0] = -1
    ids[4, 2] = E
    ids[6, :] = -1
    assert T * top_k <= ops.MOE_W4A16_DIRECT_PAIRS
    banks = banks16(ops, orc, gate_up, down)
    out1, ws = run16(ops, banks, x, ids, w)
    check16(ops, orc, banks, x, ids, w, out1, ws)
    out2, _ = run16(ops, banks, x, ids, w, workspace=ws)
    assert (bf16_host(out1) == bf16_host(out2)).all(), "W4A16 MoE must be deterministic"
    assert (bf16_host(out1)[6] == 0).all(), "a token with every route skipped is zero"


def test_moe_w4a16_many_pairs(ops, orc):
    # 1200 pairs (more than one align chunk: the three-launch align), ragged
    # entries of 16 over 8 experts; outputs checked on sampled tokens
    E, top_k, K, I, T = 8, 2, 256, 256, 600
    x, ids, w, _, _, _, gate_up, down = _small_case(505, T, E, top_k, K, I)
    banks = banks16(ops, orc, gate_up, down)
    out, ws = run16(ops, banks, x, ids, w)
    check16(ops, orc, banks, x, ids, w, out, ws, tokens=[0, 1, 299, 300, 598, 599])


def test_moe_align_large_count_table(ops, orc):
    # E = 1024 experts, top-8, T = 2100: 16800 pairs in 17 align chunks, so
    # the [chunks, E] count table (17408 entries) is larger than the scan's LDS
    # staging and the scan walks it in global memory.  The align of both
    # layers against a stable sort, W4A16 outputs on sampled tokens, and the
    # W4A4 layer's align on the same inputs; a second W4A16 call gives the
    # same bits.
    E, top_k, K, I, T = 1024, 8, 256, 256, 2100
    x, ids, w, _, _, _, gate_up, down = _small_case(606, T, E, top_k, K, I)
    assert -(-T * top_k // 1024) * E > 16384
    banks = banks16(ops, orc, gate_up, down, check_experts=[0, 511, E - 1])
    out1, ws = run16(ops, banks, x, ids, w)
    check16(ops, orc, banks, x, ids, w, out1, ws, tokens=[0, 1, 1049, 2098, 2099])
    out2, _ = run16(ops, banks, x, ids, w, workspace=ws)
    assert (bf16_host(out1) == bf16_host(out2)).all(), "W4A16 MoE must be deterministic"
    _, ws4 = banks.run(ops, x, ids, w)
    check_align(ops.moe_workspace_views(ws4, T, top_k, E, K, I), ids, E)


def test_moe_w4a16_long_k_and_empty(ops, orc):
    # K = 4096, I = 512 (16 and 2 steps per GEMM: two steps per wave on gate_up)
    import torch

    E, top_k, K, I, T = 4, 2, 4096, 512, 6
    x, ids, w, _, _, _, gate_up, down = _small_case(404, T, E, top_k, K, I)
    banks = banks16(ops, orc, gate_up, down)
    out, ws = run16(ops, banks, x, ids, w)
    check16(ops, orc, banks, x, ids, w, out, ws)
    xe = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    ie = torch.empty((0, top_k), dtype=torch.int32, device="cuda")
    we = torch.empty((0, top_k), dtype=torch.float32, device="cuda")
    assert ops.moe_w4a16(xe, ie, we, banks.w_gu, banks.w_dn, E, banks.alpha_gu, banks.alpha_dn).shape == (0, K)


def test_moe_dispatch_routes(ops, orc):
    # the dispatched layer runs exactly the layer it reports, on both routes
    import torch

    E, top_k, K, I, T = 4, 2, 256, 256, 40
    x, ids, w, cal, cids, cw, gate_up, down = _small_case(606, T, E, top_k, K, I)
    b4 = Banks(ops, orc, gate_up, down, orc.global_scale(cal), cal=(cal, cids, cw), check_experts=[0])
    a_gu16 = torch.empty(E, dtype=torch.float32, device="cuda")
    a_dn16 = torch.empty(E, dtype=torch.float32, device="cuda")
    for e in range(E):  # 1/g_e from the W4A4 alphas' globals: alpha(g_e, 1)
        a_gu16[e] = float(orc.alpha(orc.global_scale(gate_up[e]), np.float32(1.0)))
        a_dn16[e] = float(orc.alpha(orc.global_scale(down[e]), np.float32(1.0)))
    xd, idd, wd = bf16_dev(x), to_dev(ids), to_dev(w)
    g1, g2 = f32_dev(b4.g1), f32_dev(b4.g2)
    direct16 = ops.moe_w4a16(xd, idd, wd, b4.w_gu, b4.w_dn, E, a_gu16, a_dn16)
    direct4 = ops.moe_w4a4(xd, idd, wd, b4.w_gu, b4.w_dn, E, g1, g2, b4.alpha_gu, b4.alpha_dn)
    try:
        for tpe, want in ((20, 0), (0, 1)):   # 40*2/4 = 20 tokens per expert
            ops.set_moe_route_tokens_per_expert(tpe)
            out, route = ops.moe(xd, idd, wd, b4.w_gu, b4.w_dn, E, g1, g2, b4.alpha_gu, b4.alpha_dn, a_gu16, a_dn16)
            assert route == want
            ref = direct16 if want == 0 else direct4
            assert (bf16_host(out) == bf16_host(ref)).all()
        out, route = ops.moe(xd, idd, wd, b4.w_gu, b4.w_dn, E, None, None, None, None, a_gu16, a_dn16)
        assert route == 0 and (bf16_host(out) == bf16_host(direct16)).all()
    finally:
        ops.set_moe_route_tokens_per_expert(14)


# ------------------------------------------------------------ gated MLP
@pytest.mark.parametrize("M,K,I", [(20, 1024, 512), (50, 256, 256), (100, 512, 768), (300, 512, 256),
                                   (1024, 2048, 768), (4000, 512, 2304)])
def test_gated_mlp_w4a4(ops, orc, M, K, I):
    # the dense gated MLP = the MoE layer with one expert, one route of weight
    # 1: h (NVFP4 under g2) against the oracle's with benign flips, then the
    # down linear on the GPU's h against the layer's output.  Tiles of at most
    # 128 rows take the few-rows loop: (20, ...) one group of 32 rows, (50,
    # 256, 256) two, over a single 256-k unit in both GEMMs, (100, ...) four,
    # (300, ...) a 44-row tail tile (two).  (4000, 512, 2304): 16
    # row tiles x 18 blocks = 288 workgroup items on 256 CUs, so the last 32
    # run as 128-row halves, one of them on the ragged last 32 rows
    import torch

    x, _, _, cal, _, _, gate_up, down = _small_case(707 + M, M, 1, 1, K, I, calib_rows=64)
    ids = np.zeros((M, 1), np.int32)
    w = np.ones((M, 1), np.float32)
    cids = np.zeros((cal.shape[0], 1), np.int32)
    cw = np.ones((cal.shape[0], 1), np.float32)
    banks = Banks(ops, orc, gate_up, down, orc.global_scale(cal), cal=(cal, cids, cw))
    xc, xs = ops.quantize_act(bf16_dev(x), f32_dev(banks.g1))
    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    hc, hs = ops.gated_mlp_w4a4(xc, xs, banks.w_gu, banks.alpha_gu[0:1], f32_dev(banks.g2), h_amax=h_amax)
    out = ops.linear_w4a4(hc, hs, banks.w_dn, banks.alpha_dn[0:1])
    res = banks.oracle(orc, x, ids, w)
    views = {"h_codes": hc, "h_scales": hs}
    inv = np.arange(M)
    flipped, ncf, nsf = check_h(views, inv, res, np.arange(M), 1, I)
    stats = check_out(bf16_host(out), res, np.arange(M), flipped)
    assert abs(h_amax.item() - res["h_amax"]) <= 1e-5 * res["h_amax"]
    print(f"M={M}: flipped rows {len(flipped)}, code flips {ncf}, scale flips {nsf}, {stats}")
