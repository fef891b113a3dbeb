"""GPU parity of the W4A16 and W4A4 linears and the dispatch against the
oracle: max |err| <= 2 bf16 ulp (with the Sabs floor) and rel-L2 <= 1e-3."""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_host, f32_dev, gemm_check, schedules_for, u8_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


class Quantized:
    """A bf16 weight quantized on the GPU (checked against the oracle's codes)
    plus the oracle's own codes for the reference."""

    def __init__(self, ops, orc, w_bits, check_rows=None):
        self.bits = w_bits
        self.g = orc.global_scale(w_bits)
        wd = bf16_dev(w_bits)
        gd = ops.global_scale(wd)
        assert gd.item() == self.g
        c, s = ops.quantize_act(wd, gd)
        self.w = ops.prepare_weight(c, s)
        self.alpha = ops.alpha(gd)
        assert self.alpha.item() == orc.alpha(self.g)
        self.g_dev = gd
        rows = np.arange(w_bits.shape[0]) if check_rows is None else check_rows
        oc, os_ = orc.quantize(w_bits[rows], self.g)
        assert (u8_host(c)[rows] == oc).all() and (u8_host(s)[rows] == os_).all(), "weight quantization mismatch"
        if check_rows is None:
            self.codes, self.scales = oc, os_


def test_w4a16_small_config(ops, orc):
    # W4A16 linear, M=4, N=512, K=1024
    W = synth.normal_bf16(synth.seed_for("w4a16_small", synth.ROLE_W), 512, 1024)
    a = synth.normal_bf16(synth.seed_for("w4a16_small", synth.ROLE_A), 4, 1024)
    q = Quantized(ops, orc, W)
    out = ops.linear_w4a16(bf16_dev(a), q.w, q.alpha)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    gemm_check(bf16_host(out), ref, sabs)


@pytest.mark.parametrize("shape_index", range(4))
def test_w4a16_decode_sweep(ops, orc, shape_index):
    N, K = synth.W4A16_DECODE_SHAPES[shape_index]
    W = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_W, shape_index), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_A, shape_index), 16, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for M in synth.W4A16_DECODE_M:
        out = ops.linear_w4a16(ad[:M], q.w, q.alpha)
        gemm_check(bf16_host(out), ref[:M], sabs[:M])


def test_w4a16_every_schedule(ops, orc):
    # ragged N (not a multiple of 16 or of a workgroup's 8 tiles), K with an odd
    # number of 256-k steps (17: uneven chunks), M between powers of two
    N, K, M = 1000, 4352, 7
    W = synth.normal_bf16(11, N, K)
    a = synth.normal_bf16(12, M, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for sch, ks, kc in schedules_for(M, K):
        out = ops.linear_w4a16(ad, q.w, q.alpha, schedule=sch, ksplit=ks, chunk_steps=kc)
        gemm_check(bf16_host(out), ref, sabs)
    # every token count on a short K, including a chunk longer than K
    K2 = 512
    W2 = synth.normal_bf16(13, 300, K2)
    a2 = synth.normal_bf16(14, 16, K2)
    q2 = Quantized(ops, orc, W2)
    ref2, _, sabs2 = orc.linear_w4a16(a2, q2.codes, q2.scales, orc.alpha(q2.g))
    a2d = bf16_dev(a2)
    for M in range(1, 17):
        dot = ([(4, 2, 0), (4, 1, 0)] if M <= 4 else []) + [(3, 2, 2)]
        for sch, ks, kc in [(0, 0, 0), (1, 2, 0), (2, 0, 1), (2, 0, 4 if M <= 16 else 1)] + dot:
            out = ops.linear_w4a16(a2d[:M], q2.w, q2.alpha, schedule=sch, ksplit=ks, chunk_steps=kc)
            gemm_check(bf16_host(out), ref2[:M], sabs2[:M])


def test_w4a16_cache_policies(ops, orc):
    # the dot schedule's cache-policy tactic changes load hints only: the
    # same bits as the default policy, within the bar of the oracle
    N, K = 1000, 4352
    W = synth.normal_bf16(21, N, K)
    a = synth.normal_bf16(22, 4, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for M in (1, 2, 4):
        base = bf16_host(ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=4, ksplit=7))
        gemm_check(base, ref[:M], sabs[:M])
        for cp in (1, 2):
            got = bf16_host(ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=4, ksplit=7, cache_policy=cp))
            assert (got == base).all(), (M, cp)


def test_w4a16_long_k(ops, orc):
    # K/256 = 72 steps: long runs per wave, many LDS chunks
    N, K = 200, 256 * 72
    W = synth.normal_bf16(15, N, K)
    a = synth.normal_bf16(16, 16, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for sch, ks, kc in [(0, 0, 0), (1, 1, 0), (1, 16, 0), (2, 0, 4), (2, 0, 3)]:
        for M in (1, 16):
            out = ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=sch, ksplit=ks, chunk_steps=kc)
            gemm_check(bf16_host(out), ref[:M], sabs[:M])
    out = ops.linear_w4a16(ad[:1], q.w, q.alpha, schedule=2, chunk_steps=64)  # one chunk of 64 steps (M = 1)
    gemm_check(bf16_host(out), ref[:1], sabs[:1])
    for sch, ks, r in ((4, 16, 0), (4, 9, 0)):  # dot: 72 steps over 15 / 8 waves
        for M in (1, 2, 3, 4):
            out = ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=sch, ksplit=ks, chunk_steps=r)
            gemm_check(bf16_host(out), ref[:M], sabs[:M])


def test_w4a16_many_tokens(ops, orc):
    # 17..64 tokens: the shared schedule with up to four 16-token groups on
    # one dequantized weight, on a ragged N and an odd number of K steps, at
    # the default chunk and at explicit chunks
    N, K = 1000, 4352
    W = synth.normal_bf16(25, N, K)
    a = synth.normal_bf16(26, 64, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for M in (17, 24, 31, 32, 33, 47, 48, 49, 63, 64):
        out = ops.linear_w4a16(ad[:M], q.w, q.alpha)
        gemm_check(bf16_host(out), ref[:M], sabs[:M])
        for kc in (1, 64 // (16 * -(-M // 16))):  # the largest chunk of the padded rows
            out = ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=2, chunk_steps=kc)
            gemm_check(bf16_host(out), ref[:M], sabs[:M])
    # long K: 72 steps in chunks of one step
    N2, K2 = 200, 256 * 72
    W2 = synth.normal_bf16(27, N2, K2)
    a2 = synth.normal_bf16(28, 64, K2)
    q2 = Quantized(ops, orc, W2)
    ref2, _, sabs2 = orc.linear_w4a16(a2, q2.codes, q2.scales, orc.alpha(q2.g))
    a2d = bf16_dev(a2)
    for M in (20, 64):
        gemm_check(bf16_host(ops.linear_w4a16(a2d[:M], q2.w, q2.alpha)), ref2[:M], sabs2[:M])


def test_w4a16_default_very_long_k(ops, orc):
    # K = 256 * 129: more steps than the dot schedule's 16 waves x 8 steps, so
    # the default takes a split schedule at every M (an invalid dot config
    # there would fail the launch)
    N, K = 40, 256 * 129
    W = synth.normal_bf16(23, N, K)
    a = synth.normal_bf16(24, 16, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for M in (1, 2, 3, 16):
        out = ops.linear_w4a16(ad[:M], q.w, q.alpha)
        gemm_check(bf16_host(out), ref[:M], sabs[:M])


def test_w4a16_default_many_tiles(ops, orc):
    # 688 tiles (more than 2.5 per CU on 256 CUs): the default runs two tiles
    # per workgroup; at 43 steps of K it keeps about 4 steps per wave
    for N, K, seed in ((11008, 512, 17), (512, 256 * 43, 19)):
        W = synth.normal_bf16(seed, N, K)
        a = synth.normal_bf16(seed + 1, 16, K)
        q = Quantized(ops, orc, W)
        ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
        ad = bf16_dev(a)
        for M in (1, 3, 4, 8, 13, 16):
            out = ops.linear_w4a16(ad[:M], q.w, q.alpha)
            gemm_check(bf16_host(out), ref[:M], sabs[:M])


def test_w4a16_shared_wide_ragged(ops, orc):
    # 3073 tiles (at least 1.5 x 8 tiles per CU on 256 CUs): the shared schedule
    # runs 16 tiles per workgroup, the last workgroup holding one partial tile
    # (N = 3072 * 16 + 8); M = 16 (one token group) and 40 (three), default and
    # explicit chunks; M = 5 and 8 take the two-tile split there
    N, K = 3072 * 16 + 8, 512
    W = synth.normal_bf16(29, N, K)
    a = synth.normal_bf16(30, 40, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for M in (5, 8, 16, 40):
        out = ops.linear_w4a16(ad[:M], q.w, q.alpha)
        gemm_check(bf16_host(out), ref[:M], sabs[:M])
    for M, kc in ((16, 1), (16, 2), (40, 1)):
        out = ops.linear_w4a16(ad[:M], q.w, q.alpha, schedule=2, chunk_steps=kc)
        gemm_check(bf16_host(out), ref[:M], sabs[:M])


def test_prepared_layout(ops, orc):
    """The tiled weight follows the documented unit layout byte for byte."""
    N, K = 40, 512
    W = synth.normal_bf16(17, N, K)
    q = Quantized(ops, orc, W)
    tiled = u8_host(q.w.data)
    steps, tiles = K // 256, (N + 15) // 16
    assert tiled.size >= tiles * steps * 2304
    codes = np.zeros((tiles * 16, K // 2), np.uint8)
    scales = np.zeros((tiles * 16, K // 16), np.uint8)
    codes[:N], scales[:N] = q.codes, q.scales
    for t in range(tiles):
        for s in range(steps):
            u = tiled[(t * steps + s) * 2304:(t * steps + s + 1) * 2304]
            for lane in range(64):
                r, qq = lane % 16, lane // 16
                row = 16 * t + r
                groups = [4 * p + qq for p in range(4)]
                want = np.concatenate([codes[row, 128 * s + 8 * g:128 * s + 8 * g + 8] for g in groups])
                got = np.concatenate([u[16 * lane:16 * lane + 16], u[1024 + 16 * lane:1024 + 16 * lane + 16]])
                assert (got == want).all(), (t, s, lane)
                assert (u[2048 + 4 * lane:2048 + 4 * lane + 4] == scales[row, 16 * s + np.array(groups)]).all()


@pytest.mark.parametrize("M,N,K", [(1, 12, 256), (16, 12, 512), (3, 17, 768), (9, 100, 1024), (13, 4000, 2048)])
def test_w4a16_edges(ops, orc, M, N, K):
    import torch

    W = synth.normal_bf16(20 + N, N, K)
    a = synth.normal_bf16(30 + M, M, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    # strided input (lda > K) and output (ldo > N), with guard values around the output
    lda, ldo = K + 64, N + 5
    abuf = torch.zeros((M, lda), dtype=torch.bfloat16, device="cuda")
    abuf[:, :K] = bf16_dev(a)
    obuf = torch.full((M + 1, ldo), 7.0, dtype=torch.bfloat16, device="cuda")
    ops.linear_w4a16(abuf[:, :K], q.w, q.alpha, out=obuf[:M, :N])
    o = bf16_host(obuf)
    gemm_check(o[:M, :N], ref, sabs)
    assert (o[:M, N:] == 0x40E0).all() and (o[M] == 0x40E0).all(), "write outside the output"


def test_w4a16_empty_and_limits(ops, orc):
    import torch

    W = synth.normal_bf16(5, 64, 256)
    q = Quantized(ops, orc, W)
    out = ops.linear_w4a16(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), q.w, q.alpha)
    assert out.shape == (0, 64)
    with pytest.raises(ValueError):
        ops.linear_w4a16(torch.zeros((65, 256), dtype=torch.bfloat16, device="cuda"), q.w, q.alpha)
    with pytest.raises(ValueError):  # above 16 tokens only the shared schedule
        ops.linear_w4a16(torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda"), q.w, q.alpha, schedule=1,
                         ksplit=1)


def test_w4a16_deterministic(ops, orc):
    W = synth.normal_bf16(8, 3584, 5120)
    q = Quantized(ops, orc, W, check_rows=np.arange(0, 3584, 97))
    a = bf16_dev(synth.normal_bf16(9, 16, 5120))
    for M, sch, ks, kc in [(16, 0, 0, 0), (16, 1, 7, 0), (16, 2, 0, 4), (4, 0, 0, 0), (4, 4, 7, 0), (1, 0, 0, 0), (2, 4, 7, 0), (16, 3, 4, 2), (8, 3, 7, 2)]:
        o1 = bf16_host(ops.linear_w4a16(a[:M], q.w, q.alpha, schedule=sch, ksplit=ks, chunk_steps=kc))
        for _ in range(3):
            o2 = ops.linear_w4a16(a[:M], q.w, q.alpha, schedule=sch, ksplit=ks, chunk_steps=kc)
            assert (bf16_host(o2) == o1).all()


# ------------------------------------------------------------------ W4A4

def _w4a4_case(ops, orc, W, a, cal, rows=None):
    """Quantize W and a on the GPU (codes checked against the oracle), run the
    W4A4 linear and check it against the oracle on all outputs (or on the
    given rows, all columns)."""
    q = Quantized(ops, orc, W)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    assert gad.item() == ga
    ad = bf16_dev(a)
    ac, as_ = ops.quantize_act(ad, gad)
    al = ops.alpha(q.g_dev, gad)
    assert al.item() == orc.alpha(q.g, ga)
    out = bf16_host(ops.linear_w4a4(ac, as_, q.w, al))
    sel = slice(None) if rows is None else rows
    oac, oas = orc.quantize(a[sel], ga)
    assert (u8_host(ac)[sel] == oac).all() and (u8_host(as_)[sel] == oas).all()
    ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
    return gemm_check(out[sel], ref, sabs)


@pytest.fixture(scope="module")
def prefill(ops, orc):
    """The W4A4 prefill workload (N=8704, K=5120, a of 8192 rows whose
    prefixes are the smaller batches, 512-row calibration batch): the weight
    and activations quantized on the GPU and checked against the oracle's
    codes, and the oracle's output over all 8192 x 8704 outputs."""
    N, K = 8704, 5120
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 8192, K)
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    q = Quantized(ops, orc, W)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    assert gad.item() == ga
    ac, as_ = ops.quantize_act(bf16_dev(a), gad)
    oac, oas = orc.quantize(a, ga)
    assert (u8_host(ac) == oac).all() and (u8_host(as_) == oas).all(), "activation quantization mismatch"
    al = ops.alpha(q.g_dev, gad)
    assert al.item() == orc.alpha(q.g, ga)
    ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
    return dict(q=q, ac=ac, as_=as_, al=al, ref=ref, sabs=sabs)


@pytest.mark.parametrize("M", [1024, 4096, 8192])
def test_w4a4_prefill_full(ops, prefill, M):
    # every output of the W4A4 prefill linear at each batch size
    p = prefill
    out = bf16_host(ops.linear_w4a4(p["ac"][:M], p["as_"][:M], p["q"].w, p["al"]))
    stats = gemm_check(out, p["ref"][:M], p["sabs"][:M])
    print(f"M={M}: {stats}")


def test_w4a4_split_final_round(ops, orc):
    # 17 x 16 tiles of 256 x 256 on 256 CUs: the 16 tiles of the final round
    # run as 128-row halves; checked in full
    N, K, M = 4352, 1024, 4096
    W = synth.normal_bf16(81, N, K)
    a = synth.normal_bf16(82, M, K)
    cal = synth.normal_bf16(83, 64, K)
    _w4a4_case(ops, orc, W, a, cal)


def test_w4a4_whole_round_and_leftover(ops, orc):
    # 9 x 34 = 306 tiles: a whole round, then 50 leftover tiles run as
    # 128-row halves (on a 256-CU device); checked in full
    N, K, M = 8704, 1024, 2304
    W = synth.normal_bf16(84, N, K)
    a = synth.normal_bf16(85, M, K)
    cal = synth.normal_bf16(86, 64, K)
    _w4a4_case(ops, orc, W, a, cal)


def test_w4a4_few_tiles_long_k(ops, orc):
    # 32 tiles over 80 steps of K, far fewer tiles than CUs; checked in full
    N, K, M = 2048, 5120, 1024
    W = synth.normal_bf16(87, N, K)
    a = synth.normal_bf16(88, M, K)
    cal = synth.normal_bf16(89, 64, K)
    _w4a4_case(ops, orc, W, a, cal)


@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (130, 200, 512), (127, 129, 768), (300, 1000, 1024), (17, 8, 256),
                                   (700, 520, 2048)])
def test_w4a4_ragged(ops, orc, M, N, K):
    W = synth.normal_bf16(40 + N, N, K)
    a = synth.normal_bf16(50 + M, M, K)
    cal = synth.normal_bf16(60 + M, 64, K)
    _w4a4_case(ops, orc, W, a, cal)


@pytest.mark.parametrize("N,K", [(1000, 1280), (4104, 256), (600, 3072)])
def test_w4a4_few_rows_every_group(ops, orc, N, K):
    # batches of at most 128 rows run on 256 weight rows per workgroup with
    # 1, 2 or 4 groups of 32 activation rows: every group count, the ragged
    # rows of each, N not a multiple of 16 or 256, K of 5, 1 and 12 units
    # (an odd count, a single one); with and without the split of K.  Each
    # batch checked in full
    import torch

    M_max = 128
    W = synth.normal_bf16(170 + N, N, K)
    a = synth.normal_bf16(171 + N, M_max, K)
    cal = synth.normal_bf16(172 + N, 64, K)
    q = Quantized(ops, orc, W)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    ac, as_ = ops.quantize_act(bf16_dev(a), gad)
    al = ops.alpha(q.g_dev, gad)
    oac, oas = orc.quantize(a, ga)
    ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
    for M in (1, 2, 31, 32, 33, 63, 64, 65, 97, 128):
        out = bf16_host(ops.linear_w4a4(ac[:M], as_[:M], q.w, al))
        gemm_check(out, ref[:M], sabs[:M])
        need = ops.linear_w4a4_workspace_bytes(M, N, K)
        if need:
            ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
            gemm_check(bf16_host(ops.linear_w4a4(ac[:M], as_[:M], q.w, al, workspace=ws)), ref[:M], sabs[:M])


def test_w4a4_deterministic(ops, orc):
    W = synth.normal_bf16(70, 1024, 1024)
    q = Quantized(ops, orc, W)
    a = bf16_dev(synth.normal_bf16(71, 512, 1024))
    g = f32_dev(400.0)
    ac, as_ = ops.quantize_act(a, g)
    al = ops.alpha(q.g_dev, g)
    o1 = bf16_host(ops.linear_w4a4(ac, as_, q.w, al))
    for _ in range(3):
        assert (bf16_host(ops.linear_w4a4(ac, as_, q.w, al)) == o1).all()


@pytest.mark.parametrize("M,N,K", [(1, 512, 2048), (17, 1002, 4352), (128, 3000, 2048), (200, 1000, 1024),
                                   (300, 520, 5120)])
def test_w4a4_split_k(ops, orc, M, N, K):
    # few output tiles (on a 256-CU device): K split across workgroups, fp32
    # partials added in range order by a second launch.  Checked in full
    # against the oracle; the workspace is poisoned with NaN bytes, so an
    # element a partial tile does not write shows up; repeated calls give the
    # same bits
    import torch

    need = ops.linear_w4a4_workspace_bytes(M, N, K)
    assert need > 0, "the shape should split K"
    W = synth.normal_bf16(120 + N, N, K)
    a = synth.normal_bf16(130 + M, M, K)
    cal = synth.normal_bf16(140 + M, 64, K)
    q = Quantized(ops, orc, W)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    ac, as_ = ops.quantize_act(bf16_dev(a), gad)
    al = ops.alpha(q.g_dev, gad)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=ws))
    oac, oas = orc.quantize(a, ga)
    ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
    print(gemm_check(out, ref, sabs))
    for _ in range(2):
        ws.fill_(0xFF)
        assert (bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=ws)) == out).all()
    # one launch over all of K (no workspace) meets the same bar
    gemm_check(bf16_host(ops.linear_w4a4(ac, as_, q.w, al)), ref, sabs)


def test_w4a4_split_k_not_taken(ops, orc):
    # fewer than four 256-k units, or tiles for more than half the CUs: one
    # launch, and the workspace call needs no workspace
    assert ops.linear_w4a4_workspace_bytes(16, 1000, 768) == 0
    assert ops.linear_w4a4_workspace_bytes(1024, 8704, 5120) == 0
    M, N, K = 16, 1000, 768
    W = synth.normal_bf16(150, N, K)
    q = Quantized(ops, orc, W)
    a = bf16_dev(synth.normal_bf16(151, M, K))
    g = f32_dev(400.0)
    ac, as_ = ops.quantize_act(a, g)
    al = ops.alpha(q.g_dev, g)
    o1 = bf16_host(ops.linear_w4a4(ac, as_, q.w, al))
    o2 = bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=True))
    assert (o1 == o2).all()


def test_w4a4_split_k_entry_points_agree(ops, orc):
    # the dispatched linear's W4A4 route, its allocation-free form and
    # linear_w4a4 with a workspace run the same split-K kernels: same bits
    import torch

    N, K, M = 3000, 2048, 100
    assert ops.linear_w4a4_workspace_bytes(M, N, K) > 0
    W = synth.normal_bf16(160, N, K)
    a = synth.normal_bf16(161, M, K)
    cal = synth.normal_bf16(162, 64, K)
    q = Quantized(ops, orc, W)
    gad = ops.global_scale(bf16_dev(cal))
    a4 = ops.alpha(q.g_dev, gad)
    ad = bf16_dev(a)
    ops.set_route_m_max(64)
    try:
        out_lin, route = ops.linear(ad, q.w, gad, q.alpha, a4)
        assert route == 1
        out_na = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        assert ops.linear_noalloc(ad, q.w, gad, q.alpha, a4, out_na) == 1
    finally:
        ops.set_route_m_max(16)
    ac, as_ = ops.quantize_act(ad, gad)
    out_ws = ops.linear_w4a4(ac, as_, q.w, a4, workspace=True)
    assert (bf16_host(out_lin) == bf16_host(out_ws)).all()
    assert (bf16_host(out_na) == bf16_host(out_ws)).all()
    # a workspace with room for the activations only: the one-launch kernel
    act_bytes = ops.linear_workspace_bytes(M, N, K) - ops.linear_w4a4_workspace_bytes(M, N, K)
    small = torch.empty(act_bytes, dtype=torch.uint8, device="cuda")
    ops.set_route_m_max(64)
    try:
        out_small, route = ops.linear(ad, q.w, gad, q.alpha, a4, workspace=small)
    finally:
        ops.set_route_m_max(16)
    assert route == 1
    assert (bf16_host(out_small) == bf16_host(ops.linear_w4a4(ac, as_, q.w, a4))).all()


# ------------------------------------------------------------------ dispatch

def test_dispatch_routes_and_numerics(ops, orc):
    # the routes at a smaller N (they do not depend on N), and a missing
    # activation global
    N, K = 4096, 5120
    W = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_A), 256, K)
    cal = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_CAL), 512, K)
    q = Quantized(ops, orc, W)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    a16 = q.alpha
    a4 = ops.alpha(q.g_dev, gad)
    ad = bf16_dev(a)
    ops.set_route_m_max(16)
    for M in [1, 8, 16, 17, 64, 256]:
        out, route = ops.linear(ad[:M], q.w, gad, a16, a4)
        assert route == ops.route(M, N, K, True) == (1 if M > 16 else 0)
        if route == 0:
            ref, _, sabs = orc.linear_w4a16(a[:M], q.codes, q.scales, orc.alpha(q.g))
        else:
            oac, oas = orc.quantize(a[:M], ga)
            ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
        gemm_check(bf16_host(out), ref, sabs)
    # no activation global: always W4A16
    out, route = ops.linear(ad[:8], q.w, None, a16, None)
    assert route == 0
    # the largest threshold M* = 64 (the W4A16 kernels' limit): W4A16 up to 64
    # tokens, W4A4 above
    ops.set_route_m_max(64)
    for M in (17, 40, 64, 65, 100):
        out, route = ops.linear(ad[:M], q.w, gad, a16, a4)
        assert route == (1 if M > 64 else 0)
        if route == 0:
            ref, _, sabs = orc.linear_w4a16(a[:M], q.codes, q.scales, orc.alpha(q.g))
        else:
            oac, oas = orc.quantize(a[:M], ga)
            ref, _, sabs = orc.linear_w4a4(oac, oas, q.codes, q.scales, orc.alpha(q.g, ga))
        gemm_check(bf16_host(out), ref, sabs)
    ops.set_route_m_max(16)


@pytest.fixture(scope="module")
def fused_large(ops, orc):
    """The large fused-weight workload at its own shape: N=62080, K=5120 (one
    global for the whole tensor), a of 8192 rows (the sweep's batches are its
    prefixes), a 512-row calibration batch.  Weight and activation codes are
    checked against the oracle's."""
    import torch

    N, K = synth.FUSED_LARGE["N"], synth.FUSED_LARGE["K"]
    W = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_A), 8192, K)
    cal = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_CAL), 512, K)
    q = Quantized(ops, orc, W)
    del W
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    assert gad.item() == ga
    ad = bf16_dev(a)
    ac, as_ = ops.quantize_act(ad, gad)
    oac, oas = orc.quantize(a, ga)
    assert (u8_host(ac) == oac).all() and (u8_host(as_) == oas).all(), "activation quantization mismatch"
    del ac, as_
    torch.cuda.empty_cache()
    return dict(q=q, a=a, ad=ad, ga=ga, gad=gad, oac=oac, oas=oas, a4=ops.alpha(q.g_dev, gad), N=N, K=K)


def test_fused_large_w4a16_full(ops, orc, fused_large):
    # the dispatched linear on the W4A16 route at M = 1, 8, 16, and the W4A16
    # kernels at M = 24, 32, 64: every output
    f = fused_large
    q = f["q"]
    ref, _, sabs = orc.linear_w4a16(f["a"][:64], q.codes, q.scales, orc.alpha(q.g))
    ops.set_route_m_max(16)
    for M in (1, 8, 16):
        out, route = ops.linear(f["ad"][:M], q.w, f["gad"], q.alpha, f["a4"])
        assert route == 0
        stats = gemm_check(bf16_host(out), ref[:M], sabs[:M])
        print(f"M={M}: {stats}")
    # the W4A16 kernels above 16 tokens (the crossover region), called directly
    for M in (24, 32, 64):
        out = ops.linear_w4a16(f["ad"][:M], q.w, q.alpha)
        stats = gemm_check(bf16_host(out), ref[:M], sabs[:M])
        print(f"M={M}: {stats}")


def test_fused_large_w4a4_full(ops, orc, fused_large):
    # the dispatched linear on the W4A4 route at M = 64, 256, 1024 (every
    # output), and the W4A4 route called directly at M = 16 (the crossover)
    f = fused_large
    q = f["q"]
    ref, _, sabs = orc.linear_w4a4(f["oac"][:1024], f["oas"][:1024], q.codes, q.scales, orc.alpha(q.g, f["ga"]))
    ops.set_route_m_max(16)
    for M in (64, 256, 1024):
        out, route = ops.linear(f["ad"][:M], q.w, f["gad"], q.alpha, f["a4"])
        assert route == 1
        stats = gemm_check(bf16_host(out), ref[:M], sabs[:M])
        print(f"M={M}: {stats}")
    ac, as_ = ops.quantize_act(f["ad"][:16], f["gad"])
    out = ops.linear_w4a4(ac, as_, q.w, f["a4"])
    gemm_check(bf16_host(out), ref[:16], sabs[:16])


def test_fused_large_w4a4_row_blocks(ops, orc, fused_large):
    # M = 4096 and 8192 through the dispatched linear: every output of whole
    # 256-row blocks (the first, one in the middle, and the last)
    import torch

    f = fused_large
    q = f["q"]
    ops.set_route_m_max(16)
    for M in (4096, 8192):
        out, route = ops.linear(f["ad"][:M], q.w, f["gad"], q.alpha, f["a4"])
        assert route == 1
        rows = np.concatenate([np.arange(0, 256), np.arange(M // 2, M // 2 + 256), np.arange(M - 256, M)])
        ref, _, sabs = orc.linear_w4a4(f["oac"][rows], f["oas"][rows], q.codes, q.scales, orc.alpha(q.g, f["ga"]))
        got = bf16_host(out[torch.from_numpy(rows).cuda()])
        stats = gemm_check(got, ref, sabs)
        print(f"M={M}: {stats}")
        del out


# ------------------------------------------------------ read diagnostic

def test_stream_read_reads_every_piece(ops):
    """The streaming-read diagnostic loads every 16-byte piece: a piece whose
    dwords XOR to the kernel's constant, placed anywhere (the first, a middle
    and the last piece), is seen; a buffer without one leaves the sink alone.
    The buffer is left unchanged."""
    import torch

    n = 1 << 20  # bytes: 65536 pieces, 256 workgroups
    for where in (None, 0, 12345, n // 16 - 1):
        buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
        if where is not None:
            buf[4 * where] = np.int32(np.uint32(0x6A09E667).view(np.int32))
        before = buf.clone()
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        ops.stream_read(buf, sink)
        torch.cuda.synchronize()
        got = int(np.int32(sink.item()).view(np.uint32))
        assert got == (0 if where is None else 0x6A09E667), where
        assert torch.equal(buf, before)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    buf[60] = np.int32(np.uint32(0x6A09E667).view(np.int32))
    ops.stream_read(buf, sink, nbytes=224)  # the last piece is past nbytes
    torch.cuda.synchronize()
    assert sink.item() == 0
