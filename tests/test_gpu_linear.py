"""GPU parity of the W4A16 and W4A4 linears and the dispatch against the
oracle: max |err| <= 2 bf16 ulp (with the Sabs floor) and rel-L2 <= 1e-3."""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_f64, bf16_host, f32_dev, gemm_check, u8_host

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


SCHEDULES = ([(1, ks, 0) for ks in (1, 2, 3, 7, 16)] + [(2, 0, kc) for kc in (1, 2, 3, 4, 17)]
             + [(3, ks, 0) for ks in (1, 3, 7, 16)] + [(3, ks, 2) for ks in (1, 3, 7, 8)]
             + [(4, ks, 0) for ks in (1, 3, 7, 16)])


def _valid(sch, M, K):
    steps = K // 256
    if sch[0] == 2:
        return M * min(sch[2], steps) <= 64
    if sch[0] == 3:  # chunk_steps 2: two tiles per workgroup, at most 8 waves
        ks = min(sch[1], steps)
        per = -(-steps // ks)
        return per <= 8 and (sch[2] < 2 or -(-steps // per) <= 8)
    if sch[0] == 4:  # dot: M <= 4, <= 8 steps per wave
        ks = min(sch[1], steps)
        return M <= 4 and -(-steps // ks) <= 8
    return True


def _schedules_for(M, K):
    return [(0, 0, 0)] + [sch for sch in SCHEDULES if _valid(sch, M, K)]


def test_w4a16_every_schedule(ops, orc):
    # ragged N (not a multiple of 16 or of a workgroup's 8 tiles), K with an odd
    # number of 256-k steps (17: uneven chunks), M between powers of two
    N, K, M = 1000, 4352, 7
    W = synth.normal_bf16(11, N, K)
    a = synth.normal_bf16(12, M, K)
    q = Quantized(ops, orc, W)
    ref, _, sabs = orc.linear_w4a16(a, q.codes, q.scales, orc.alpha(q.g))
    ad = bf16_dev(a)
    for sch, ks, kc in _schedules_for(M, K):
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
        ops.linear_w4a16(torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda"), q.w, q.alpha)


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

def _w4a4_case(ops, orc, W, a, cal, rows=None, cols=None, check_rows=None, ws=None):
    q = Quantized(ops, orc, W, check_rows=check_rows)
    ga = orc.global_scale(cal)
    gad = ops.global_scale(bf16_dev(cal))
    assert gad.item() == ga
    ad = bf16_dev(a)
    ac, as_ = ops.quantize_act(ad, gad)
    al = ops.alpha(q.g_dev, gad)
    assert al.item() == orc.alpha(q.g, ga)
    out = bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=ws))
    if ws is not None:
        check_ws_clean(ops, ws)
    oac, oas = orc.quantize(a if rows is None else a[rows], ga)
    if rows is None:
        assert (u8_host(ac) == oac).all() and (u8_host(as_) == oas).all()
    else:
        assert (u8_host(ac)[rows] == oac).all() and (u8_host(as_)[rows] == oas).all()
    if cols is None:
        wc, ws = q.codes, q.scales
        sel_out = out if rows is None else out[rows]
        ref, _, sabs = orc.linear_w4a4(oac, oas, wc, ws, orc.alpha(q.g, ga))
    else:
        wc, ws = orc.quantize(W[cols], q.g)
        ref, _, sabs = orc.linear_w4a4(oac, oas, wc, ws, orc.alpha(q.g, ga))
        sel_out = out[np.ix_(rows, cols)]
    return gemm_check(sel_out, ref, sabs)


def test_w4a4_prefill_m1024_full(ops, orc):
    N, K = 8704, 5120
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 1024, K)
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    _w4a4_case(ops, orc, W, a, cal)


@pytest.mark.parametrize("M", [4096, 8192])
def test_w4a4_prefill_sampled(ops, orc, M):
    N, K = 8704, 5120
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 8192, K)[:M]
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([rng.integers(0, M, 96), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, N, 384), [0, N - 1]]))
    _w4a4_case(ops, orc, W, a, cal, rows=rows, cols=cols, check_rows=cols)


def test_w4a4_split_final_round(ops, orc):
    # 17 x 16 tiles of 256 x 256 on 256 CUs: the 16 tiles of the final round
    # run as 128-row halves (rows 3072.., cols 3328.. in the grouped tile
    # order); checked in full there, and on sampled rows elsewhere
    N, K, M = 4352, 1024, 4096
    W = synth.normal_bf16(81, N, K)
    a = synth.normal_bf16(82, M, K)
    cal = synth.normal_bf16(83, 64, K)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(3072, 4096), rng.integers(0, 3072, 64)]))
    cols = np.unique(np.concatenate([np.arange(3328, 4352), rng.integers(0, 3328, 64)]))
    _w4a4_case(ops, orc, W, a, cal, rows=rows, cols=cols)


@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (130, 200, 512), (127, 129, 768), (300, 1000, 1024), (17, 8, 256)])
def test_w4a4_ragged(ops, orc, M, N, K):
    W = synth.normal_bf16(40 + N, N, K)
    a = synth.normal_bf16(50 + M, M, K)
    cal = synth.normal_bf16(60 + M, 64, K)
    _w4a4_case(ops, orc, W, a, cal)


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


# ------------------------------------------------------- W4A4, stream-K finish

def poisoned_ws(ops, ws=None):
    """A stream-K workspace whose partial slots hold NaN (flags zero), so a
    finishing workgroup that read a stale copy of a partial instead of the
    one just published would produce NaN, not a plausible sum."""
    import torch

    if ws is None:
        ws = ops.w4a4_workspace()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws[:cus * 256 * 1024].fill_(0xFF)
    return ws


def check_ws_clean(ops, ws):
    """After a call the stream-K flags and the timed-out-wait count are zero."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tail = ws[cus * 256 * 1024:cus * 256 * 1024 + 4 * cus + 4].cpu().numpy()
    assert (tail == 0).all(), "stream-K flags left set or a wait timed out"


def test_w4a4_streamk_full_rounds(ops, orc):
    # 9 x 34 = 306 tiles: a whole round, then 50 leftover tiles cut between
    # the CUs (on a 256-CU device); checked in full
    N, K, M = 8704, 1024, 2304
    W = synth.normal_bf16(84, N, K)
    a = synth.normal_bf16(85, M, K)
    cal = synth.normal_bf16(86, 64, K)
    _w4a4_case(ops, orc, W, a, cal, ws=poisoned_ws(ops))


def test_w4a4_streamk_small_full(ops, orc):
    # 32 tiles, each cut into 4 pieces of 20 steps; checked in full
    N, K, M = 2048, 5120, 1024
    W = synth.normal_bf16(87, N, K)
    a = synth.normal_bf16(88, M, K)
    cal = synth.normal_bf16(89, 64, K)
    _w4a4_case(ops, orc, W, a, cal, ws=poisoned_ws(ops))


def test_w4a4_streamk_m4096_sampled(ops, orc):
    # 544 tiles: two whole rounds, then the 32 tiles of grouped positions
    # 512.. (rows 3072.., cols 6656.. on a 256-CU device) split 8 ways
    N, K, M = 8704, 5120, 4096
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 8192, K)[:M]
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.integers(3072, M, 64), rng.integers(0, 3072, 32), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(6656, N, 256), rng.integers(0, 6656, 96), [0, N - 1]]))
    _w4a4_case(ops, orc, W, a, cal, rows=rows, cols=cols, check_rows=cols, ws=poisoned_ws(ops))


@pytest.mark.parametrize("M,N,K", [(1, 16, 256), (130, 200, 512), (300, 1000, 1024), (700, 520, 2048)])
def test_w4a4_streamk_ragged(ops, orc, M, N, K):
    # fewer tiles than CUs: each tile cut into up to 8 pieces of a few steps
    W = synth.normal_bf16(40 + N, N, K)
    a = synth.normal_bf16(50 + M, M, K)
    cal = synth.normal_bf16(60 + M, 64, K)
    _w4a4_case(ops, orc, W, a, cal, ws=poisoned_ws(ops))


def test_w4a4_streamk_reuse_and_deterministic(ops, orc):
    # one workspace across calls of different shapes: repeated calls give the
    # same bits, and the stream-K result matches the workspace-free one to
    # fp32 rounding
    import torch

    ws = ops.w4a4_workspace()
    W = synth.normal_bf16(72, 1000, 2048)
    q = Quantized(ops, orc, W)
    g = f32_dev(400.0)
    al = ops.alpha(q.g_dev, g)
    for M in (300, 1024, 5, 300):
        a = bf16_dev(synth.normal_bf16(73 + M, M, 2048))
        ac, as_ = ops.quantize_act(a, g)
        o1 = bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=poisoned_ws(ops, ws)))
        check_ws_clean(ops, ws)
        o2 = bf16_host(ops.linear_w4a4(ac, as_, q.w, al, workspace=poisoned_ws(ops, ws)))
        if not (o1 == o2).all():
            f1, f2 = bf16_f64(o1), bf16_f64(o2)
            diff = np.nonzero(o1 != o2)
            raise AssertionError(
                f"M={M}: {len(diff[0])} outputs differ between two calls (rows {np.unique(diff[0])[:8]}, "
                f"cols {np.unique(diff[1])[:8]}); non-finite: first {int((~np.isfinite(f1)).sum())}, "
                f"second {int((~np.isfinite(f2)).sum())}; workspace tail after the second: "
                f"{int(np.count_nonzero(ws[-(4 * torch.cuda.get_device_properties(0).multi_processor_count + 4):].cpu().numpy()))} "
                f"nonzero bytes")
        ref = bf16_f64(bf16_host(ops.linear_w4a4(ac, as_, q.w, al)))
        got = bf16_f64(o1)
        assert np.linalg.norm(got - ref) <= 1e-3 * np.linalg.norm(ref)


# ------------------------------------------------------------------ dispatch

def test_dispatch_routes_and_numerics(ops, orc):
    # Large fused-weight shape scaled down in N (the routes do not depend on N).
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
