"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-side validation returns the documented status
before any launch (no call here reaches a kernel)."""
import ctypes as C
import subprocess

import pytest

from nvfp4_block_scaled_act_amd import lib as L

OK, ARG, SHAPE, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5
A16 = 0x10000  # a fake, 16-byte aligned device address: never dereferenced here


@pytest.fixture(scope="module")
def nv():
    return L.load()


def test_exports_every_declared_function(nv):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    declared = L.header_functions()
    assert declared, "no declarations parsed"
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(nv, f)


def test_built_from_this_tree(nv, monkeypatch):
    # the library embeds the hash of the sources it was built from, and the
    # loader refuses one whose hash is not the tree's
    from nvfp4_block_scaled_act_amd import build as B

    assert nv.nvfp4_build_source_hash().decode() == B.source_hash()
    monkeypatch.setattr(B, "source_hash", lambda: "0" * 16)
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="other sources"):
        L.load()
    monkeypatch.undo()
    assert L.load() is not None


def test_status_strings(nv):
    for code in range(7):
        assert nv.nvfp4_status_str(code)
    assert nv.nvfp4_version() >= 100


def _w(N=64, K=256, data=A16, layout=L.LAYOUT_TILED):
    w = L.Weight()
    w.data, w.N, w.K, w.layout, w.reserved = data, N, K, layout, 0
    return w


def test_quantize_validation(nv):
    q = nv.nvfp4_quantize_act
    assert q(A16, 4, 24, 24, A16, A16, A16, None) == SHAPE          # K % 16
    assert q(A16, 4, 32, 16, A16, A16, A16, None) == SHAPE          # lda < K
    assert q(None, 4, 32, 32, A16, A16, A16, None) == ARG
    assert q(A16, 4, 32, 32, None, A16, A16, None) == ARG
    assert q(A16 + 2, 4, 32, 32, A16, A16, A16, None) == ALIGN      # a not 16-byte aligned
    assert q(A16, 4, 32, 36, A16, A16, A16, None) == ALIGN          # lda % 8
    assert q(A16, 4, 32, 32, A16, A16 + 8, A16, None) == ALIGN      # codes
    assert q(A16, -1, 32, 32, A16, A16, A16, None) == SHAPE
    assert q(A16, 0, 32, 32, A16, A16, A16, None) == OK             # empty: no launch
    assert q(None, 0, 32, 32, None, None, None, None) == OK         # empty: null buffers allowed


def test_prepare_weight_validation(nv):
    d = L.Weight()
    # ceil(N/16) tiles x K/256 steps x 2304 bytes
    assert nv.nvfp4_prepared_weight_bytes(128, 256) == 8 * 2304
    assert nv.nvfp4_prepared_weight_bytes(100, 512) == 7 * 2 * 2304
    assert nv.nvfp4_prepared_weight_bytes(62080, 5120) == 62080 * 5120 * 9 // 16
    assert nv.nvfp4_prepared_weight_bytes(128, 24) == 0      # invalid shape
    need = nv.nvfp4_prepared_weight_bytes(128, 256)
    p = nv.nvfp4_prepare_weight
    assert p(A16, A16, 128, 24, A16, need, C.byref(d), None) == SHAPE
    assert p(A16, A16, 128, 128, A16, need, C.byref(d), None) == UNSUP   # K % 256
    assert p(A16, A16, 128, 256, A16, need - 1, C.byref(d), None) == WS  # dst too small
    assert p(A16, A16, 128, 256, None, need, C.byref(d), None) == ARG    # no dst
    assert p(None, A16, 128, 256, A16, need, C.byref(d), None) == ARG
    assert p(A16, A16, 128, 256, A16 + 8, need, C.byref(d), None) == ALIGN  # dst not 16-byte aligned
    assert p(A16 + 4, A16, 128, 256, A16, need, C.byref(d), None) == ALIGN  # codes not 8-byte aligned
    assert p(A16, A16, -1, 256, A16, need, C.byref(d), None) == SHAPE
    assert p(A16, A16, 128, 256, A16, need, None, None) == ARG
    # N = 0: nothing to re-tile, a valid empty descriptor
    assert p(None, None, 0, 256, None, 0, C.byref(d), None) == OK
    assert (d.N, d.K, d.layout) == (0, 256, L.LAYOUT_TILED)


def test_w4a16_validation(nv):
    f = nv.nvfp4_linear_w4a16
    w = _w()
    assert f(A16, 65, 256, C.byref(w), A16, A16, 64, None) == UNSUP    # M > 64
    assert f(A16, 16, 1 << 27, C.byref(w), A16, A16, 64, None) == UNSUP  # offsets past 2^31 bytes
    assert f(A16, 4, 256, C.byref(w), None, A16, 64, None) == ARG      # alpha
    assert f(A16, 4, 256, C.byref(w), A16, A16, 63, None) == SHAPE     # ldo < N
    assert f(A16, 4, 255, C.byref(w), A16, A16, 64, None) == SHAPE     # lda < K
    assert f(A16, 4, 260, C.byref(w), A16, A16, 64, None) == ALIGN     # lda % 8
    assert f(A16, 4, 256, C.byref(w), A16, A16 + 1, 64, None) == ALIGN  # odd output address
    assert f(A16, 4, 256, None, A16, A16, 64, None) == ARG
    assert f(A16, -2, 256, C.byref(w), A16, A16, 64, None) == ARG
    assert f(A16, 0, 256, C.byref(w), A16, A16, 64, None) == OK        # empty
    assert f(None, 0, 256, C.byref(w), A16, None, 64, None) == OK      # empty, null buffers
    wz = _w(N=0)
    assert f(A16, 4, 256, C.byref(wz), A16, A16, 1, None) == OK         # N = 0
    g = nv.nvfp4_linear_w4a16_ex
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 5, 1, 1, 0, None) == ARG    # schedule 5
    assert g(A16, 5, 256, C.byref(w), A16, A16, 64, 4, 1, 0, 0, None) == ARG    # dot: M > 4
    assert g(A16, 2, 256, C.byref(w), A16, A16, 64, 4, 0, 0, 0, None) == ARG    # dot: ksplit 0
    assert g(A16, 2, 256, C.byref(w), A16, A16, 64, 4, 17, 0, 0, None) == ARG   # dot: ksplit 17
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 1, 0, 0, 0, None) == ARG    # split: ksplit 0
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 1, 17, 0, 0, None) == ARG   # split: ksplit 17
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 2, 0, 0, 0, None) == ARG    # shared: chunk 0
    wl = _w(N=64, K=256 * 8)
    assert g(A16, 16, 256 * 8, C.byref(wl), A16, A16, 64, 2, 0, 5, 0, None) == ARG  # 16 x 5 > 64
    assert g(A16, 0, 256, C.byref(w), A16, A16, 64, 2, 0, 5, 0, None) == OK     # empty
    assert g(A16, 4, 256 * 8, C.byref(wl), A16, A16, 64, 3, 0, 0, 0, None) == ARG   # burst: ksplit 0
    wk = _w(N=64, K=256 * 20)
    assert g(A16, 4, 256 * 20, C.byref(wk), A16, A16, 64, 3, 2, 0, 0, None) == ARG  # burst: 10 steps per wave > 8
    assert g(A16, 4, 256 * 20, C.byref(wk), A16, A16, 64, 3, 4, 4, 0, None) == ARG  # 4 tiles per workgroup
    assert g(A16, 4, 256 * 20, C.byref(wk), A16, A16, 64, 3, 2, 3, 0, None) == ARG  # 2-3 tiles: 10 steps per wave
    w2 = _w(N=64, K=256 * 2)
    assert g(A16, 4, 256 * 2, C.byref(w2), A16, A16, 64, 3, 4, 3, 0, None) == ARG  # 2-3 tiles on 2 waves (< 3)
    assert g(A16, 4, 256 * 20, C.byref(wk), A16, A16, 64, 3, 10, 2, 0, None) == ARG  # two tiles: 10 waves > 8
    assert g(A16, 1, 256 * 20, C.byref(wk), A16, A16, 64, 4, 2, 0, 0, None) == ARG  # dot: 10 steps per wave > 8
    assert g(A16, 1, 256, C.byref(w), A16, A16, 64, 4, 1, 0, 3, None) == ARG     # cache policy 3
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 3, 1, 0, 1, None) == ARG     # cache policy off the dot schedule
    assert g(A16, 4, 256, C.byref(w), A16, A16, 64, 0, 0, 0, 2, None) == ARG     # ... or with the default


def test_w4a4_validation(nv):
    f = nv.nvfp4_linear_w4a4
    w = _w()
    assert f(None, A16, 8, C.byref(w), A16, A16, 64, None) == ARG
    assert f(A16, A16 + 4, 8, C.byref(w), A16, A16, 64, None) == ALIGN
    assert f(A16, A16, 8, C.byref(w), A16, A16, 10, None) == SHAPE
    assert f(A16, A16, 0, C.byref(w), A16, A16, 64, None) == OK
    assert f(None, None, 0, C.byref(w), A16, None, 64, None) == OK
    wbad = _w(K=512 + 16)
    assert f(A16, A16, 8, C.byref(wbad), A16, A16, 64, None) == UNSUP
    wlay = _w(layout=0)
    assert f(A16, A16, 8, C.byref(wlay), A16, A16, 64, None) == UNSUP   # not a prepared weight
    wmis = _w(data=A16 + 8)
    assert f(A16, A16, 8, C.byref(wmis), A16, A16, 64, None) == ALIGN
    # K above 2^24: the kernels' 32-bit offsets into a workgroup's weight tiles
    wbig = _w(K=(1 << 24) + 256)
    assert f(A16, A16, 8, C.byref(wbig), A16, A16, 64, None) == UNSUP
    nv.nvfp4_set_route_m_max(16)
    r = C.c_int(-1)
    assert nv.nvfp4_linear(A16, 32, (1 << 24) + 256, C.byref(wbig), A16, A16, A16, A16, 64, A16, 1 << 30,
                           C.byref(r), None) == UNSUP


def test_route_default_threshold():
    # a fresh process sees the documented default M* = 16 (the measured
    # crossover on the large fused weight)
    import sys

    code = "from nvfp4_block_scaled_act_amd import lib; print(lib.load().nvfp4_get_route_m_max())"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=L.HERE + "/..").stdout
    assert out.strip() == "16"


def test_route_is_a_pure_threshold(nv):
    nv.nvfp4_set_route_m_max(16)
    assert nv.nvfp4_get_route_m_max() == 16
    for M in range(0, 40):
        for has_g in (0, 1):
            want = 1 if (has_g and M > 16) else 0
            assert nv.nvfp4_route(M, 8704, 5120, has_g) == want
    nv.nvfp4_set_route_m_max(4)
    assert nv.nvfp4_route(5, 1, 256, 1) == 1 and nv.nvfp4_route(4, 1, 256, 1) == 0
    nv.nvfp4_set_route_m_max(100)          # clamped to the W4A16 kernels' limit
    assert nv.nvfp4_get_route_m_max() == 64
    nv.nvfp4_set_route_m_max(-3)
    assert nv.nvfp4_get_route_m_max() == 0
    nv.nvfp4_set_route_m_max(16)


def test_linear_dispatch_validation(nv):
    f = nv.nvfp4_linear
    w = _w()
    r = C.c_int(-1)
    nv.nvfp4_set_route_m_max(16)
    # W4A4 route without workspace
    assert f(A16, 32, 256, C.byref(w), A16, A16, A16, A16, 64, None, 0, C.byref(r), None) == WS
    need = nv.nvfp4_linear_workspace_bytes(32, 64, 256)
    assert need >= 32 * 128 + 32 * 16
    assert f(A16, 32, 256, C.byref(w), A16, A16, A16, A16, 64, A16, need - 1, C.byref(r), None) == WS
    # W4A16 route beyond its limit (64) when no activation global is given
    assert f(A16, 65, 256, C.byref(w), None, A16, None, A16, 64, None, 0, C.byref(r), None) == UNSUP
    # W4A4 route needs alpha_w4a4
    assert f(A16, 32, 256, C.byref(w), A16, A16, None, A16, 64, A16, need, C.byref(r), None) == ARG
    # empty batch, either route
    r.value = -1
    assert f(A16, 0, 256, C.byref(w), None, A16, None, A16, 64, None, 0, C.byref(r), None) == OK
    assert r.value == 0


def test_linear_noalloc_validation(nv):
    # the allocation-free dispatch validates as nvfp4_linear and rejects, before
    # touching the device, a W4A4 call whose quantized activations would not
    # fit its fixed scratch (64 MiB)
    f = nv.nvfp4_linear_noalloc
    w = _w(N=64, K=2048)
    r = C.c_int(-1)
    nv.nvfp4_set_route_m_max(16)
    assert nv.nvfp4_linear_workspace_bytes(60000, 64, 2048) > (64 << 20)
    assert f(A16, 60000, 2048, C.byref(w), A16, A16, A16, A16, 64, C.byref(r), None) == WS
    assert f(A16, 32, 2048, C.byref(w), A16, A16, None, A16, 64, C.byref(r), None) == ARG    # no alpha_w4a4
    assert f(A16, 65, 2048, C.byref(w), None, A16, None, A16, 64, C.byref(r), None) == UNSUP  # W4A16 beyond 64
    assert f(A16 + 2, 32, 2048, C.byref(w), A16, A16, A16, A16, 64, C.byref(r), None) == ALIGN
    assert f(A16, 32, 2048, C.byref(w), A16, A16, A16, A16, 10, C.byref(r), None) == SHAPE  # ldo < N
    r.value = -1
    assert f(None, 0, 2048, C.byref(w), A16, A16, A16, None, 64, C.byref(r), None) == OK   # empty batch
    assert r.value == 0  # M = 0 <= M*: the W4A16 route, no launch


def test_moe_workspace_layout(nv):
    T, top_k, E, K, I = 8192, 8, 128, 2048, 768
    lay = L.MoeLayout()
    assert nv.nvfp4_moe_workspace_layout(T, top_k, E, K, I, C.byref(lay)) == OK
    P = T * top_k
    parts = [("x_codes", T * K // 2), ("x_scales", T * K // 16), ("counts", 4 * 64 * E), ("offsets", 4 * (E + 1)),
             ("tiles", 16 * lay.max_tiles), ("sorted", 4 * P), ("h_codes", P * I // 2), ("h_scales", P * I // 16),
             ("inv", 4 * P), ("ys", 4 * P * K)]
    assert lay.max_tiles == P // 256 + E
    end = 0
    for name, size in parts:
        off = getattr(lay, name)
        assert off % 256 == 0 and off >= end, name
        end = off + size
    assert lay.total_bytes >= end
    assert nv.nvfp4_moe_workspace_bytes(T, top_k, E, K, I) == lay.total_bytes
    # invalid shapes report 0 bytes / an error
    assert nv.nvfp4_moe_workspace_bytes(T, top_k, E, K, 100) == 0
    assert nv.nvfp4_moe_workspace_layout(T, top_k, E, K, 128, C.byref(lay)) == UNSUP   # I % 256
    assert nv.nvfp4_moe_workspace_layout(T, 0, E, K, I, C.byref(lay)) == ARG          # top_k
    assert nv.nvfp4_moe_workspace_layout(T, top_k, 1025, K, I, C.byref(lay)) == ARG   # E > 1024
    assert nv.nvfp4_moe_workspace_layout(T, top_k, E, K, I, None) == ARG


def test_moe_validation(nv):
    T, top_k, E, K, I = 64, 2, 4, 512, 256
    gu, dn = _w(N=E * 2 * I, K=K), _w(N=E * K, K=I)
    need = nv.nvfp4_moe_workspace_bytes(T, top_k, E, K, I)
    WS0 = 0x100000  # 256-byte aligned fake address

    def call(x=A16, T=T, ldx=K, ids=A16, w=A16, top_k=top_k, E=E, I=I, gu=gu, dn=dn, g1=A16, g2=A16, agu=A16,
             adn=A16, out=A16, ldo=K, ws=WS0, ws_bytes=need, h_amax=None):
        return nv.nvfp4_moe_w4a4(x, T, ldx, ids, w, top_k, E, I, C.byref(gu) if gu is not None else None,
                                 C.byref(dn) if dn is not None else None, g1, g2, agu, adn, out, ldo, ws, ws_bytes,
                                 h_amax, None)

    assert call(gu=None) == ARG
    assert call(g2=None) == ARG
    assert call(ids=None) == ARG
    assert call(top_k=0) == ARG
    assert call(E=2000) == ARG
    assert call(dn=_w(N=E * K, K=512)) == SHAPE          # down K != I
    assert call(gu=_w(N=E * 2 * I - 16, K=K)) == SHAPE   # gate_up N != E*2I
    assert call(I=128, gu=_w(N=E * 256, K=K), dn=_w(N=E * K, K=128)) == UNSUP  # I % 256
    assert call(ldx=K - 8) == SHAPE
    assert call(ldo=K + 4) == ALIGN
    assert call(out=A16 + 2) == ALIGN
    assert call(ws=WS0 + 16) == ALIGN
    assert call(ws_bytes=need - 1) == WS
    assert call(ws=None) == WS
    assert call(x=None, T=0, ids=None, w=None, out=None, ws=None, ws_bytes=0) == OK   # empty batch
    # an expert's gate_up past 2^32 bytes (the grouped GEMMs' 32-bit weight offsets)
    big = 1 << 20
    lay = L.MoeLayout()
    assert nv.nvfp4_moe_workspace_layout(1, 1, 1, big, big, C.byref(lay)) == UNSUP
    assert nv.nvfp4_moe_w4a4(A16, 1, big, A16, A16, 1, 1, big, C.byref(_w(N=2 * big, K=big)),
                             C.byref(_w(N=big, K=big)), A16, A16, A16, A16, A16, big, WS0, 1 << 40, None,
                             None) == UNSUP


def test_stream_read_validation(nv):
    f = nv.nvfp4_stream_read
    assert f(None, 0, None, None) == OK              # nothing to read
    assert f(None, 16, A16, None) == ARG             # null source
    assert f(A16, 16, None, None) == ARG             # null sink
    assert f(A16, 24, A16, None) == SHAPE            # bytes % 16
    assert f(A16 + 8, 16, A16, None) == ALIGN        # source alignment
    assert f(A16, 16, A16 + 2, None) == ALIGN        # sink alignment



def test_moe_w4a16_workspace_and_validation(nv):
    T, top_k, E, K, I = 16, 8, 128, 2048, 768
    lay = L.MoeW4A16Layout()
    assert nv.nvfp4_moe_w4a16_workspace_layout(T, top_k, E, K, I, C.byref(lay)) == OK
    P = T * top_k
    assert lay.max_tiles == P // 16 + E
    end = 0
    for name, size in [("counts", 4 * E), ("offsets", 4 * (E + 1)), ("tiles", 16 * lay.max_tiles),
                       ("sorted", 4 * P), ("h", 2 * P * I), ("inv", 4 * P), ("ys", 4 * P * K)]:
        off = getattr(lay, name)
        assert off % 256 == 0 and off >= end, name
        end = off + size
    assert lay.total_bytes >= end and nv.nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, K, I) == lay.total_bytes
    assert nv.nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, 64 * 256 + 256, I) == 0   # K beyond 64 steps
    assert nv.nvfp4_moe_w4a16_workspace_layout(T, top_k, E, K, 128, C.byref(lay)) == UNSUP   # I % 256

    T, top_k, E, K, I = 4, 2, 4, 512, 256
    gu, dn = _w(N=E * 2 * I, K=K), _w(N=E * K, K=I)
    need = nv.nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, K, I)
    WS0 = 0x100000

    def call(x=A16, T=T, ldx=K, ids=A16, w=A16, top_k=top_k, E=E, I=I, gu=gu, dn=dn, agu=A16, adn=A16, out=A16,
             ldo=K, ws=WS0, ws_bytes=need):
        return nv.nvfp4_moe_w4a16(x, T, ldx, ids, w, top_k, E, I, C.byref(gu) if gu is not None else None,
                                  C.byref(dn) if dn is not None else None, agu, adn, out, ldo, ws, ws_bytes, None)

    assert call(gu=None) == ARG
    assert call(agu=None) == ARG
    assert call(ids=None) == ARG
    assert call(top_k=0) == ARG
    assert call(dn=_w(N=E * K, K=512)) == SHAPE
    assert call(gu=_w(N=E * 2 * I - 16, K=K)) == SHAPE
    assert call(ldx=K - 8) == SHAPE
    assert call(ldx=1 << 29) == UNSUP                # x's rows past 2^31 bytes
    assert call(ldo=K + 4) == ALIGN
    assert call(ws=WS0 + 16) == ALIGN
    assert call(ws_bytes=need - 1) == WS
    assert call(ws=None) == WS
    assert call(T=0, x=None, ids=None, w=None, out=None, ws=None, ws_bytes=0) == OK


def test_moe_route_and_dispatch_validation(nv):
    assert nv.nvfp4_get_moe_route_tokens_per_expert() == 14
    assert nv.nvfp4_moe_route(100000, 8, 128, 0) == 0   # no static globals: W4A16 only
    assert nv.nvfp4_moe_route(224, 8, 128, 1) == 0      # 14 tokens per expert
    assert nv.nvfp4_moe_route(225, 8, 128, 1) == 1
    try:
        nv.nvfp4_set_moe_route_tokens_per_expert(4)
        assert nv.nvfp4_moe_route(64, 8, 128, 1) == 0 and nv.nvfp4_moe_route(65, 8, 128, 1) == 1
        nv.nvfp4_set_moe_route_tokens_per_expert(-5)
        assert nv.nvfp4_get_moe_route_tokens_per_expert() == 0
        assert nv.nvfp4_moe_route(1, 1, 128, 1) == 1 and nv.nvfp4_moe_route(0, 8, 128, 1) == 0
    finally:
        nv.nvfp4_set_moe_route_tokens_per_expert(14)
    for T, g in ((16, 1), (16, 0), (8192, 1)):
        want = (nv.nvfp4_moe_workspace_bytes if nv.nvfp4_moe_route(T, 8, 128, g) else
                nv.nvfp4_moe_w4a16_workspace_bytes)(T, 8, 128, 2048, 768)
        assert nv.nvfp4_moe_dispatch_workspace_bytes(T, 8, 128, 2048, 768, g) == want > 0
    E, K, I = 4, 512, 256
    gu, dn = _w(N=E * 2 * I, K=K), _w(N=E * K, K=I)
    route = C.c_int32(-1)
    # one static global without the other
    assert nv.nvfp4_moe(A16, 4, K, A16, A16, 2, E, I, C.byref(gu), C.byref(dn), A16, None, A16, A16, A16, A16,
                        A16, K, 0x100000, 1 << 30, C.byref(route), None) == ARG
    # the W4A16 route needs its alphas
    assert nv.nvfp4_moe(A16, 4, K, A16, A16, 2, E, I, C.byref(gu), C.byref(dn), None, None, None, None, None, A16,
                        A16, K, 0x100000, 1 << 30, C.byref(route), None) == ARG
    assert route.value == 0


def test_gated_mlp_validation(nv):
    M, K, I = 64, 512, 256
    gu = _w(N=2 * I, K=K)
    f = nv.nvfp4_gated_mlp_w4a4
    assert f(A16, A16, M, C.byref(gu), None, A16, A16, A16, None, None) == ARG        # alpha
    assert f(A16, A16, M, C.byref(gu), A16, None, A16, A16, None, None) == ARG        # g2
    assert f(A16, A16, M, C.byref(_w(N=2 * I + 16, K=K)), A16, A16, A16, A16, None, None) == SHAPE  # odd N
    assert f(A16, A16, M, C.byref(_w(N=2 * 128, K=K)), A16, A16, A16, A16, None, None) == UNSUP   # I % 256
    assert f(A16, A16, M, C.byref(gu), A16, A16, A16 + 8, A16, None, None) == ALIGN   # h codes
    assert f(A16, A16, M, C.byref(gu), A16, A16, None, A16, None, None) == ARG
    assert f(None, None, 0, C.byref(gu), A16, A16, None, None, None, None) == OK        # empty batch
    # gate_up past 2^32 bytes (the kernel's 32-bit weight offsets)
    assert f(A16, A16, M, C.byref(_w(N=1 << 17, K=1 << 16)), A16, A16, A16, A16, None, None) == UNSUP


def test_swizzled_scales_validation(nv):
    # roundup(rows, 128) x roundup(K/16, 4) bytes
    assert nv.nvfp4_swizzled_scales_bytes(300, 272) == 384 * 20
    assert nv.nvfp4_swizzled_scales_bytes(128, 256) == 128 * 16
    assert nv.nvfp4_swizzled_scales_bytes(0, 256) == 0
    assert nv.nvfp4_swizzled_scales_bytes(128, 24) == 0      # K % 16
    q = nv.nvfp4_quantize_act_swizzled
    need = nv.nvfp4_swizzled_scales_bytes(300, 272)
    assert q(A16, 300, 272, 272, A16, A16, A16, need - 1, None) == WS
    assert q(A16, 300, 24, 24, A16, A16, A16, need, None) == SHAPE
    assert q(A16, 300, 272, 272, None, A16, A16, need, None) == ARG
    assert q(A16, 300, 272, 272, A16, A16 + 8, A16, need, None) == ALIGN
    assert q(None, 0, 272, 272, A16, None, None, 0, None) == OK         # empty batch
    d = L.Weight()
    p = nv.nvfp4_prepare_weight_swizzled
    wneed = nv.nvfp4_prepared_weight_bytes(128, 256)
    sneed = nv.nvfp4_swizzled_scales_bytes(128, 256)
    assert p(A16, A16, sneed - 1, 128, 256, A16, wneed, C.byref(d), None) == WS
    assert p(A16, A16, sneed, 128, 256, A16, wneed - 1, C.byref(d), None) == WS
    assert p(A16, A16, sneed, 128, 24, A16, wneed, C.byref(d), None) == SHAPE
    assert p(A16, A16, sneed, 128, 256, A16, wneed, None, None) == ARG


def test_fused_weight_global(nv):
    # the largest per-part global; a warning when the parts differ by more than 5 %
    f = nv.nvfp4_fused_weight_global

    def call(gs):
        arr = (C.c_float * len(gs))(*gs)
        g, w = C.c_float(0.0), C.c_int32(-1)
        st = f(C.cast(arr, C.c_void_p), len(gs), C.cast(C.byref(g), C.c_void_p), C.cast(C.byref(w), C.c_void_p))
        return st, g.value, w.value

    st, g, w = call([400.0, 410.0, 405.0])
    assert (st, g, w) == (OK, 410.0, 0)
    st, g, w = call([400.0, 430.0])       # 7.5 % apart
    assert (st, g, w) == (OK, 430.0, 1)
    st, g, w = call([400.0, 419.0])       # 4.75 % apart
    assert (st, g, w) == (OK, 419.0, 0)
    assert call([512.0])[:3] == (OK, 512.0, 0)
    assert call([400.0, 0.0])[0] == ARG
    assert call([400.0, float("inf")])[0] == ARG
    assert call([400.0, float("nan")])[0] == ARG
    g = C.c_float(0.0)
    assert f(None, 1, C.cast(C.byref(g), C.c_void_p), None) == ARG
    arr = (C.c_float * 1)(1.0)
    assert f(C.cast(arr, C.c_void_p), 0, C.cast(C.byref(g), C.c_void_p), None) == ARG


def test_fused_weight_global_binding_warns():
    import warnings

    from nvfp4_block_scaled_act_amd import ops

    with warnings.catch_warnings(record=True) as rec:
        warnings.simplefilter("always")
        assert ops.fused_weight_global([300.0, 330.0]) == (330.0, True)
        assert ops.fused_weight_global([300.0, 301.0]) == (301.0, False)
    assert len(rec) == 1 and "5 %" in str(rec[0].message)


def test_moe_w4a16_direct_pairs_constant():
    # the binding's copy of the direct-path threshold matches the header
    import os
    import re

    hdr = open(os.path.join(os.path.dirname(L.__file__), "..", "include", "nvfp4.h")).read()
    m = re.search(r"#define NVFP4_MOE_W4A16_DIRECT_PAIRS (\d+)", hdr)
    from nvfp4_block_scaled_act_amd import ops

    assert m and int(m.group(1)) == ops.MOE_W4A16_DIRECT_PAIRS
