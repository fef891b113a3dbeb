"""HIP-graph capture of the compute calls: every replay must give the eager
result bit for bit (all three paths have a fixed summation order), with eager
work and host synchronizations between the replays.  The MoE layer clears its
h amax inside a kernel, not with a memset, so it is capturable too.
"""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_host, f32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


def _weight(ops, seed, N, K):
    wd = bf16_dev(synth.normal_bf16(seed, N, K))
    g = ops.global_scale(wd)
    c, s = ops.quantize_act(wd, g)
    return ops.prepare_weight(c, s), g


def _capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the code paths before capture
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(torch, g, out, eager_bits, noise, n=4):
    for i in range(n):
        out.zero_()
        noise()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (bf16_host(out) == eager_bits).all(), f"replay {i} differs from the eager result"


def test_graph_w4a16(ops):
    import torch

    w, g = _weight(ops, 301, 1000, 4352)
    a = bf16_dev(synth.normal_bf16(302, 7, 4352))
    al = ops.alpha(g)
    eager = bf16_host(ops.linear_w4a16(a, w, al))
    out = torch.empty((7, 1000), dtype=torch.bfloat16, device="cuda")
    gr = _capture(torch, lambda: ops.linear_w4a16(a, w, al, out=out))
    _replays_match(torch, gr, out, eager, lambda: torch.randn(1 << 20, device="cuda").sum())


def test_graph_w4a4(ops):
    import torch

    # 32 tiles of 256 x 256 (fewer than one per CU), then 9 x 34 = 306 tiles:
    # a whole round on 256 CUs and 50 leftover tiles run as 128-row halves
    for N, K, M, seed in ((2048, 2048, 1024, 303), (2304, 1024, 8704, 309)):
        w, gw = _weight(ops, seed, N, K)
        ga = f32_dev(500.0)
        ac, as_ = ops.quantize_act(bf16_dev(synth.normal_bf16(seed + 1, M, K)), ga)
        al = ops.alpha(gw, ga)
        eager = bf16_host(ops.linear_w4a4(ac, as_, w, al))
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        gr = _capture(torch, lambda: ops.linear_w4a4(ac, as_, w, al, out=out))
        _replays_match(torch, gr, out, eager, lambda: ops.linear_w4a4(ac, as_, w, al))


def test_graph_w4a4_split_k(ops):
    import torch

    # few tiles: K split across workgroups, two launches per call (partial
    # tiles, then their fixed-order sum).  Captured with a caller workspace,
    # through the dispatched linear, and through the allocation-free form,
    # whose scratch eager calls on other inputs overwrite between replays
    M, N, K = 100, 3000, 2048
    assert ops.linear_w4a4_workspace_bytes(M, N, K) > 0
    w, gw = _weight(ops, 311, N, K)
    ga = f32_dev(500.0)
    a = bf16_dev(synth.normal_bf16(312, M, K))
    other = bf16_dev(synth.normal_bf16(313, M, K))
    ac, as_ = ops.quantize_act(a, ga)
    al, a16 = ops.alpha(gw, ga), ops.alpha(gw)
    ws = torch.empty(ops.linear_w4a4_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    eager = bf16_host(ops.linear_w4a4(ac, as_, w, al, workspace=ws))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gr = _capture(torch, lambda: ops.linear_w4a4(ac, as_, w, al, out=out, workspace=ws))
    _replays_match(torch, gr, out, eager, lambda: ops.linear_w4a4(ac, as_, w, al, workspace=True))
    ops.set_route_m_max(64)
    try:
        lws = torch.empty(ops.linear_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        lin, route = ops.linear(a, w, ga, a16, al, workspace=lws)
        assert route == 1 and (bf16_host(lin) == eager).all()
        gr = _capture(torch, lambda: ops.linear(a, w, ga, a16, al, out=out, workspace=lws))
        _replays_match(torch, gr, out, eager, lambda: ops.linear(other, w, ga, a16, al))
        scratch_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        gr = _capture(torch, lambda: ops.linear_noalloc(a, w, ga, a16, al, out))
        _replays_match(torch, gr, out, eager, lambda: ops.linear_noalloc(other, w, ga, a16, al, scratch_out))
    finally:
        ops.set_route_m_max(16)


def test_graph_moe(ops):
    import torch

    E, top_k, K, I, T = 8, 2, 512, 256, 300
    x = bf16_dev(synth.normal_bf16(305, T, K))
    ids, wts = synth.route_top_k(synth.normal_f32(306, T, E), top_k)
    ids, wts = torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()
    banks = []
    for seed, rows, cols in ((307, 2 * I, K), (308, K, I)):
        bank = synth.normal_bf16(seed, E * rows, cols)
        c = torch.empty((E * rows, cols // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((E * rows, cols // 16), dtype=torch.uint8, device="cuda")
        for e in range(E):
            sl = slice(e * rows, (e + 1) * rows)
            part = bf16_dev(bank[sl])
            ops.quantize_act(part, ops.global_scale(part), codes=c[sl], scales=s[sl])
        banks.append(ops.prepare_weight(c, s))
    g1, g2 = f32_dev(300.0), f32_dev(0.5)
    a_gu = torch.full((E,), 1e-4, dtype=torch.float32, device="cuda")
    a_dn = torch.full((E,), 1e-3, dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.moe_workspace_bytes(T, top_k, E, K, I), dtype=torch.uint8, device="cuda")
    hmax = torch.zeros(1, dtype=torch.float32, device="cuda")

    def call(out=None):
        return ops.moe_w4a4(x, ids, wts, banks[0], banks[1], E, g1, g2, a_gu, a_dn, out=out, workspace=ws,
                            h_amax=hmax)

    eager = bf16_host(call())
    eager_amax = hmax.item()
    assert np.isfinite(eager_amax) and eager_amax > 0
    out = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    gr = _capture(torch, lambda: call(out))
    _replays_match(torch, gr, out, eager, lambda: call())
    assert hmax.item() == eager_amax  # cleared and recomputed on every call
