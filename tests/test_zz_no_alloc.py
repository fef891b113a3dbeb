"""The allocation-free dispatched linear (nvfp4_linear_noalloc) against
nvfp4_linear with a caller workspace: the same kernels, so the same bits and
the same route, on consecutive calls that reuse the library's scratch (the
second W4A4 call smaller than the first), and within the linears' bar of the
oracle.  Collected last: its calls share the per-GPU scratch, which keeps the
previous call's contents."""
import numpy as np
import pytest

from nvfp4_block_scaled_act_amd import synth

from helpers import bf16_dev, bf16_host, gemm_check, u8_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from nvfp4_block_scaled_act_amd import ops as O

    return O


def test_noalloc_matches_workspace_call(ops, orc):
    import torch

    N, K = 1000, 2048
    W = synth.normal_bf16(901, N, K)
    a = synth.normal_bf16(902, 1024, K)
    cal = synth.normal_bf16(903, 128, K)
    g_w, g_a = orc.global_scale(W), orc.global_scale(cal)
    wd = bf16_dev(W)
    gwd, gad = ops.global_scale(wd), ops.global_scale(bf16_dev(cal))
    c, s = ops.quantize_act(wd, gwd)
    oc, os_ = orc.quantize(W, g_w)
    assert (u8_host(c) == oc).all() and (u8_host(s) == os_).all()
    w = ops.prepare_weight(c, s)
    a16, a4 = ops.alpha(gwd), ops.alpha(gwd, gad)
    ad = bf16_dev(a)
    ops.set_route_m_max(16)
    # W4A4 at M = 1024, then a smaller W4A4 call (M = 300) on the scratch the
    # first one filled, then the W4A16 route, then W4A4 again
    for M in (1024, 300, 8, 700):
        out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        route = ops.linear_noalloc(ad[:M], w, gad, a16, a4, out)
        want, want_route = ops.linear(ad[:M], w, gad, a16, a4)
        assert route == want_route == (1 if M > 16 else 0)
        got = bf16_host(out)
        assert (got == bf16_host(want)).all(), f"M={M}: outputs differ from the workspace call"
        if M == 1024:
            oac, oas = orc.quantize(a[:M], g_a)
            ref, _, sabs = orc.linear_w4a4(oac, oas, oc, os_, orc.alpha(g_w, g_a))
            gemm_check(got, ref, sabs)
        if M == 8:
            ref, _, sabs = orc.linear_w4a16(a[:M], oc, os_, orc.alpha(g_w))
            gemm_check(got, ref, sabs)


def test_noalloc_rejects_beyond_scratch(ops):
    import torch

    # K = 2048 needs 1152 bytes per row: 60000 rows exceed the 64 MiB scratch
    N, K, M = 64, 2048, 60000
    assert ops.linear_workspace_bytes(M, N, K) > ops.NOALLOC_MAX_WORKSPACE_BYTES
    c = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    w = ops.prepare_weight(c, s)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        ops.linear_noalloc(a, w, one, one, one, out)
    torch.cuda.synchronize()
    assert (out == 3.0).all(), "a rejected call must not write the output"
