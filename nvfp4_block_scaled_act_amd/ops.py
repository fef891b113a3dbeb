"""PyTorch-facing wrappers of the C ABI: argument marshalling only.

Tensors live on the current HIP device; every call launches on torch's current
stream.  All arithmetic happens in the gfx950 kernels of libnvfp4.so.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import lib as _L


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0)


def _scalar(t: torch.Tensor, name: str) -> None:
    _need(t, torch.float32, name)
    if t.numel() < 1:
        raise ValueError(f"{name} must hold one fp32 value")


@dataclass
class Weight:
    """A prepared NVFP4 weight: the tiled device buffer and its descriptor."""
    data: torch.Tensor
    desc: _L.Weight

    @property
    def N(self) -> int:
        return int(self.desc.N)

    @property
    def K(self) -> int:
        return int(self.desc.K)


def global_scale(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    _need(x, torch.bfloat16, "x")
    ld = _rows(x, "x")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    _L.check("nvfp4_global_scale",
             _L.load().nvfp4_global_scale(_ptr(x), x.shape[0], x.shape[1], ld, _ptr(out), _stream()))
    return out


def alpha(g_w: torch.Tensor, g_a: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    _scalar(g_w, "g_w")
    if g_a is not None:
        _scalar(g_a, "g_a")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=g_w.device)
    _L.check("nvfp4_alpha", _L.load().nvfp4_alpha(_ptr(g_w), _ptr(g_a), _ptr(out), _stream()))
    return out


def quantize_act(a: torch.Tensor, g: torch.Tensor, codes: torch.Tensor | None = None,
                 scales: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    _need(a, torch.bfloat16, "a")
    _scalar(g, "g")
    lda = _rows(a, "a")
    M, K = a.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=a.device)
    _L.check("nvfp4_quantize_act",
             _L.load().nvfp4_quantize_act(_ptr(a), M, K, lda, _ptr(g), _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def fused_weight_global(g_parts) -> tuple[float, bool]:
    """The global of a fused weight from its parts' globals (host floats):
    the largest one, and whether the parts differ by more than 5 %."""
    import warnings

    arr = (C.c_float * len(g_parts))(*[float(g) for g in g_parts])
    g, warn = C.c_float(0.0), C.c_int32(0)
    _L.check("nvfp4_fused_weight_global",
             _L.load().nvfp4_fused_weight_global(C.cast(arr, C.c_void_p), len(g_parts), C.cast(C.byref(g), C.c_void_p),
                                                 C.cast(C.byref(warn), C.c_void_p)))
    if warn.value:
        warnings.warn("fused NVFP4 weight: the parts' globals differ by more than 5 %% (%s); the largest is used "
                      "with the block scales unchanged" % list(g_parts))
    return g.value, bool(warn.value)


def swizzled_scales_bytes(rows: int, K: int) -> int:
    return int(_L.load().nvfp4_swizzled_scales_bytes(rows, K))


def quantize_act_swizzled(a: torch.Tensor, g: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """quantize_act with the scales in the 128x4-swizzled layout (a flat
    uint8 tensor of swizzled_scales_bytes(M, K) bytes, padding zeroed)."""
    _need(a, torch.bfloat16, "a")
    _scalar(g, "g")
    lda = _rows(a, "a")
    M, K = a.shape
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=a.device)
    nb = swizzled_scales_bytes(M, K)
    scales = torch.empty(max(nb, 1), dtype=torch.uint8, device=a.device)
    _L.check("nvfp4_quantize_act_swizzled",
             _L.load().nvfp4_quantize_act_swizzled(_ptr(a), M, K, lda, _ptr(g), _ptr(codes), _ptr(scales), nb,
                                                   _stream()))
    return codes, scales[:nb]


def prepare_weight_swizzled(codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None) -> Weight:
    """prepare_weight from row-major codes [N, K/2] and 128x4-swizzled
    scales (a flat uint8 tensor of swizzled_scales_bytes(N, K) bytes)."""
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if not codes.is_contiguous() or not scales.is_contiguous():
        raise ValueError("weight codes and scales must be contiguous")
    N, half = codes.shape
    K = 2 * half
    nbytes = prepared_weight_bytes(N, K)
    if out is None:
        out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    _need(out, torch.uint8, "out")
    desc = _L.Weight()
    _L.check("nvfp4_prepare_weight_swizzled",
             _L.load().nvfp4_prepare_weight_swizzled(_ptr(codes), _ptr(scales), scales.numel(), N, K, _ptr(out),
                                                     out.numel(), C.byref(desc), _stream()))
    return Weight(out, desc)


def prepared_weight_bytes(N: int, K: int) -> int:
    return int(_L.load().nvfp4_prepared_weight_bytes(N, K))


def prepare_weight(codes: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None) -> Weight:
    """Re-tile canonical NVFP4 codes [N, K/2] and scales [N, K/16] into the
    layout the linears read (one launch on the current stream)."""
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if not codes.is_contiguous() or not scales.is_contiguous():
        raise ValueError("weight codes and scales must be contiguous")
    N, half = codes.shape
    K = 2 * half
    if tuple(scales.shape) != (N, K // 16):
        raise ValueError(f"scales must be [N, K/16] = [{N}, {K // 16}], got {tuple(scales.shape)}")
    nbytes = prepared_weight_bytes(N, K)
    if out is None:
        out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=codes.device)
    _need(out, torch.uint8, "out")
    desc = _L.Weight()
    _L.check("nvfp4_prepare_weight",
             _L.load().nvfp4_prepare_weight(_ptr(codes), _ptr(scales), N, K, _ptr(out), out.numel(),
                                            C.byref(desc), _stream()))
    return Weight(out, desc)


def _out(out, M, N, device):
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _need(out, torch.bfloat16, "out")
    return out, _rows(out, "out")


def linear_w4a16(a: torch.Tensor, w: Weight, alpha_: torch.Tensor, out: torch.Tensor | None = None,
                 schedule: int = 0, ksplit: int = 0, chunk_steps: int = 0, cache_policy: int = 0) -> torch.Tensor:
    """W4A16 linear; schedule 0 picks the default schedule for (M, N, K)
    (1 = split with ksplit waves per tile, 2 = shared with LDS chunks of
    chunk_steps steps, 3 = split with interleaved steps and chunk_steps (1,
    2, or 3 = two to three) tiles per workgroup, 4 = dot: split on the VALU,
    M <= 4).  cache_policy (dot only): 0 default, 1 weight loads without the
    nontemporal hint, 2 activation loads with it."""
    _need(a, torch.bfloat16, "a")
    _scalar(alpha_, "alpha")
    lda = _rows(a, "a")
    M = a.shape[0]
    if a.shape[1] != w.K:
        raise ValueError("a.shape[1] != K")
    out, ldo = _out(out, M, w.N, a.device)
    _L.check("nvfp4_linear_w4a16_ex",
             _L.load().nvfp4_linear_w4a16_ex(_ptr(a), M, lda, C.byref(w.desc), _ptr(alpha_), _ptr(out), ldo,
                                             schedule, ksplit, chunk_steps, cache_policy, _stream()))
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None) -> None:
    """Measurement aid: read the first nbytes (default: all) of src once, as
    the W4A16 kernels read weights, computing nothing (see nvfp4_stream_read)."""
    if not src.is_cuda or not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("src must be a CUDA tensor and sink a CUDA int32 tensor")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size():
        raise ValueError("nbytes beyond src")
    _L.check("nvfp4_stream_read", _L.load().nvfp4_stream_read(_ptr(src), n, _ptr(sink), _stream()))


def linear_w4a4_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of fp32 split-K partials linear_w4a4 takes with a workspace (0:
    the shape runs one launch over all of K)."""
    return int(_L.load().nvfp4_linear_w4a4_workspace_bytes(M, N, K))


def linear_w4a4(a_codes: torch.Tensor, a_scales: torch.Tensor, w: Weight, alpha_: torch.Tensor,
                out: torch.Tensor | None = None, workspace: torch.Tensor | bool | None = None) -> torch.Tensor:
    """W4A4 linear.  workspace: None -> one launch over K (nvfp4_linear_w4a4);
    a uint8 device tensor, or True to allocate one -> nvfp4_linear_w4a4_ws
    (split-K where the shape takes it)."""
    _need(a_codes, torch.uint8, "a_codes")
    _need(a_scales, torch.uint8, "a_scales")
    _scalar(alpha_, "alpha")
    M = a_codes.shape[0]
    if a_codes.shape[1] * 2 != w.K or tuple(a_scales.shape) != (M, w.K // 16):
        raise ValueError("activation codes/scales do not match the weight's K")
    if not a_codes.is_contiguous() or not a_scales.is_contiguous():
        raise ValueError("activation codes and scales must be contiguous")
    out, ldo = _out(out, M, w.N, a_codes.device)
    if workspace is None:
        _L.check("nvfp4_linear_w4a4",
                 _L.load().nvfp4_linear_w4a4(_ptr(a_codes), _ptr(a_scales), M, C.byref(w.desc), _ptr(alpha_),
                                             _ptr(out), ldo, _stream()))
        return out
    if workspace is True:
        need = linear_w4a4_workspace_bytes(M, w.N, w.K)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a_codes.device)
    _need(workspace, torch.uint8, "workspace")
    _L.check("nvfp4_linear_w4a4_ws",
             _L.load().nvfp4_linear_w4a4_ws(_ptr(a_codes), _ptr(a_scales), M, C.byref(w.desc), _ptr(alpha_),
                                            _ptr(out), ldo, _ptr(workspace), workspace.numel(), _stream()))
    return out


def route(M: int, N: int, K: int, has_act_global: bool) -> int:
    return int(_L.load().nvfp4_route(M, N, K, 1 if has_act_global else 0))


def set_route_m_max(m: int) -> None:
    _L.load().nvfp4_set_route_m_max(int(m))


def get_route_m_max() -> int:
    return int(_L.load().nvfp4_get_route_m_max())


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(_L.load().nvfp4_linear_workspace_bytes(M, N, K))


def linear(a: torch.Tensor, w: Weight, g_act: torch.Tensor | None, alpha_w4a16: torch.Tensor,
           alpha_w4a4: torch.Tensor | None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, int]:
    """Dispatched linear; returns (out, route taken)."""
    _need(a, torch.bfloat16, "a")
    lda = _rows(a, "a")
    M = a.shape[0]
    out, ldo = _out(out, M, w.N, a.device)
    need = linear_workspace_bytes(M, w.N, w.K)
    ws = workspace
    if ws is None and g_act is not None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=a.device)
    ws_bytes = 0 if ws is None else ws.numel()
    r = C.c_int(-1)
    _L.check("nvfp4_linear",
             _L.load().nvfp4_linear(_ptr(a), M, lda, C.byref(w.desc), _ptr(g_act), _ptr(alpha_w4a16),
                                    _ptr(alpha_w4a4), _ptr(out), ldo, _ptr(ws), ws_bytes, C.byref(r),
                                    _stream()))
    return out, int(r.value)


NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20  # NVFP4_LINEAR_NOALLOC_MAX_WORKSPACE_BYTES
MOE_W4A16_DIRECT_PAIRS = 64  # NVFP4_MOE_W4A16_DIRECT_PAIRS


def linear_noalloc(a: torch.Tensor, w: Weight, g_act: torch.Tensor | None, alpha_w4a16: torch.Tensor,
                   alpha_w4a4: torch.Tensor | None, out: torch.Tensor) -> int:
    """The dispatched linear with no workspace and no allocation (the caller
    passes the output; the W4A4 route's quantized activations go to the
    library's scratch on the GPU).  Returns the route taken."""
    _need(a, torch.bfloat16, "a")
    _need(out, torch.bfloat16, "out")
    lda = _rows(a, "a")
    ldo = _rows(out, "out")
    M = a.shape[0]
    if tuple(out.shape) != (M, w.N):
        raise ValueError(f"out must be [{M}, {w.N}], got {tuple(out.shape)}")
    r = C.c_int(-1)
    _L.check("nvfp4_linear_noalloc",
             _L.load().nvfp4_linear_noalloc(_ptr(a), M, lda, C.byref(w.desc), _ptr(g_act), _ptr(alpha_w4a16),
                                            _ptr(alpha_w4a4), _ptr(out), ldo, C.byref(r), _stream()))
    return int(r.value)


def moe_workspace_layout(T: int, top_k: int, E: int, K: int, I: int) -> dict:
    """Byte offsets of the MoE workspace's parts (and max_tiles, total_bytes)."""
    lay = _L.MoeLayout()
    _L.check("nvfp4_moe_workspace_layout", _L.load().nvfp4_moe_workspace_layout(T, top_k, E, K, I, C.byref(lay)))
    return {name: int(getattr(lay, name)) for name, _ in _L.MoeLayout._fields_}


def moe_workspace_bytes(T: int, top_k: int, E: int, K: int, I: int) -> int:
    return int(_L.load().nvfp4_moe_workspace_bytes(T, top_k, E, K, I))


def moe_workspace_views(ws: torch.Tensor, T: int, top_k: int, E: int, K: int, I: int) -> dict:
    """Views of what a MoE call leaves in its workspace: the align results
    (sorted pairs, expert offsets, tile table) and h's codes and scales by slot."""
    lay = moe_workspace_layout(T, top_k, E, K, I)
    P = T * top_k

    def part(name, nbytes):
        return ws[lay[name]:lay[name] + nbytes]

    return dict(
        sorted=part("sorted", 4 * P).view(torch.int32),
        offsets=part("offsets", 4 * (E + 1)).view(torch.int32),
        tiles=part("tiles", 16 * lay["max_tiles"]).view(torch.int32).view(lay["max_tiles"], 4),
        h_codes=part("h_codes", P * I // 2).view(P, I // 2),
        h_scales=part("h_scales", P * I // 16).view(P, I // 16),
        inv=part("inv", 4 * P).view(torch.int32),
        x_codes=part("x_codes", T * K // 2).view(T, K // 2),
        x_scales=part("x_scales", T * K // 16).view(T, K // 16),
    )


def moe_w4a4(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate_up: Weight, down: Weight,
             num_experts: int, g1: torch.Tensor, g2: torch.Tensor, alpha_gu: torch.Tensor, alpha_dn: torch.Tensor,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             h_amax: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 MoE expert layer (W4A4 gate_up with SiLU gate, W4A4 down, fp32
    route sum).  gate_up holds the E stacked [2I, K] banks, down the E stacked
    [K, I] banks; h_amax (fp32[1], optional) receives max |h|."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    for t, n in ((g1, "g1"), (g2, "g2")):
        _scalar(t, n)
    E = int(num_experts)
    for t, n in ((alpha_gu, "alpha_gu"), (alpha_dn, "alpha_dn")):
        _need(t, torch.float32, n)
        if t.numel() < E or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous fp32 tensor of E values")
    if h_amax is not None:
        _scalar(h_amax, "h_amax")
    ldx = _rows(x, "x")
    T, K = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [T, top_k] tensor")
    if tuple(topk_w.shape) != tuple(topk_ids.shape) or not topk_w.is_contiguous():
        raise ValueError("topk_w must be a contiguous tensor shaped like topk_ids")
    top_k = topk_ids.shape[1]
    I = down.K
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    ldo = _rows(out, "out")
    ws = workspace
    if ws is None:
        need = moe_workspace_bytes(T, top_k, E, K, I)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _L.check("nvfp4_moe_w4a4",
             _L.load().nvfp4_moe_w4a4(_ptr(x), T, ldx, _ptr(topk_ids), _ptr(topk_w), top_k, E, I,
                                      C.byref(gate_up.desc), C.byref(down.desc), _ptr(g1), _ptr(g2),
                                      _ptr(alpha_gu), _ptr(alpha_dn), _ptr(out), ldo, _ptr(ws), ws.numel(),
                                      _ptr(h_amax), _stream()))
    return out


def moe_w4a16_workspace_layout(T: int, top_k: int, E: int, K: int, I: int) -> dict:
    """Byte offsets of the W4A16 MoE workspace's parts (and max_tiles, total_bytes)."""
    lay = _L.MoeW4A16Layout()
    _L.check("nvfp4_moe_w4a16_workspace_layout",
             _L.load().nvfp4_moe_w4a16_workspace_layout(T, top_k, E, K, I, C.byref(lay)))
    return {name: int(getattr(lay, name)) for name, _ in _L.MoeW4A16Layout._fields_}


def moe_w4a16_workspace_bytes(T: int, top_k: int, E: int, K: int, I: int) -> int:
    return int(_L.load().nvfp4_moe_w4a16_workspace_bytes(T, top_k, E, K, I))


def moe_w4a16_workspace_views(ws: torch.Tensor, T: int, top_k: int, E: int, K: int, I: int) -> dict:
    """Views of what a W4A16 MoE call leaves in its workspace: the align
    results (sorted pairs, expert offsets, entries of up to 16 pairs, slot of
    each pair) and h (bf16 bits) by slot."""
    lay = moe_w4a16_workspace_layout(T, top_k, E, K, I)
    P = T * top_k

    def part(name, nbytes):
        return ws[lay[name]:lay[name] + nbytes]

    return dict(
        sorted=part("sorted", 4 * P).view(torch.int32),
        offsets=part("offsets", 4 * (E + 1)).view(torch.int32),
        tiles=part("tiles", 16 * lay["max_tiles"]).view(torch.int32).view(lay["max_tiles"], 4),
        h=part("h", 2 * P * I).view(torch.int16).view(P, I),
        inv=part("inv", 4 * P).view(torch.int32),
    )


def moe_w4a16(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate_up: Weight, down: Weight,
              num_experts: int, alpha_gu: torch.Tensor, alpha_dn: torch.Tensor, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 MoE expert layer with W4A16 on both GEMMs (bf16 x and h), for
    decode-sized batches: gate_up with SiLU gate into bf16 h, down, fp32 route
    sum.  alpha_gu[e] = 1/g_gu[e], alpha_dn[e] = 1/g_dn[e]."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    E = int(num_experts)
    for t, n in ((alpha_gu, "alpha_gu"), (alpha_dn, "alpha_dn")):
        _need(t, torch.float32, n)
        if t.numel() < E or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous fp32 tensor of E values")
    ldx = _rows(x, "x")
    T, K = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [T, top_k] tensor")
    if tuple(topk_w.shape) != tuple(topk_ids.shape) or not topk_w.is_contiguous():
        raise ValueError("topk_w must be a contiguous tensor shaped like topk_ids")
    top_k = topk_ids.shape[1]
    I = down.K
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    ldo = _rows(out, "out")
    ws = workspace
    if ws is None:
        need = moe_w4a16_workspace_bytes(T, top_k, E, K, I)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _L.check("nvfp4_moe_w4a16",
             _L.load().nvfp4_moe_w4a16(_ptr(x), T, ldx, _ptr(topk_ids), _ptr(topk_w), top_k, E, I,
                                       C.byref(gate_up.desc), C.byref(down.desc), _ptr(alpha_gu), _ptr(alpha_dn),
                                       _ptr(out), ldo, _ptr(ws), ws.numel(), _stream()))
    return out


def moe_route(T: int, top_k: int, E: int, has_act_globals: bool) -> int:
    return int(_L.load().nvfp4_moe_route(T, top_k, E, 1 if has_act_globals else 0))


def set_moe_route_tokens_per_expert(tpe: int) -> None:
    _L.load().nvfp4_set_moe_route_tokens_per_expert(int(tpe))


def get_moe_route_tokens_per_expert() -> int:
    return int(_L.load().nvfp4_get_moe_route_tokens_per_expert())


def moe(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, gate_up: Weight, down: Weight,
        num_experts: int, g1: torch.Tensor | None, g2: torch.Tensor | None, alpha_gu_w4a4: torch.Tensor | None,
        alpha_dn_w4a4: torch.Tensor | None, alpha_gu_w4a16: torch.Tensor, alpha_dn_w4a16: torch.Tensor,
        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, int]:
    """Dispatched MoE layer (W4A4 above the tokens-per-expert threshold when
    both static globals are given, else W4A16); returns (out, route taken)."""
    _need(x, torch.bfloat16, "x")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    E = int(num_experts)
    ldx = _rows(x, "x")
    T, K = x.shape
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be a contiguous [T, top_k] tensor")
    if tuple(topk_w.shape) != tuple(topk_ids.shape) or not topk_w.is_contiguous():
        raise ValueError("topk_w must be a contiguous tensor shaped like topk_ids")
    top_k = topk_ids.shape[1]
    I = down.K
    for t, n in ((alpha_gu_w4a4, "alpha_gu_w4a4"), (alpha_dn_w4a4, "alpha_dn_w4a4"),
                 (alpha_gu_w4a16, "alpha_gu_w4a16"), (alpha_dn_w4a16, "alpha_dn_w4a16")):
        if t is not None:
            _need(t, torch.float32, n)
            if t.numel() < E or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous fp32 tensor of E values")
    for t, n in ((g1, "g1"), (g2, "g2")):
        if t is not None:
            _scalar(t, n)
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    ldo = _rows(out, "out")
    ws = workspace
    if ws is None:
        need = int(_L.load().nvfp4_moe_dispatch_workspace_bytes(T, top_k, E, K, I, 1 if g1 is not None else 0))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    route = C.c_int32(-1)
    _L.check("nvfp4_moe",
             _L.load().nvfp4_moe(_ptr(x), T, ldx, _ptr(topk_ids), _ptr(topk_w), top_k, E, I, C.byref(gate_up.desc),
                                 C.byref(down.desc), _ptr(g1), _ptr(g2), _ptr(alpha_gu_w4a4), _ptr(alpha_dn_w4a4),
                                 _ptr(alpha_gu_w4a16), _ptr(alpha_dn_w4a16), _ptr(out), ldo, _ptr(ws), ws.numel(),
                                 C.byref(route), _stream()))
    return out, int(route.value)


def gated_mlp_w4a4(a_codes: torch.Tensor, a_scales: torch.Tensor, gate_up: Weight, alpha_: torch.Tensor,
                   g2: torch.Tensor, h_codes: torch.Tensor | None = None, h_scales: torch.Tensor | None = None,
                   h_amax: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """First GEMM of a gated MLP on NVFP4 activations: h = SiLU(z_gate) * z_up,
    quantized to NVFP4 under g2; returns (h_codes [M, I/2], h_scales [M, I/16])."""
    _need(a_codes, torch.uint8, "a_codes")
    _need(a_scales, torch.uint8, "a_scales")
    _scalar(alpha_, "alpha")
    _scalar(g2, "g2")
    M = a_codes.shape[0]
    if a_codes.shape[1] * 2 != gate_up.K or tuple(a_scales.shape) != (M, gate_up.K // 16):
        raise ValueError("activation codes/scales do not match the weight's K")
    if not a_codes.is_contiguous() or not a_scales.is_contiguous():
        raise ValueError("activation codes and scales must be contiguous")
    I = gate_up.N // 2
    if h_codes is None:
        h_codes = torch.empty((M, I // 2), dtype=torch.uint8, device=a_codes.device)
    if h_scales is None:
        h_scales = torch.empty((M, I // 16), dtype=torch.uint8, device=a_codes.device)
    if tuple(h_codes.shape) != (M, I // 2) or tuple(h_scales.shape) != (M, I // 16):
        raise ValueError("h_codes / h_scales must be [M, I/2] / [M, I/16]")
    if not h_codes.is_contiguous() or not h_scales.is_contiguous():
        raise ValueError("h_codes and h_scales must be contiguous")
    if h_amax is not None:
        _scalar(h_amax, "h_amax")
    _L.check("nvfp4_gated_mlp_w4a4",
             _L.load().nvfp4_gated_mlp_w4a4(_ptr(a_codes), _ptr(a_scales), M, C.byref(gate_up.desc), _ptr(alpha_),
                                            _ptr(g2), _ptr(h_codes), _ptr(h_scales), _ptr(h_amax), _stream()))
    return h_codes, h_scales
