"""Benchmark of the NVFP4 quantized linear on one MI355X.

Headline: W4A16 decode throughput in HBM TB/s over the decode sweep
M in {1, 2, 4, 8, 16} x (N, K) in {(3584, 5120), (8704, 5120), (5120, 1536),
(5120, 4352)} (the shapes of 1Cat-vLLM PR #611, Test Plan), with the W4A4
prefill GEMM at M = 8192, N = 8704, K = 5120 reported beside it in TFLOP/s.

Method (cold weights, as the pages measure decode linears with every layer
read from DRAM: FreeToken PR #737, Results; FlashInfer PR #4038, cold L2):
  * every (shape, M) call cycles through C copies of its weight so that more
    than 2 GB of other weights is read between two uses of one copy (the
    256 MB last-level cache cannot hold them);
  * the calls of one (shape, M) are captured in a HIP graph (C launches) and
    replayed; one step = one replay of each of the 20 graphs;
  * times come from HIP events on the stream the kernels run on.
Algorithmic bytes of one W4A16 launch: N*K/2 (codes) + N*K/16 (scales) +
2*M*K (activations) + 2*M*N (output) + 4 (alpha); of the W4A4 GEMM: 2*M*N*K
FLOPs.

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV HBM TB/s at M=1..16; W4A4 prefill TFLOP/s at M=8192 (% of peak)"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA, MI355X
COLD_BYTES = 2.2e9


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w4a16_bytes(M, N, K):
    return N * K // 2 + N * K // 16 + 2 * M * K + 2 * M * N + 4


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_act_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if they
    were taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    try:
        d = json.load(open(p))
    except Exception:
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("hbm_bytes_per_launch")


def bench_w4a16(ops, torch, steps, warmup):
    from nvfp4_block_scaled_act_amd import synth

    shapes = synth.W4A16_DECODE_SHAPES
    Ms = synth.W4A16_DECODE_M
    per_set = sum(N * K * 9 // 16 for N, K in shapes)
    C = max(2, int(np.ceil(COLD_BYTES / per_set)))
    log(f"[w4a16] {len(shapes)} shapes x M {Ms}; {C} cold copies per weight ({C * per_set / 1e9:.2f} GB)")
    entries = []
    for si, (N, K) in enumerate(shapes):
        W = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_W, si), N, K)
        a = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_A, si), 16, K)
        wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
        g = ops.global_scale(wd)
        codes, scales = ops.quantize_act(wd, g)
        del wd
        alpha = ops.alpha(g)
        copies = [ops.prepare_weight(codes.clone(), scales.clone()) for _ in range(C)]
        ad = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        for M in Ms:
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            entries.append(dict(N=N, K=K, M=M, a=ad[:M], alpha=alpha, out=out, copies=copies))
    torch.cuda.synchronize()
    # capture one graph per (shape, M): C launches over the C copies
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for e in entries:
            for w in e["copies"][:2]:
                ops.linear_w4a16(e["a"], w, e["alpha"], out=e["out"])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for e in entries:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for w in e["copies"]:
                ops.linear_w4a16(e["a"], w, e["alpha"], out=e["out"])
        e["graph"] = g
    torch.cuda.synchronize()
    for _ in range(warmup):
        for e in entries:
            e["graph"].replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in entries]
    per = np.zeros(len(entries))
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(steps):
        for i, e in enumerate(entries):
            evs[i][0].record()
            e["graph"].replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        for i in range(len(entries)):
            per[i] += evs[i][0].elapsed_time(evs[i][1])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    rows = []
    tot_bytes = 0
    tot_kernel_ms = 0.0
    for i, e in enumerate(entries):
        us = per[i] / steps / C * 1e3
        b = w4a16_bytes(e["M"], e["N"], e["K"])
        rows.append(dict(N=e["N"], K=e["K"], M=e["M"], us_per_launch=round(us, 3), tb_s=round(b / us / 1e6, 3)))
        tot_bytes += b * C * steps
        tot_kernel_ms += per[i]
        log(f"[w4a16] N={e['N']:5d} K={e['K']:5d} M={e['M']:2d}: {us:7.2f} us/launch  {b / us / 1e6:6.3f} TB/s")
    step_bytes = sum(w4a16_bytes(e["M"], e["N"], e["K"]) for e in entries) * C
    for e in entries:
        del e["graph"]
    return dict(rows=rows, C=C, total_ms=total_ms, kernel_ms=tot_kernel_ms, bytes=tot_bytes, step_bytes=step_bytes,
                launches=len(entries) * C * steps)


def bench_w4a4(ops, torch, reps=10):
    from nvfp4_block_scaled_act_amd import synth

    N, K = synth.W4A4_PREFILL["N"], synth.W4A4_PREFILL["K"]
    M = 8192
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), M, K)
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    wd = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
    ad = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    cd = torch.from_numpy(cal.view(np.int16)).cuda().view(torch.bfloat16)
    gw, ga = ops.global_scale(wd), ops.global_scale(cd)
    w = ops.prepare_weight(*ops.quantize_act(wd, gw))
    al = ops.alpha(gw, ga)
    ac, as_ = ops.quantize_act(ad, ga)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        ops.quantize_act(ad, ga, ac, as_)
        ops.linear_w4a4(ac, as_, w, al, out=out)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    tq = tg = 0.0
    for _ in range(reps):
        e0.record()
        ops.quantize_act(ad, ga, ac, as_)
        e1.record()
        ops.linear_w4a4(ac, as_, w, al, out=out)
        e2.record()
        torch.cuda.synchronize()
        tq += e0.elapsed_time(e1)
        tg += e1.elapsed_time(e2)
    gemm_us = tg / reps * 1e3
    quant_us = tq / reps * 1e3
    flops = 2.0 * M * N * K
    qbytes = M * K * (2 + 0.5 + 1 / 16)
    log(f"[w4a4] M={M} N={N} K={K}: gemm {gemm_us:.1f} us = {flops / gemm_us / 1e6:.1f} TFLOP/s; "
        f"quantize {quant_us:.1f} us = {qbytes / quant_us / 1e3:.1f} GB/s")
    return dict(M=M, N=N, K=K, gemm_us=gemm_us, quant_us=quant_us, tflops=flops / gemm_us / 1e6,
                linear_tflops=flops / (gemm_us + quant_us) / 1e6, quant_gbs=qbytes / quant_us / 1e3)


def cpu_baseline(target_s=15.0):
    """The oracle (untuned) on a bounded sample of the W4A16 decode sweep:
    shape (8704, 5120) at M = 16 over a prefix of the weight rows."""
    import oracle
    from nvfp4_block_scaled_act_amd import synth

    N, K, M = 8704, 5120, 16
    rows_w = 512
    W = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_W, 1), rows_w, K)
    a = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_A, 1), M, K)
    g = oracle.global_scale(W)
    c, s = oracle.quantize(W, g)
    al = oracle.alpha(g)
    t0 = time.perf_counter()
    n_done = 0
    while True:
        oracle.linear_w4a16(a, c, s, al)
        n_done += rows_w
        if time.perf_counter() - t0 > target_s or n_done >= 64 * rows_w:
            break
    dt = time.perf_counter() - t0
    b = (w4a16_bytes(M, rows_w, K)) * (n_done // rows_w)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return dict(value=b / dt / 1e12, unit="TB/s", cores=cores, kind="oracle",
                sample=f"W4A16 N=8704,K=5120,M=16 on {rows_w} weight rows x {n_done // rows_w} passes, {dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-w4a4", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the NVFP4 linear has no multi-GPU path here); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from nvfp4_block_scaled_act_amd import ops

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    r16 = bench_w4a16(ops, torch, args.steps, args.warmup)
    r4 = None if args.skip_w4a4 else bench_w4a4(ops, torch)
    value_tbs = r16["bytes"] / (r16["kernel_ms"] * 1e-3) / 1e12
    achieved_gbs = r16["bytes"] / (r16["kernel_ms"] * 1e-3) / 1e9
    src16 = kernel_source_hash(["w4a16.hip", "device.hpp"])
    traffic = load_traffic("w4a16_decode_sweep", src16)
    res = {
        "metric": METRIC,
        "value": round(value_tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r16["kernel_ms"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "W4A16 decode sweep: M in {1,2,4,8,16} x (N,K) in {(3584,5120),(8704,5120),(5120,1536),"
                        "(5120,4352)}, NVFP4 weights N(0,1), cold (rotated over %d copies, %.1f GB)"
                        % (r16["C"], r16["C"] * sum(N * K * 9 / 16 for N, K in [(3584, 5120), (8704, 5120),
                                                                            (5120, 1536), (5120, 4352)]) / 1e9),
            "launches_per_step": len(r16["rows"]) * r16["C"],
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "w4a16_kernel", "source_hash": src16},
        "per_shape": r16["rows"],
    }
    if r4 is not None:
        res["w4a4_prefill"] = {
            "workload": "W4A4 M=8192 N=8704 K=5120, NVFP4 activations (static global, 512-row calibration)",
            "tflops": round(r4["tflops"], 2), "unit": "TFLOP/s", "gemm_us": round(r4["gemm_us"], 2),
            "frac_of_fp16_mfma_peak": round(r4["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "linear_tflops_incl_quantize": round(r4["linear_tflops"], 2),
            "quantize_us": round(r4["quant_us"], 2), "quantize_gb_s": round(r4["quant_gbs"], 1),
            "roofline": {"bound": "mfma", "achieved": round(r4["tflops"], 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r4["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": load_traffic("w4a4_prefill_m8192", kernel_source_hash(["w4a4.hip", "device.hpp"]))},
        }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
