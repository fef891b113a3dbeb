"""Benchmark of the NVFP4 quantized linear on one MI355X.

Headline (`value`): W4A16 decode throughput in HBM TB/s over the decode sweep
M in {1, 2, 4, 8, 16} x (N, K) in {(3584, 5120), (8704, 5120), (5120, 1536),
(5120, 4352)} -- the decode shapes of 1Cat-vLLM PR #611 (Test Plan) -- as
total algorithmic bytes over total kernel time.  Reported beside it: the large
fused-weight decode (N = 62080, K = 5120, M in {1, 8, 16}), the W4A4 prefill
GEMM at M = 8192, N = 8704, K = 5120 in TFLOP/s with its activation quantizer,
the one-time weight prepare, and the CPU oracle on a bounded sample.

Method (cold weights, as the pages measure decode linears with every layer
read from DRAM: FreeToken PR #737, Results; FlashInfer PR #4038, cold L2):
  * every (shape, M) call cycles through C prepared copies of its weight so
    that more than 2 GB of other weights is read between two uses of one copy
    (the 256 MB last-level cache cannot hold them);
  * the C calls of one (shape, M) are captured in a HIP graph and replayed;
    one step = one replay of each graph of the sweep;
  * times come from HIP events recorded on the stream the graphs run on.
Beside `value`, `read_floor` times a plain streaming read (nvfp4_stream_read:
one 16-byte nontemporal load per thread, nothing computed) of each call's weight
bytes over the same copies and graphs: what launching a kernel and reading those
bytes from cold memory costs at these sizes, the attainable bound for the sweep.
Algorithmic bytes of one W4A16 call: N*K/2 (codes) + N*K/16 (scales) +
2*M*K (activations) + 2*M*N (output) + 4 (alpha); of one W4A4 GEMM: 2*M*N*K
FLOPs; of one quantizer call: M*K*(2 + 1/2 + 1/16) bytes.

Prints ONE JSON line on stdout; progress goes to stderr.
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


def trace_summary(root):
    """Markdown table of dispatch durations per (kernel, grid, block) from the
    rocprofv3 kernel traces under root: dispatches, median, p10, p90 and mean
    in us, heaviest first."""
    import csv
    import glob

    rows = {}
    for path in sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].replace("nvfp4::(anonymous namespace)::", "").replace("void ", "")
                name = name.split("(")[0]
                grid = r.get("Grid_Size_X") or r.get("Grid_Size", "?")
                block = r.get("Workgroup_Size_X") or r.get("Workgroup_Size", "?")
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                rows.setdefault((name, grid, block), []).append(us)
    out = ["| kernel | grid x block (threads) | dispatches | median us | p10 us | p90 us | mean us |",
           "|---|---|---|---|---|---|---|"]
    for (name, grid, block), ts in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(ts)
        out.append(f"| {name} | {grid} x {block} | {a.size} | {np.median(a):.2f} | {np.percentile(a, 10):.2f} | "
                   f"{np.percentile(a, 90):.2f} | {a.mean():.2f} |")
    return "\n".join(out)


def w4a16_bytes(M, N, K):
    return N * K // 2 + N * K // 16 + 2 * M * K + 2 * M * N + 4


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "nvfp4_block_scaled_act_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/
    counters.json), if they were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("hbm_bytes_per_launch")


def dev_bf16(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def warm_gpu(torch, fn, ms=150.0, max_calls=10000):
    """Run fn until at least `ms` of GPU time has passed.  The MI355X raises
    its clock over the first tens of milliseconds of sustained load (a W4A4
    GEMM at M = 8192 took 740 us in its first calls and 620 us after about 20
    ms), so every timed leg first runs its own calls to the steady state."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    calls = 0
    while calls < max_calls:
        for _ in range(4):
            fn()
        calls += 4
        e1.record()
        e1.synchronize()
        if e0.elapsed_time(e1) >= ms:
            break


def per_call_us(torch, fns, reps):
    """Per-call times (us) of each function in `fns`, called in turn reps
    times, each call between two HIP events, one host synchronization at the
    end.  Returns one list of reps times per function."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(reps)]
    for r in range(reps):
        for i, fn in enumerate(fns):
            ev[r][i][0].record()
            fn()
            ev[r][i][1].record()
    torch.cuda.synchronize()
    return [[ev[r][i][0].elapsed_time(ev[r][i][1]) * 1e3 for r in range(reps)] for i in range(len(fns))]


def stats_us(ts):
    """median, p10, p90 of per-call times (us)."""
    a = np.asarray(ts, np.float64)
    return dict(median=round(float(np.median(a)), 2), p10=round(float(np.percentile(a, 10)), 2),
                p90=round(float(np.percentile(a, 90)), 2), n=int(a.size))


def bench_w4a16(ops, torch, workload, shapes, Ms, steps, warmup, graphs=True):
    """Cold-weight W4A16 timing of every (shape, M); returns per-call rows and
    totals.  graphs=False launches the calls directly (for counter runs, which
    do not see kernels replayed from a graph)."""
    from nvfp4_block_scaled_act_amd import synth

    entries = []
    keep = []
    for si, (N, K) in enumerate(shapes):
        W = synth.normal_bf16(synth.seed_for(workload, synth.ROLE_W, si), N, K)
        a = synth.normal_bf16(synth.seed_for(workload, synth.ROLE_A, si), max(Ms), K)
        wd = dev_bf16(torch, W)
        g = ops.global_scale(wd)
        codes, scales = ops.quantize_act(wd, g)
        del wd
        alpha = ops.alpha(g)
        C = max(2, int(np.ceil(COLD_BYTES / (N * K * 9 / 16))))
        copies = [ops.prepare_weight(codes, scales) for _ in range(C)]
        del codes, scales
        ad = dev_bf16(torch, a)
        keep.append((copies, ad, alpha))
        for M in Ms:
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            entries.append(dict(N=N, K=K, M=M, a=ad[:M], alpha=alpha, out=out, copies=copies, C=C))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the code paths before capture
        for e in entries:
            for w in e["copies"][:2]:
                ops.linear_w4a16(e["a"], w, e["alpha"], out=e["out"])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for e in entries:
        if graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for w in e["copies"]:
                    ops.linear_w4a16(e["a"], w, e["alpha"], out=e["out"])
            e["graph"] = g.replay
            e["_g"] = g
        else:
            e["graph"] = (lambda e=e: [ops.linear_w4a16(e["a"], w, e["alpha"], out=e["out"]) for w in e["copies"]])
    # the read floor: a plain streaming read of each call's weight bytes over
    # the same copies, captured and replayed the same way (graphs only)
    floor = {}
    if graphs:
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        for copies, _, _ in keep:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for w in copies:
                    ops.stream_read(w.data, sink)
            floor[id(copies)] = g
    torch.cuda.synchronize()
    for _ in range(warmup):
        for e in entries:
            e["graph"]()
    warm_gpu(torch, lambda: [e["graph"]() for e in entries], ms=150.0, max_calls=4 * max(1, warmup))
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in entries]
    per = np.zeros(len(entries))
    for _ in range(steps):
        for i, e in enumerate(entries):
            evs[i][0].record()
            e["graph"]()
            evs[i][1].record()
        torch.cuda.synchronize()
        for i in range(len(entries)):
            per[i] += evs[i][0].elapsed_time(evs[i][1])
    fper = {}
    if floor:
        fev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in floor}
        fper = {k: 0.0 for k in floor}
        for g in floor.values():
            g.replay()
        torch.cuda.synchronize()
        for _ in range(steps):
            for k, g in floor.items():
                fev[k][0].record()
                g.replay()
                fev[k][1].record()
            torch.cuda.synchronize()
            for k in floor:
                fper[k] += fev[k][0].elapsed_time(fev[k][1])
    rows, tot_bytes, tot_ms, floor_ms = [], 0.0, 0.0, 0.0
    for i, e in enumerate(entries):
        us = per[i] / steps / e["C"] * 1e3
        b = w4a16_bytes(e["M"], e["N"], e["K"])
        row = dict(N=e["N"], K=e["K"], M=e["M"], us_per_launch=round(us, 3), tb_s=round(b / us / 1e6, 3))
        extra = ""
        if fper:
            fus = fper[id(e["copies"])] / steps / e["C"] * 1e3
            row["read_floor_us"] = round(fus, 3)
            floor_ms += fus * e["C"] * steps / 1e3
            extra = f"  (read floor {fus:5.2f} us)"
        rows.append(row)
        tot_bytes += b * e["C"] * steps
        tot_ms += per[i]
        log(f"[{workload}] N={e['N']:5d} K={e['K']:5d} M={e['M']:2d}: {us:7.2f} us/launch  {b / us / 1e6:6.3f} TB/s{extra}")
    launches = sum(e["C"] for e in entries)
    for e in entries:
        e.pop("graph")
        e.pop("_g", None)
    del keep, floor
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return dict(rows=rows, bytes=tot_bytes, kernel_ms=tot_ms, floor_ms=floor_ms, launches_per_step=launches,
                weight_gb=sum(N * K * 9 / 16 * max(2, int(np.ceil(COLD_BYTES / (N * K * 9 / 16)))) for N, K in shapes) / 1e9)


def bench_w4a4(ops, torch, reps=20):
    from nvfp4_block_scaled_act_amd import synth

    N, K = synth.W4A4_PREFILL["N"], synth.W4A4_PREFILL["K"]
    M = 8192
    W = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), M, K)
    cal = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_CAL), 512, K)
    wd, ad, cd = dev_bf16(torch, W), dev_bf16(torch, a), dev_bf16(torch, cal)
    gw, ga = ops.global_scale(wd), ops.global_scale(cd)
    codes, scales = ops.quantize_act(wd, gw)
    # the one-time prepare step, timed on its second call (the first touches
    # a fresh output buffer) after a warm-up of the clocks
    wbuf = torch.empty(ops.prepared_weight_bytes(N, K), dtype=torch.uint8, device="cuda")
    warm_gpu(torch, lambda: ops.prepare_weight(codes, scales, out=wbuf), ms=30.0)
    prepare_us = stats_us(per_call_us(torch, [lambda: ops.prepare_weight(codes, scales, out=wbuf)], 5)[0])["median"]
    del wbuf
    w = ops.prepare_weight(codes, scales)
    al = ops.alpha(gw, ga)
    ac, as_ = ops.quantize_act(ad, ga)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def quant():
        ops.quantize_act(ad, ga, ac, as_)

    def gemm():
        ops.linear_w4a4(ac, as_, w, al, out=out)

    # quantize -> GEMM pairs issued back to back (as consecutive prefill
    # layers would), after a warm-up to steady clocks; each call between two
    # HIP events; medians over the calls
    warm_gpu(torch, lambda: (quant(), gemm()), ms=200.0)
    tq, tg = per_call_us(torch, [quant, gemm], reps)
    gemm_st, quant_st = stats_us(tg), stats_us(tq)
    gemm_us, quant_us = gemm_st["median"], quant_st["median"]
    # the quantizer on cold inputs: the pairs above re-read one input, which
    # the GEMM between two calls leaves in the 256 MB last-level cache; here
    # each call takes the next of 6 copies (504 MB), so it reads from HBM
    cold = [ad.clone() for _ in range(6)]
    turn = [0]

    def quant_cold():
        ops.quantize_act(cold[turn[0] % len(cold)], ga, ac, as_)
        turn[0] += 1

    warm_gpu(torch, quant_cold, ms=30.0)
    quant_cold_st = stats_us(per_call_us(torch, [quant_cold], 3 * reps)[0])
    del cold
    # the smaller prefill batches of the same workload (prefixes of a)
    sweep = []
    for Ms in synth.W4A4_PREFILL["M"]:
        o = out[:Ms]

        def gm(Ms=Ms, o=o):
            ops.linear_w4a4(ac[:Ms], as_[:Ms], w, al, out=o)

        warm_gpu(torch, gm, ms=30.0)
        st = stats_us(per_call_us(torch, [gm], reps)[0])
        us = st["median"]
        sweep.append(dict(M=Ms, gemm_us=round(us, 2), tflops=round(2.0 * Ms * N * K / us / 1e6, 1), p10_us=st["p10"],
                          p90_us=st["p90"]))
        log(f"[w4a4] M={Ms}: gemm {us:.1f} us = {2.0 * Ms * N * K / us / 1e6:.1f} TFLOP/s (p10 {st['p10']}, p90 "
            f"{st['p90']})")
    # small batches (prefixes of a) on cold copies of the same weight: one
    # launch over all of K (nvfp4_linear_w4a4) against K split across
    # workgroups (nvfp4_linear_w4a4_ws, the dispatched linear's W4A4 kernels)
    small = []
    copies = [ops.prepare_weight(codes, scales) for _ in range(max(2, int(np.ceil(COLD_BYTES / (N * K * 9 / 16)))))]

    def cold_us(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for wc in copies:
                fn(wc)
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            gr.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / len(copies))
        return float(np.median(ts))

    for Ms in (16, 64, 128, 256, 512):
        o = out[:Ms]
        need = ops.linear_w4a4_workspace_bytes(Ms, N, K)
        wsp = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        one = cold_us(lambda wc, Ms=Ms, o=o: ops.linear_w4a4(ac[:Ms], as_[:Ms], wc, al, out=o))
        spl = cold_us(lambda wc, Ms=Ms, o=o, wsp=wsp: ops.linear_w4a4(ac[:Ms], as_[:Ms], wc, al, out=o, workspace=wsp))
        small.append(dict(M=Ms, one_launch_us=round(one, 2), split_k_us=round(spl, 2), partial_mb=round(need / 1e6, 1),
                          split_k_tflops=round(2.0 * Ms * N * K / spl / 1e6, 1)))
        log(f"[w4a4] M={Ms} (cold weight): one launch {one:.1f} us, split-K {spl:.1f} us ({need / 1e6:.1f} MB partials)")
    del copies
    # the gated MLP's gate_up on the same weight read as [2I, K] (I = N/2):
    # the GEMM plus the SiLU gate and NVFP4 quantization of h in its epilogue
    I = N // 2
    hc = torch.empty((M, I // 2), dtype=torch.uint8, device="cuda")
    hs = torch.empty((M, I // 16), dtype=torch.uint8, device="cuda")
    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.gated_mlp_w4a4(ac, as_, w, al, torch.ones(1, dtype=torch.float32, device="cuda"), hc, hs, h_amax=h_amax)
    g2 = (torch.full((1,), 2688.0, dtype=torch.float32, device="cuda") / h_amax).contiguous()

    def gated():
        ops.gated_mlp_w4a4(ac, as_, w, al, g2, hc, hs)

    warm_gpu(torch, gated, ms=60.0)
    gated_st = stats_us(per_call_us(torch, [gated], reps)[0])
    gated_us = gated_st["median"]
    log(f"[w4a4] gated MLP gate_up M={M} 2I={N} K={K}: {gated_us:.1f} us = "
        f"{2.0 * M * N * K / gated_us / 1e6:.1f} TFLOP/s (GEMM alone {sweep[-1]['gemm_us']:.1f} us)")
    flops = 2.0 * M * N * K
    qbytes = M * K * (2 + 0.5 + 1 / 16)
    log(f"[w4a4] M={M} N={N} K={K}: gemm {gemm_us:.1f} us = {flops / gemm_us / 1e6:.1f} TFLOP/s; "
        f"quantize {quant_us:.1f} us = {qbytes / quant_us / 1e3:.1f} GB/s (cold input {quant_cold_st['median']:.1f} us = "
        f"{qbytes / quant_cold_st['median'] / 1e3:.1f} GB/s); prepare {prepare_us:.1f} us")
    return dict(M=M, N=N, K=K, gemm_us=gemm_us, quant_us=quant_us, tflops=flops / gemm_us / 1e6,
                quant_cold_us=quant_cold_st["median"], quant_cold_gbs=qbytes / quant_cold_st["median"] / 1e3,
                linear_tflops=flops / (gemm_us + quant_us) / 1e6, quant_gbs=qbytes / quant_us / 1e3,
                prepare_us=prepare_us, prepare_bytes=2 * N * K * 9 // 16, m_sweep=sweep, small_m=small,
                gemm_stats_us=gemm_st, quant_stats_us=quant_st,
                gated_mlp=dict(M=M, two_I=N, K=K, us=round(gated_us, 2), p10_us=gated_st["p10"],
                               p90_us=gated_st["p90"],
                               tflops=round(2.0 * M * N * K / gated_us / 1e6, 1),
                               gemm_alone_us=sweep[-1]["gemm_us"]))


def moe_flops(T, top_k, K, I):
    """FLOPs of the MoE layer as the pages count them: 2*T*top_k*3*K*I
    (gate_up 2I x K plus down K x I per routed pair; FreeToken PR #736, Results)."""
    return 2.0 * T * top_k * 3 * K * I


def bench_moe(ops, torch, reps=20):
    """The NVFP4 MoE layer (E=128, top-8, K=2048, I=768, T=8192): whole-layer
    time of nvfp4_moe_w4a4 (quantize x, align, gate_up, down, route sum) with
    HIP events.  Banks are quantized per expert on the GPU; g1 comes from the
    512-row calibration batch's amax, g2 from the h amax of the layer run on
    that batch (the layer's own calibration output)."""
    from nvfp4_block_scaled_act_amd import synth

    m = synth.MOE
    E, top_k, K, I, T = m["E"], m["top_k"], m["K"], m["I"], m["T"]
    d = synth.moe_inputs()
    t_setup = time.perf_counter()
    prepared, globals_ = [], []
    for bank in (d["gate_up"], d["down"]):
        rows, cols = bank.shape[1], bank.shape[2]
        dev = dev_bf16(torch, bank.reshape(E * rows, cols))
        codes = torch.empty((E * rows, cols // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((E * rows, cols // 16), dtype=torch.uint8, device="cuda")
        gs = torch.empty(E, dtype=torch.float32, device="cuda")
        for e in range(E):
            sl = slice(e * rows, (e + 1) * rows)
            ops.global_scale(dev[sl], out=gs[e:e + 1])
            ops.quantize_act(dev[sl], gs[e:e + 1], codes=codes[sl], scales=scales[sl])
        del dev
        prepared.append(ops.prepare_weight(codes, scales))
        del codes, scales
        globals_.append(gs)
    w_gu, w_dn = prepared
    g1 = ops.global_scale(dev_bf16(torch, d["cal"]))
    a_gu = torch.empty(E, dtype=torch.float32, device="cuda")
    a_dn = torch.empty(E, dtype=torch.float32, device="cuda")
    for e in range(E):
        ops.alpha(globals_[0][e:e + 1], g1, out=a_gu[e:e + 1])
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    for e in range(E):
        ops.alpha(globals_[1][e:e + 1], one, out=a_dn[e:e + 1])
    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.moe_w4a4(dev_bf16(torch, d["cal"]), torch.from_numpy(d["cal_ids"]).cuda(),
                 torch.from_numpy(d["cal_w"]).cuda(), w_gu, w_dn, E, g1, one, a_gu, a_dn, h_amax=h_amax)
    g2 = (torch.full((1,), 2688.0, dtype=torch.float32, device="cuda") / h_amax).contiguous()
    for e in range(E):
        ops.alpha(globals_[1][e:e + 1], g2, out=a_dn[e:e + 1])
    x = dev_bf16(torch, d["x"])
    ids = torch.from_numpy(d["ids"]).cuda()
    w = torch.from_numpy(d["w"]).cuda()
    ws = torch.empty(ops.moe_workspace_bytes(T, top_k, E, K, I), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"[moe] setup {time.perf_counter() - t_setup:.1f} s, g2 = {g2.item():.6g}")
    def layer():
        ops.moe_w4a4(x, ids, w, w_gu, w_dn, E, g1, g2, a_gu, a_dn, out=out, workspace=ws)

    warm_gpu(torch, layer, ms=200.0)
    st = stats_us(per_call_us(torch, [layer], reps)[0])
    layer_us = st["median"]
    flops = moe_flops(T, top_k, K, I)
    log(f"[moe] T={T} E={E} top_k={top_k} K={K} I={I}: layer {layer_us:.1f} us = "
        f"{flops / layer_us / 1e6:.1f} TFLOP/s (p10 {st['p10']}, p90 {st['p90']})")
    return dict(T=T, E=E, top_k=top_k, K=K, I=I, layer_us=layer_us, tflops=flops / layer_us / 1e6,
                p10_us=st["p10"], p90_us=st["p90"])


def bench_w4a16_tactics(ops, torch, shapes=((11008, 4096), (4096, 11008), (14336, 4096), (4096, 14336),
                                            (28672, 4096)), Ms=(1, 2, 4, 8, 16), reps=3):
    """Cold check of the W4A16 default schedule on shapes outside the decode
    sweep: every candidate (schedule, waves per tile, tiles per workgroup or
    chunk) timed over graph replays of rotated weight copies (about 2.2 GB,
    so each call reads its weight from HBM), the default against the best."""
    import math

    from nvfp4_block_scaled_act_amd import synth
    from nvfp4_block_scaled_act_amd.lib import NVFP4Error

    rows = []
    for N, K in shapes:
        steps = K // 256
        wd = torch.from_numpy(synth.normal_bf16(1, N, K).view(np.int16)).cuda().view(torch.bfloat16)
        g = ops.global_scale(wd)
        c, s = ops.quantize_act(wd, g)
        del wd
        copies = [ops.prepare_weight(c, s) for _ in range(max(2, math.ceil(2.2e9 / (N * K * 9 // 16))))]
        al = ops.alpha(g)
        a = torch.from_numpy(synth.normal_bf16(2, 16, K).view(np.int16)).cuda().view(torch.bfloat16)
        for M in Ms:
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            cands = [(0, 0, 0)]
            for ks in (2, 4, 6, 8, 12, 16):
                per = -(-steps // min(ks, steps))
                if per <= 8:
                    cands.append((3, ks, 0))
                    if -(-steps // per) <= 8:
                        cands.append((3, ks, 2))
                    if M <= 4:
                        cands.append((4, ks, 0))
            cands += [(2, 0, kc) for kc in (1, 2, 4) if M * min(kc, steps) <= 64]
            res = []
            for sch, ks, kc in cands:
                def call(w, sch=sch, ks=ks, kc=kc):
                    ops.linear_w4a16(a[:M], w, al, out=out, schedule=sch, ksplit=ks, chunk_steps=kc)
                try:
                    call(copies[0])
                except NVFP4Error:
                    continue  # not a valid candidate at this shape
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for w in copies:
                        call(w)
                gr.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    gr.replay()
                e1.record()
                torch.cuda.synchronize()
                res.append((e0.elapsed_time(e1) / reps / len(copies) * 1e3, sch, ks, kc))
                del gr
            best = min(res)
            rows.append({"N": N, "K": K, "M": M, "default_us": round(res[0][0], 2), "best_us": round(best[0], 2),
                         "best": {"schedule": best[1], "ksplit": best[2], "chunk_steps": best[3]},
                         "default_over_best": round(res[0][0] / best[0], 3)})
            print("[tactics] N=%d K=%d M=%d default %.2f us, best %.2f us %s" % (N, K, M, res[0][0], best[0],
                  best[1:]), file=sys.stderr, flush=True)
        del copies
        torch.cuda.empty_cache()
    return {"workload": "W4A16 default vs best candidate, cold, N x K in %s, M in %s" % (list(shapes), list(Ms)),
            "geomean_default_over_best": round(float(np.exp(np.mean([np.log(r["default_over_best"]) for r in rows]))),
                                               4),
            "per_shape": rows}


def bench_w4a16_cache_policy(ops, torch, reps=5):
    """Cache-policy bits of the W4A16 loads measured in a sequence, as a decode
    step runs them: per step one decode linear (the dot schedule) on a cold
    weight copy, then a kernel on a buffer that stays cache-resident across
    steps (8 MB, inside the L2s; 64 MB, inside the last-level cache only).
    Per policy: the linear alone, the buffer kernel alone, and the sequence,
    whose excess over the linear is what the linear costs the kernel after it."""
    import math

    from nvfp4_block_scaled_act_amd import synth

    rows = []
    policies = {0: "weights nontemporal, activations default (default)", 1: "weights default",
                2: "weights and activations nontemporal"}
    for N, K, ks in ((8704, 5120, 4), (3584, 5120, 10)):
        wd = dev_bf16(torch, synth.normal_bf16(1, N, K))
        g = ops.global_scale(wd)
        c, s = ops.quantize_act(wd, g)
        del wd
        C = max(2, math.ceil(COLD_BYTES / (N * K * 9 / 16)))
        copies = [ops.prepare_weight(c, s) for _ in range(C)]
        al = ops.alpha(g)
        a = dev_bf16(torch, synth.normal_bf16(2, 2, K))
        for hot_mb in (8, 64):
            hot = torch.ones(hot_mb << 18, dtype=torch.float32, device="cuda")
            for M in (1, 2):
                out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                for cp, name in policies.items():
                    def lin(w, cp=cp):
                        ops.linear_w4a16(a[:M], w, al, out=out, schedule=4, ksplit=ks, cache_policy=cp)

                    for w in copies[:2]:
                        lin(w)
                    torch.cuda.synchronize()
                    graphs = {}
                    for key, fn in (("linear", lambda: [lin(w) for w in copies]),
                                    ("sequence", lambda: [(lin(w), hot.mul_(1.0)) for w in copies]),
                                    ("buffer", lambda: [hot.mul_(1.0) for _ in copies])):
                        gr = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(gr):
                            fn()
                        graphs[key] = gr
                    warm_gpu(torch, lambda: (graphs["linear"].replay(), graphs["sequence"].replay()), ms=50.0)
                    t = {}
                    for key, gr in graphs.items():
                        ts = per_call_us(torch, [gr.replay], reps)[0]
                        t[key] = float(np.median(ts)) / C
                    row = dict(N=N, K=K, M=M, buffer_mb=hot_mb, cache_policy=cp, policy=name,
                               linear_us=round(t["linear"], 2), buffer_alone_us=round(t["buffer"], 2),
                               sequence_us=round(t["sequence"], 2),
                               buffer_in_sequence_us=round(t["sequence"] - t["linear"], 2))
                    rows.append(row)
                    log(f"[cache_policy] N={N} M={M} buffer {hot_mb} MB, {name}: linear {row['linear_us']} us, "
                        f"buffer kernel alone {row['buffer_alone_us']} us, in sequence {row['buffer_in_sequence_us']} us")
                    del graphs
        del copies
        torch.cuda.empty_cache()
    return rows


def bench_moe_decode(ops, torch, Ts=(1, 4, 16), cross_Ts=(16, 64, 128, 192, 256, 512, 1024, 2048), reps=3):
    """The same MoE layer at decode batch sizes through nvfp4_moe_w4a16 (bf16
    x and h, align into entries of up to 16 pairs, grouped W4A16 gate_up with
    the SiLU gate, grouped W4A16 down, route sum).  Cold banks: each call uses
    the next of C prepared copies of both banks (over 2.2 GB in all) and the
    next T tokens of the workload's inputs and routing, inside one HIP graph
    per T.  Bytes per call: the gate_up and down banks of the experts the call
    routes to (each read once: at most 16 pairs per expert here) plus x and
    out; TB/s = bytes / time.  For the layer's tokens-per-expert dispatch,
    both layers (this one and nvfp4_moe_w4a4 with its static globals g1 =
    2688/amax of the calibration batch and g2 from the layer's own h amax on
    it) are also timed the same way at T in cross_Ts."""
    from nvfp4_block_scaled_act_amd import synth

    m = synth.MOE
    E, top_k, K, I = m["E"], m["top_k"], m["K"], m["I"]
    d = synth.moe_inputs()
    banks, gws = [], []
    for bank in (d["gate_up"], d["down"]):
        rows, cols = bank.shape[1], bank.shape[2]
        dev = dev_bf16(torch, bank.reshape(E * rows, cols))
        codes = torch.empty((E * rows, cols // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((E * rows, cols // 16), dtype=torch.uint8, device="cuda")
        gs = torch.empty(E, dtype=torch.float32, device="cuda")
        for e in range(E):
            sl = slice(e * rows, (e + 1) * rows)
            ops.global_scale(dev[sl], out=gs[e:e + 1])
            ops.quantize_act(dev[sl], gs[e:e + 1], codes=codes[sl], scales=scales[sl])
        del dev
        banks.append((codes, scales))
        gws.append(gs)
    expert_bytes = (2 * I * K + K * I) * 9 // 16
    C = max(2, int(np.ceil(COLD_BYTES / (E * expert_bytes))))
    copies = [(ops.prepare_weight(*banks[0]), ops.prepare_weight(*banks[1])) for _ in range(C)]
    del banks
    a_gu = torch.empty(E, dtype=torch.float32, device="cuda")
    a_dn = torch.empty(E, dtype=torch.float32, device="cuda")
    for e in range(E):
        ops.alpha(gws[0][e:e + 1], out=a_gu[e:e + 1])
        ops.alpha(gws[1][e:e + 1], out=a_dn[e:e + 1])
    x = dev_bf16(torch, d["x"])
    ids = torch.from_numpy(d["ids"]).cuda()
    w = torch.from_numpy(d["w"]).cuda()
    # the W4A4 layer's static globals and alphas
    g1 = ops.global_scale(dev_bf16(torch, d["cal"]))
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    a_gu4 = torch.empty(E, dtype=torch.float32, device="cuda")
    a_dn4 = torch.empty(E, dtype=torch.float32, device="cuda")
    for e in range(E):
        ops.alpha(gws[0][e:e + 1], g1, out=a_gu4[e:e + 1])
        ops.alpha(gws[1][e:e + 1], one, out=a_dn4[e:e + 1])
    h_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.moe_w4a4(dev_bf16(torch, d["cal"]), torch.from_numpy(d["cal_ids"]).cuda(),
                 torch.from_numpy(d["cal_w"]).cuda(), *copies[0], E, g1, one, a_gu4, a_dn4, h_amax=h_amax)
    g2 = (torch.full((1,), 2688.0, dtype=torch.float32, device="cuda") / h_amax).contiguous()
    for e in range(E):
        ops.alpha(gws[1][e:e + 1], g2, out=a_dn4[e:e + 1])

    def timed(T, layer):
        n = 2 * C  # calls per graph replay: every copy twice, a new token window each call
        if layer == "w4a16":
            ws = torch.empty(ops.moe_w4a16_workspace_bytes(T, top_k, E, K, I), dtype=torch.uint8, device="cuda")
        else:
            ws = torch.empty(ops.moe_workspace_bytes(T, top_k, E, K, I), dtype=torch.uint8, device="cuda")
        out = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        wins = [(i * T) % (m["T"] - T) for i in range(n)]
        experts = [len(set(d["ids"][s:s + T].reshape(-1).tolist())) for s in wins]
        nbytes = sum(ne * expert_bytes + 4 * T * K for ne in experts)

        def call(i):
            s = wins[i]
            w_gu, w_dn = copies[i % C]
            if layer == "w4a16":
                ops.moe_w4a16(x[s:s + T], ids[s:s + T], w[s:s + T], w_gu, w_dn, E, a_gu, a_dn, out=out,
                              workspace=ws)
            else:
                ops.moe_w4a4(x[s:s + T], ids[s:s + T], w[s:s + T], w_gu, w_dn, E, g1, g2, a_gu4, a_dn4, out=out,
                             workspace=ws)

        for i in range(2):
            call(i)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(n):
                call(i)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        del gr
        us = e0.elapsed_time(e1) * 1e3 / (reps * n)
        return us, sum(experts) / n, nbytes / n

    rows = []
    for T in Ts:
        us, ne, nb = timed(T, "w4a16")
        rows.append(dict(T=T, us=round(us, 2), experts=round(ne, 1), mb=round(nb / 1e6, 2),
                         tb_s=round(nb / us / 1e6, 3)))
        log(f"[moe_decode] T={T}: {us:.2f} us per layer, {ne:.1f} experts, {nb / 1e6:.1f} MB, "
            f"{nb / us / 1e6:.3f} TB/s")
    cross = []
    for T in cross_Ts:
        u16, _, _ = timed(T, "w4a16")
        u4, _, _ = timed(T, "w4a4")
        cross.append(dict(T=T, tokens_per_expert=T * top_k / E, w4a16_us=round(u16, 2), w4a4_us=round(u4, 2)))
        log(f"[moe_crossover] T={T} ({T * top_k / E:.1f} tokens per expert): W4A16 {u16:.2f} us, W4A4 {u4:.2f} us")
    del copies
    torch.cuda.empty_cache()
    return dict(copies=C, rows=rows, crossover=cross)


def bench_fused_sweep(ops, torch, reps=2):
    """The large fused-weight linear through the dispatch (nvfp4_linear) at
    every M of its sweep, over rotated weight copies (cold weights), and the
    W4A4 route forced at M <= 16 (quantize + GEMM) to show where the routes
    cross.  Per call: us, route, TB/s (W4A16: algorithmic bytes) or TFLOP/s
    (W4A4: 2*M*N*K over quantize + GEMM)."""
    from nvfp4_block_scaled_act_amd import synth
    from nvfp4_block_scaled_act_amd.lib import ROUTE_W4A16

    fl = synth.FUSED_LARGE
    N, K, Ms = fl["N"], fl["K"], fl["M"]
    W = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_W), N, K)
    a = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_A), max(Ms), K)
    cal = synth.normal_bf16(synth.seed_for("fused_large", synth.ROLE_CAL), fl["calib_rows"], K)
    wd = dev_bf16(torch, W)
    gw = ops.global_scale(wd)
    codes, scales = ops.quantize_act(wd, gw)
    del wd
    C = max(2, int(np.ceil(COLD_BYTES / (N * K * 9 / 16))))
    copies = [ops.prepare_weight(codes, scales) for _ in range(C)]
    del codes, scales
    ad = dev_bf16(torch, a)
    ga = ops.global_scale(dev_bf16(torch, cal))
    a16, a4 = ops.alpha(gw), ops.alpha(gw, ga)
    ws = torch.empty(ops.linear_workspace_bytes(max(Ms), N, K), dtype=torch.uint8, device="cuda")
    qc = torch.empty((128, K // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((128, K // 16), dtype=torch.uint8, device="cuda")

    warm_gpu(torch, lambda: [ops.linear_w4a16(ad[:16], w, a16) for w in copies[:8]], ms=100.0)

    def timed(fn):
        for w in copies[:2]:
            fn(w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for w in copies:
                fn(w)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * C)

    rows = []
    for M in Ms:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        route = [None]

        def disp(w):
            route[0] = ops.linear(ad[:M], w, ga, a16, a4, out=out, workspace=ws)[1]

        us = timed(disp)
        r = dict(M=M, route="w4a16" if route[0] == ROUTE_W4A16 else "w4a4", us=round(us, 2))
        if r["route"] == "w4a16":
            r["tb_s"] = round(w4a16_bytes(M, N, K) / us / 1e6, 3)
        else:
            r["tflops"] = round(2.0 * M * N * K / us / 1e6, 1)
        rows.append(r)
        rate = f"{r['tb_s']:.3f} TB/s" if "tb_s" in r else f"{r['tflops']:.1f} TFLOP/s"
        log(f"[fused_sweep] N={N} K={K} M={M:5d}: {r['route']} {us:9.2f} us ({rate})")
    # both routes forced around the crossover: W4A16 (its kernels take M <= 64)
    # and W4A4 (quantize + GEMM)
    cross = []
    for M in (8, 16, 24, 32, 40, 48, 56, 64, 96, 128):
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def forced4(w, M=M, out=out):
            ops.quantize_act(ad[:M], ga, codes=qc[:M], scales=qs[:M])
            ops.linear_w4a4(qc[:M], qs[:M], w, a4, out=out)

        c = dict(M=M, w4a4_us=round(timed(forced4), 2))
        if M <= 64:
            c["w4a16_us"] = round(timed(lambda w, M=M, out=out: ops.linear_w4a16(ad[:M], w, a16, out=out)), 2)
        cross.append(c)
        log(f"[fused_sweep] crossover M={M}: W4A16 {c.get('w4a16_us', float('nan')):.1f} us, W4A4 {c['w4a4_us']:.1f} us")
    del copies
    torch.cuda.empty_cache()
    return dict(per_m=rows, crossover=cross, route_m_max=ops.get_route_m_max())


def cpu_baseline(target_s=6.0):
    """The oracle (as it stands) timed on the host cores on bounded samples of
    each leg's workload, in the same units as the GPU figures:
      * W4A16 (the headline's unit, `value`): the call N=8704, K=5120, M=16
        restricted to its first 512 weight rows, repeated for about target_s;
      * quantize: the W4A4 prefill activations (K=5120), 512 rows per pass;
      * W4A4: the prefill GEMM (N=8704, K=5120) on 64 activation rows x 1024
        weight rows per pass;
      * MoE: the NVFP4 MoE layer (E=128, top-8, K=2048, I=768) on its first
        256 tokens, once (bank quantization not timed)."""
    import oracle
    from nvfp4_block_scaled_act_amd import synth

    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def loop(fn):
        fn()  # load the library and touch the data outside the timed loop
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < target_s:
            fn()
            n += 1
        return n, time.perf_counter() - t0

    legs = {}
    K, M, rows_w = 5120, 16, 512
    W = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_W, 1), rows_w, K)
    a = synth.normal_bf16(synth.seed_for("w4a16_decode", synth.ROLE_A, 1), M, K)
    g = oracle.global_scale(W)
    c, s = oracle.quantize(W, g)
    al = oracle.alpha(g)
    n, dt = loop(lambda: oracle.linear_w4a16(a, c, s, al))
    w16 = w4a16_bytes(M, rows_w, K) * n / dt / 1e12
    legs["w4a16"] = dict(value=round(w16, 6), unit="TB/s", sample=f"N=512 rows of (8704, 5120), M=16, {n} passes "
                         f"in {dt:.1f} s")
    N4 = synth.W4A4_PREFILL["N"]
    x = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_A), 512, K)
    ga = np.float32(512.0)
    n, dt = loop(lambda: oracle.quantize(x, ga))
    legs["quantize"] = dict(value=round(512 * K * (2 + 0.5 + 1 / 16) * n / dt / 1e9, 3), unit="GB/s",
                            sample=f"512 x {K} prefill activations, {n} passes in {dt:.1f} s")
    Wp = synth.normal_bf16(synth.seed_for("w4a4_prefill", synth.ROLE_W), 1024, K)
    gw = oracle.global_scale(Wp)
    wc, ws = oracle.quantize(Wp, gw)
    xc, xs = oracle.quantize(x[:64], ga)
    a4 = oracle.alpha(gw, ga)
    n, dt = loop(lambda: oracle.linear_w4a4(xc, xs, wc, ws, a4))
    legs["w4a4"] = dict(value=round(2.0 * 64 * 1024 * K * n / dt / 1e9, 3), unit="GFLOP/s",
                        sample=f"64 activation rows x 1024 weight rows of the ({N4}, {K}) prefill GEMM, {n} passes "
                               f"in {dt:.1f} s")
    d = synth.moe_inputs()
    E, Km, I, top_k = d["E"], d["K"], d["I"], d["top_k"]
    banks = []
    for bank in (d["gate_up"], d["down"]):
        codes = np.empty((E, bank.shape[1], bank.shape[2] // 2), np.uint8)
        scales = np.empty((E, bank.shape[1], bank.shape[2] // 16), np.uint8)
        gs = np.empty(E, np.float32)
        for e in range(E):
            gs[e] = oracle.global_scale(bank[e])
            codes[e], scales[e] = oracle.quantize(bank[e], gs[e])
        banks.append((codes, scales, gs))
    g1 = oracle.global_scale(d["cal"])
    g2 = np.float32(0.1)
    agu = np.array([oracle.alpha(gg, g1) for gg in banks[0][2]], np.float32)
    adn = np.array([oracle.alpha(gg, g2) for gg in banks[1][2]], np.float32)
    nt = 256
    t0 = time.perf_counter()
    oracle.moe_w4a4(d["x"], d["ids"], d["w"], banks[0][0], banks[0][1], banks[1][0], banks[1][1], g1, g2, agu, adn,
                    tokens=np.arange(nt))
    dt = time.perf_counter() - t0
    legs["moe"] = dict(value=round(moe_flops(nt, top_k, Km, I) / dt / 1e9, 3), unit="GFLOP/s",
                       sample=f"the MoE layer on its first {nt} tokens in {dt:.1f} s")
    return dict(value=legs["w4a16"]["value"], unit="TB/s", cores=cores, kind="oracle",
                sample=legs["w4a16"]["sample"] + "; the other legs under 'legs'", legs=legs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the W4A16 calls directly (counter runs)")
    ap.add_argument("--only", choices=["all", "headline", "fused", "fused_sweep", "w4a4", "moe", "moe_decode", "w4a16_tactics",
                                       "w4a16_cache_policy", "copy"],
                    default="all",
                    help="run one part (for profiler runs); 'copy' times a plain 256 MiB device copy, the "
                         "reference for the HBM byte counters")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print per-(kernel, grid) median, p10 and p90 dispatch durations from the rocprofv3 "
                         "kernel traces (*kernel_trace.csv) under DIR and exit (no GPU use)")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the NVFP4 linear here has no multi-GPU path (got --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from nvfp4_block_scaled_act_amd import ops, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only == "copy":
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        print(json.dumps({"copy_bytes": 256 << 20, "us": round(us, 2), "read_write_gb_s": round(2 * (256 << 20) / us / 1e3, 1)}))
        return
    if args.only == "moe":
        r5 = bench_moe(ops, torch, reps=args.steps)
        print(json.dumps({"moe": {k: round(v, 3) if isinstance(v, float) else v for k, v in r5.items()}}))
        return
    if args.only == "w4a16_cache_policy":
        print(json.dumps({"w4a16_cache_policy": bench_w4a16_cache_policy(ops, torch)}))
        return
    if args.only == "w4a16_tactics":
        print(json.dumps({"w4a16_tactics": bench_w4a16_tactics(ops, torch)}))
        return
    if args.only == "moe_decode":
        print(json.dumps({"moe_decode": bench_moe_decode(ops, torch)}))
        return
    if args.only == "fused_sweep":
        print(json.dumps({"fused_large_sweep": bench_fused_sweep(ops, torch)}))
        return
    if args.only in ("fused", "w4a4"):
        if args.only == "fused":
            fl = synth.FUSED_LARGE
            r3 = bench_w4a16(ops, torch, "fused_large", [(fl["N"], fl["K"])], [1, 8, 16], args.steps, args.warmup,
                             graphs=not args.no_graph)
            print(json.dumps({"fused_large_decode": r3["rows"]}))
        else:
            r4 = bench_w4a4(ops, torch, reps=args.steps)
            print(json.dumps({"w4a4_prefill": {k: round(v, 3) if isinstance(v, float) else v for k, v in r4.items()}}))
        return
    shapes = synth.W4A16_DECODE_SHAPES
    Ms = synth.W4A16_DECODE_M
    log(f"[w4a16_decode] {len(shapes)} shapes x M {Ms}, cold rotation over >= {COLD_BYTES / 1e9:.1f} GB per shape")
    r16 = bench_w4a16(ops, torch, "w4a16_decode", shapes, Ms, args.steps, args.warmup, graphs=not args.no_graph)
    achieved_gbs = r16["bytes"] / (r16["kernel_ms"] * 1e-3) / 1e9
    src16 = kernel_source_hash(["w4a16.hip", "device.hpp"])
    res = {
        "metric": METRIC,
        "value": round(achieved_gbs / 1e3, 4),
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
                        "(5120,4352)}, NVFP4 weights from N(0,1), cold (each weight rotated over copies, %.1f GB)"
                        % r16["weight_gb"],
            "launches_per_step": r16["launches_per_step"],
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("w4a16_decode_sweep", src16),
                     "kernel": "w4a16_dot_kernel (M <= 2), w4a16_split_fixed_kernel (M >= 4)", "source_hash": src16},
        "per_shape": r16["rows"],
    }
    if r16["floor_ms"] > 0:
        floor_gbs = r16["bytes"] / (r16["floor_ms"] * 1e-3) / 1e9
        res["read_floor"] = {
            "what": "nvfp4_stream_read of each call's weight bytes (one 16-byte nontemporal load per thread, no "
                    "compute) over the same copies, graphs and order: the launch plus the cold read at these sizes",
            "tb_s": round(floor_gbs / 1e3, 4), "frac_of_hbm_peak": round(floor_gbs / HBM_PEAK_GBS, 4),
            "value_over_floor": round(achieved_gbs / floor_gbs, 4)}
    if args.only == "headline":
        print(json.dumps({"value_tb_s": res["value"], "read_floor": res.get("read_floor"), "per_shape": res["per_shape"]}))
        return
    if args.only == "all":
        fl = synth.FUSED_LARGE
        r3 = bench_w4a16(ops, torch, "fused_large", [(fl["N"], fl["K"])], [1, 8, 16], max(2, args.steps // 2), 1)
        gbs3 = r3["bytes"] / (r3["kernel_ms"] * 1e-3) / 1e9
        res["fused_large_decode"] = {
            "workload": "W4A16 N=62080 K=5120 M in {1,8,16}, cold", "tb_s": round(gbs3 / 1e3, 4),
            "frac_of_hbm_peak": round(gbs3 / HBM_PEAK_GBS, 4),
            "kernel": "w4a16_dot_kernel (M = 1), w4a16_split_fixed_kernel (M = 8), w4a16_shared_kernel (M = 16)",
            "per_m": r3["rows"]}
        fs = bench_fused_sweep(ops, torch)
        res["fused_large_sweep"] = {
            "workload": "dispatched linear N=62080 K=5120 at every M of the sweep (route reported), cold weights; "
                        "both routes forced at M = 8..128 for the crossover",
            "route_m_max": fs["route_m_max"], "per_m": fs["per_m"], "crossover": fs["crossover"]}
        r4 = bench_w4a4(ops, torch)
        res["w4a4_prefill"] = {
            "workload": "W4A4 M=8192 N=8704 K=5120, NVFP4 activations (static global, 512-row calibration)",
            "tflops": round(r4["tflops"], 2), "unit": "TFLOP/s", "gemm_us": round(r4["gemm_us"], 2),
            "frac_of_fp16_mfma_peak": round(r4["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "linear_tflops_incl_quantize": round(r4["linear_tflops"], 2),
            "gemm_us_p10_p90": [r4["gemm_stats_us"]["p10"], r4["gemm_stats_us"]["p90"]],
            "timing": "HIP events around each call of 20 quantize -> GEMM pairs after a 200 ms warm-up; medians",
            "quantize_us": round(r4["quant_us"], 2), "quantize_gb_s": round(r4["quant_gbs"], 1),
            "quantize_cold_us": round(r4["quant_cold_us"], 2), "quantize_cold_gb_s": round(r4["quant_cold_gbs"], 1),
            "quantize_timing": "quantize_us: the pairs above (its input re-read from the last-level cache); "
                               "quantize_cold_us: each call on the next of 6 input copies (504 MB), read from HBM",
            "m_sweep": r4["m_sweep"],
            "small_m": r4["small_m"],
            "small_m_timing": "cold weight copies in HIP graphs; one_launch: nvfp4_linear_w4a4, split_k: "
                              "nvfp4_linear_w4a4_ws (the dispatched linear's W4A4 kernels)",
            "gated_mlp": dict(r4["gated_mlp"], workload="nvfp4_gated_mlp_w4a4 on the same weight as gate_up [2I=8704, "
                              "K=5120], M=8192: GEMM + SiLU gate + NVFP4 quantization of h [M, 4352]"),
            "roofline": {"bound": "mfma", "achieved": round(r4["tflops"], 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r4["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": load_traffic("w4a4_prefill_m8192",
                                                 kernel_source_hash(["w4a4.hip", "gemm_w4a4.hpp", "gemm_skinny.hpp", "device.hpp"]))},
        }
        res["prepare_weight"] = {"workload": "re-tile N=8704 K=5120 (one time, not in value)",
                                 "us": round(r4["prepare_us"], 2),
                                 "gb_s": round(r4["prepare_bytes"] / r4["prepare_us"] / 1e3, 1)}
        r5 = bench_moe(ops, torch)
        res["moe_layer"] = {
            "workload": "NVFP4 MoE W4A4, E=128, top-8, K=2048, I=768, T=8192 (whole layer: quantize, align, "
                        "gate_up + SiLU gate + NVFP4 quantize, down + routing weight + top-8 sum)",
            "tflops": round(r5["tflops"], 2), "unit": "TFLOP/s", "layer_us": round(r5["layer_us"], 2),
            "layer_us_p10_p90": [r5["p10_us"], r5["p90_us"]],
            "flops": moe_flops(r5["T"], r5["top_k"], r5["K"], r5["I"]),
            "frac_of_fp16_mfma_peak": round(r5["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
        }
        r6 = bench_moe_decode(ops, torch)
        res["moe_decode"] = {
            "workload": "NVFP4 MoE W4A16 (nvfp4_moe_w4a16), E=128, top-8, K=2048, I=768, T in {1,4,16}, cold banks "
                        "(%d copies), whole layer: align, gate_up + SiLU gate, down + routing weight, route sum"
                        % r6["copies"],
            "unit": "TB/s of the routed experts' bank bytes", "per_T": r6["rows"],
            "crossover": r6["crossover"],
        }
    if not args.no_cpu_baseline and args.only == "all":
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
