#!/usr/bin/env python3
"""Benchmark of the fused small-M FP8 block-scale quant+GEMM on one MI355X.

Workload (the shape the pages' kernel microbenchmark is quoted on, sglang "[AMD] Small-M FP8
block-scale GEMM with fused activation quant for gfx950 (Qwen3.5)", section Kernel
microbenchmarks): N=5120, K=4096 (the in_proj_qkvz shard), bf16 activations at
M = 1, 4, 8, 16, 32 rows, e4m3 weights with fp32 128x128 block scales, bf16 output, graph replay,
weights rotated over 24 distinct copies so they are not cache resident.

For every M a HIP graph of 24 fused calls is captured, call i on weight copy i.  One step is one
replay of each M's graph: 24 calls at every M of the sweep, 120 calls in all.  value = algorithmic
bytes moved by the timed calls / elapsed time of the timed steps (HIP events on the stream the
graphs run on).  Each M's graph is also timed on its own for the per-M us/call.

Prints one JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call + achieved HBM GB/s (% of MI355X peak), fused quant+FP8 GEMM, M=1–32"
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
N_DEFAULT, K_DEFAULT = 5120, 4096
M_SWEEP = (1, 4, 8, 16, 32)
COPIES = 24
# The pages' fused-kernel times for this shape (us), same hardware and method: context for vs_baseline.
PAGES_FUSED_US = {1: 6.8, 4: 7.3, 8: 7.7, 16: 9.0, 32: 12.8}
# The pages' FP8 block-scale small-M MoE kernel on MI355X (E = 513, 11 slots, hidden 4096), in us:
# intermediate 256 (TP4) and 128 (TP8) from the graph-replay table, TP8 from 24 tokens on from the
# table with 60 layers rotated (context for the MoE configs; another implementation's times)
PAGES_MOE_FP8_US = {256: {1: 26.6, 4: 43.4, 8: 63.7, 16: 97.5, 20: 115.3},
                    128: {1: 22.7, 4: 30.1, 8: 41.4, 16: 60.4, 20: 68.7, 24: 65.2, 28: 75.8, 32: 82.9,
                          36: 92.0, 48: 111.6}}
MOE_LAYERS = 16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash():
    src = os.path.join(ROOT, "precision_gemm_x128_amd", "csrc", "smallm_fp8bs.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def load_traffic(kname):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's counts), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fused_quant_gemm_5120x4096_traffic.md")
    try:
        text = open(path).read()
        d = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    k = d.get("kernels", {}).get(kname)
    return None if k is None else k.get("hbm_bytes_per_launch")


def time_config(P, torch, np, synthgen, dev, N, K, Ms, copies, reps, e8m0=False, outliers=False):
    """us/call of the fused path at each M on N x K: a HIP graph of `copies` calls on distinct
    weight copies (cold), replayed `reps` times, timed with HIP events on the replay stream.
    Returns {M: us}, plus the outputs of the last call at each M (for cross-checks)."""
    qw = P.smallm_fp8bs_quant_weight_e8m0 if e8m0 else P.smallm_fp8bs_quant_weight
    fn = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
    wps, sws = [], []
    for i in range(copies):
        w = torch.from_numpy(synthgen.gen_w(N, K, seed=0, copy=i)).to(dev)
        w8, sw = qw(w)
        wps.append(P.smallm_fp8bs_pack_weight(w8))
        sws.append(sw)
        del w, w8
    out, ys = {}, {}
    # the streaming-read floor over the same 24 weight buffers, same graph shape
    out["floor"] = graph_us(torch, lambda i: P.smallm_fp8bs_read_floor(wps[i]), copies, reps)
    for M in Ms:
        x = torch.from_numpy(synthgen.gen_x(M, K, seed=0, outliers=outliers).view(np.int16).copy()).to(dev).view(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                fn(x, wps[i], sws[i], y=y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(copies):
                fn(x, wps[i], sws[i], y=y)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        out[M] = a.elapsed_time(b) * 1e3 / (reps * copies)
        ys[M] = y.float().cpu()
    del wps, sws
    torch.cuda.empty_cache()
    return out, ys


def graph_us(torch, fn, copies, reps):
    """us per layer of a HIP graph of `copies` layers, layer i issued by fn(i), replayed `reps`
    times after warm-up, timed with HIP events on the replay stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(copies):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(copies):
            fn(i)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * copies)


def producer_pipeline(P, torch, np, synthgen, dev, copies, reps, N=5120, K=4096):
    """The producer-side fusion: per layer, (a) a plain RMSNorm then the fused quant+GEMM, and
    (b) RMSNorm with the 1x128 quantisation then the GEMM on pre-quantised input, each kernel
    also timed alone; 24 layers on distinct weight copies in one graph, both scale types."""
    res = {}
    rng = np.random.default_rng([3, 3])
    wn_bits = synthgen.f32_to_bf16_bits(rng.normal(1.0, 0.2, K).astype(np.float32))
    wn = torch.from_numpy(wn_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    for e8m0 in (False, True):
        qw = P.smallm_fp8bs_quant_weight_e8m0 if e8m0 else P.smallm_fp8bs_quant_weight
        prod = P.smallm_fp8bs_rmsnorm_quant_e8m0 if e8m0 else P.smallm_fp8bs_rmsnorm_quant
        fused = P.smallm_fp8bs_quant_gemm_e8m0 if e8m0 else P.smallm_fp8bs_quant_gemm
        preq = P.smallm_fp8bs_gemm_e8m0 if e8m0 else P.smallm_fp8bs_gemm
        wps, sws = [], []
        for i in range(copies):
            w = torch.from_numpy(synthgen.gen_w(N, K, seed=0, copy=i)).to(dev)
            w8, sw = qw(w)
            wps.append(P.smallm_fp8bs_pack_weight(w8))
            sws.append(sw)
            del w, w8
        d = {}
        for M in M_SWEEP:
            x = torch.from_numpy(synthgen.gen_x(M, K, seed=0).view(np.int16).copy()).to(dev).view(torch.bfloat16)
            y = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sx = torch.empty((M, K // 128), dtype=torch.uint8 if e8m0 else torch.float32, device=dev)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            t = {
                "rmsnorm_us": graph_us(torch, lambda i: prod(x, wn, 1e-6, y=y, emit_q=False), copies, reps),
                "rmsnorm_quant_us": graph_us(torch, lambda i: prod(x, wn, 1e-6, q=q, sx=sx, emit_y=False), copies, reps),
                "fused_gemm_us": graph_us(torch, lambda i: fused(y, wps[i], sws[i], y=out), copies, reps),
                "prequantised_gemm_us": graph_us(torch, lambda i: preq(q, sx, wps[i], sws[i], y=out), copies, reps),
                "rmsnorm_then_fused_us": graph_us(torch, lambda i: (prod(x, wn, 1e-6, y=y, emit_q=False),
                                                                     fused(y, wps[i], sws[i], y=out)), copies, reps),
                "rmsnorm_quant_then_prequantised_us": graph_us(torch, lambda i: (prod(x, wn, 1e-6, q=q, sx=sx, emit_y=False),
                                                                                  preq(q, sx, wps[i], sws[i], y=out)), copies, reps),
            }
            d[str(M)] = {k: round(v, 3) for k, v in t.items()}
            log(f"[bench] producer {'e8m0' if e8m0 else 'fp32'} M={M}: norm+fused {t['rmsnorm_then_fused_us']:.2f} "
                f"producer+prequantised {t['rmsnorm_quant_then_prequantised_us']:.2f} us/layer")
        res[f"producer_pipeline_{N}x{K}_{'e8m0' if e8m0 else 'fp32'}"] = d
        del wps, sws
        torch.cuda.empty_cache()
    return res


def two_launch_beyond(P, torch, np, synthgen, dev, copies, reps, Ms, N=4096, K=2048):
    """Beyond the small-M range: the standalone quantisation, then the GEMM on pre-quantised
    input (the MFMA-tiled kernel), each alone and back to back."""
    wps, sws = [], []
    for i in range(copies):
        w = torch.from_numpy(synthgen.gen_w(N, K, seed=0, copy=i)).to(dev)
        w8, sw = P.smallm_fp8bs_quant_weight(w)
        wps.append(P.smallm_fp8bs_pack_weight(w8))
        sws.append(sw)
        del w, w8
    d = {}
    for M in Ms:
        x = torch.from_numpy(synthgen.gen_x(M, K, seed=0).view(np.int16).copy()).to(dev).view(torch.bfloat16)
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sx = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        tq = graph_us(torch, lambda i: P.smallm_fp8bs_quant(x, q=q, sx=sx), copies, reps)
        tg = graph_us(torch, lambda i: P.smallm_fp8bs_gemm(q, sx, wps[i], sws[i], y=y), copies, reps)
        t2 = graph_us(torch, lambda i: (P.smallm_fp8bs_quant(x, q=q, sx=sx),
                                        P.smallm_fp8bs_gemm(q, sx, wps[i], sws[i], y=y)), copies, reps)
        tf = 2.0 * M * N * K / (tg * 1e-6) / 1e12
        d[str(M)] = {"quant_us": round(tq, 3), "gemm_us": round(tg, 3), "two_launch_us": round(t2, 3),
                     "gemm_TFLOP_s": round(tf, 2), "gemm_pct_fp8_mfma_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
                     "gemm_kernel": P.kernel_name(M, N, K, 2)}
    log("[bench] 4096x2048 M>32 two launches: " + " ".join(f"M={M} {d[str(M)]['two_launch_us']:.2f}us" for M in Ms))
    del wps, sws
    torch.cuda.empty_cache()
    return d


def crossover_beyond(P, torch, np, synthgen, dev, copies, reps):
    """Past 32 rows on each of the pages' shapes: the fused kernel in 32-row chunks (the C entry
    without a workspace) against the standalone quantisation plus the tiled GEMM (the workspace
    entry), and the rows from which the library takes the second (the fused Python entry)."""
    import ctypes
    L = P.lib()
    res = {}
    for N, K in ((5120, 4096), (4608, 4096), (4096, 2048), (2048, 4096)):
        wps, sws = [], []
        for i in range(copies):
            w = torch.from_numpy(synthgen.gen_w(N, K, seed=0, copy=i)).to(dev)
            w8, sw = P.smallm_fp8bs_quant_weight(w)
            wps.append(P.smallm_fp8bs_pack_weight(w8))
            sws.append(sw)
            del w, w8
        lid = P.smallm_fp8bs_weight_layout_id(N, K)
        d = {}
        for M in (33, 48, 64, 128, 256):
            x = torch.from_numpy(synthgen.gen_x(M, K, seed=0).view(np.int16).copy()).to(dev).view(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            need = P.smallm_fp8bs_quant_gemm_workspace_bytes(max(M, 33), N, K)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def chunks(i):
                st = L.smallm_fp8bs_quant_gemm(P._ptr(x), K, P._ptr(wps[i]), lid, P._ptr(sws[i]), P._ptr(y), N, M, N, K,
                                               None, None, P._stream())
                assert st == 0, st

            def two(i):
                # the workspace entry's second path, called directly (it takes it from 33 rows)
                q = ws[: M * K].view(M, K)
                sx = ws[(M * K + 255) // 256 * 256:][: M * (K // 128) * 4].view(torch.float32).view(M, K // 128)
                P.smallm_fp8bs_quant(x, q=q, sx=sx)
                P.smallm_fp8bs_gemm(q, sx, wps[i], sws[i], y=y)
            tc = graph_us(torch, chunks, copies, reps)
            tt = graph_us(torch, two, copies, reps)
            d[str(M)] = {"fused_32_row_chunks_us": round(tc, 3), "quant_then_tiled_us": round(tt, 3),
                         "library_takes": "quant_then_tiled" if P.smallm_fp8bs_quant_gemm_workspace_bytes(M, N, K) else "fused_32_row_chunks"}
        res[f"{N}x{K}"] = d
        log(f"[bench] {N}x{K} beyond 32 rows (chunks / quant+tiled): " +
            " ".join(f"M={M} {d[str(M)]['fused_32_row_chunks_us']:.1f}/{d[str(M)]['quant_then_tiled_us']:.1f}" for M in (33, 48, 64, 128, 256)))
        del wps, sws
        torch.cuda.empty_cache()
    return res


def moe_sweeps(P, torch, np, synthgen, dev, reps, layers=MOE_LAYERS):
    """The MoE layers on the pages' shapes (E = 513, 11 slots with the shared expert last, hidden
    4096): FP8 block-scale at intermediate 256 and 128, MXFP4 at intermediate 256.  Each of `layers`
    layers has its own 513 packed experts and its own routing; one HIP graph issues one call per
    layer, so every call reads experts no other call in the graph touched (cold weights).  Weight
    bytes are random codes (e4m3 without NaN codes, |w| <= 1.875 times a 2e-3 block scale; any
    e2m1 code with scale byte 120), which changes nothing in the arithmetic's timing."""
    E, S, H = 513, 11, 4096
    res = {}
    x = torch.from_numpy(synthgen.gen_x(48, H, seed=5).view(np.int16)).to(dev).view(torch.bfloat16)
    for fmt, I, Ts in (("fp8", 256, (1, 4, 8, 16, 20)), ("fp8", 128, (1, 4, 8, 16, 20, 24, 32, 48)),
                       ("mxfp4", 256, (1, 4, 8, 16, 20, 40))):
        fp4 = fmt == "mxfp4"
        g = torch.Generator(device=dev)
        g.manual_seed(1234 + I)
        kdiv = 2 if fp4 else 1
        w13 = torch.empty((layers * E, 2 * I, H // kdiv), dtype=torch.uint8, device=dev)
        w2 = torch.empty((layers * E, H, I // kdiv), dtype=torch.uint8, device=dev)
        if fp4:
            s13 = torch.empty((layers * E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
            s2 = torch.empty((layers * E, H, I // 32), dtype=torch.uint8, device=dev)
        else:
            s13 = torch.full((layers * E, 2 * I // 128, H // 128), 2e-3, dtype=torch.float32, device=dev)
            s2 = torch.full((layers * E, H // 128, I // 128), 2e-3, dtype=torch.float32, device=dev)
        for l in range(layers):
            sl = slice(l * E, (l + 1) * E)
            a = torch.randint(0, 256, (E, 2 * I, H // kdiv), dtype=torch.uint8, device=dev, generator=g)
            b = torch.randint(0, 256, (E, H, I // kdiv), dtype=torch.uint8, device=dev, generator=g)
            if fp4:
                P.smallm_fp8bs_moe_mxfp4_pack(a, torch.full((E, 2 * I, H // 32), 120, dtype=torch.uint8, device=dev),
                                              True, out=w13[sl], out_s=s13[sl])
                P.smallm_fp8bs_moe_mxfp4_pack(b, torch.full((E, H, I // 32), 120, dtype=torch.uint8, device=dev),
                                              False, out=w2[sl], out_s=s2[sl])
            else:
                P.smallm_fp8bs_moe_pack(a & 0xBF, True, out=w13[sl])
                P.smallm_fp8bs_moe_pack(b & 0xBF, False, out=w2[sl])
            del a, b
        torch.cuda.synchronize()
        d = {}
        for T in Ts:
            routes = [synthgen.gen_moe_routing(T, S, E, seed=100 * l + T) for l in range(layers)]
            ids = [torch.from_numpy(r[0]).to(dev) for r in routes]
            tw = [torch.from_numpy(r[1]).to(dev) for r in routes]
            ws = P.moe_workspace(T, S, H, I, device=dev)
            y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            xt = x[:T]

            def call(l):
                sl = slice(l * E, (l + 1) * E)
                if fp4:
                    P.smallm_fp8bs_moe_mxfp4(xt, ids[l], tw[l], w13[sl], s13[sl], w2[sl], s2[sl], workspace=ws, y=y)
                else:
                    P.smallm_fp8bs_moe(xt, ids[l], tw[l], w13[sl], s13[sl], w2[sl], s2[sl], workspace=ws, y=y)

            us = graph_us(torch, call, layers, reps)
            nbytes = sum(P.moe_algorithmic_bytes(r[0], E, H, I, mxfp4=fp4) for r in routes) / layers
            gbs = nbytes / (us * 1e-6) / 1e9
            e = {"us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes), "GB_s": round(gbs, 1),
                 "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1), "launches": 2,
                 "splits": P.smallm_fp8bs_moe_splits(T, S)}
            if not fp4 and T in PAGES_MOE_FP8_US[I]:
                e["pages_fp8_kernel_us"] = PAGES_MOE_FP8_US[I][T]
            d[str(T)] = e
        res[f"moe_{fmt}_E{E}_S{S}_H{H}_I{I}"] = d
        log(f"[bench] moe {fmt} I={I}: " + " ".join(f"T={T} {d[str(T)]['us_per_call']:.1f}us" for T in Ts))
        del w13, w2, s13, s2
        torch.cuda.empty_cache()
    return res


def config_sweeps(P, torch, np, synthgen, dev, copies, reps):
    """The other workloads of the method, timed the same way (per-M us/call, GB/s, % of peak):
    the single 4096x2048 call at M=4; the M sweeps on 4608x4096 and 4096x2048 with outlier rows
    (the latter also over 64 weight copies, more than the MALL holds);
    M = 33..256 on 4096x2048 with the MFMA rate beside the bandwidth (fused, and quant then the
    tiled GEMM on pre-quantised input); the e8m0-scale path on
    4096x2048 and 2048x4096 beside the fp32-scale path on the same data; and the producer-side
    fusion (RMSNorm with the quantisation, then the GEMM on pre-quantised input) on 5120x4096."""
    res = {}

    def entry(N, K, M, us, e8m0=False, floor=None):
        b = P.algorithmic_bytes(M, N, K, e8m0)
        gbs = b / (us * 1e-6) / 1e9
        e = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
             "kernel": P.kernel_name(M, N, K, 1 if e8m0 else 0)}
        if floor is not None:
            e["read_floor_us"] = round(floor, 3)
            e["time_over_floor"] = round(us / floor, 3)
        return e

    t, _ = time_config(P, torch, np, synthgen, dev, 4096, 2048, [4], copies, reps)
    res["single_4096x2048_m4"] = entry(4096, 2048, 4, t[4], floor=t["floor"])
    for N, K in ((4608, 4096), (4096, 2048)):
        t, _ = time_config(P, torch, np, synthgen, dev, N, K, list(M_SWEEP), copies, reps, outliers=True)
        res[f"sweep_{N}x{K}_outliers"] = {str(M): entry(N, K, M, t[M], floor=t["floor"]) for M in M_SWEEP}
        log(f"[bench] {N}x{K} outliers: " + " ".join(f"M={M} {t[M]:.2f}us" for M in M_SWEEP))
    # 24 copies of an 8 MiB weight (192 MiB) fit in the 256 MB MALL: the same sweep over 64 copies
    # (512 MiB) shows whether the 24-copy figures were helped by it
    t, _ = time_config(P, torch, np, synthgen, dev, 4096, 2048, list(M_SWEEP), 64, reps, outliers=True)
    res["sweep_4096x2048_outliers_64copies"] = {str(M): entry(4096, 2048, M, t[M], floor=t["floor"]) for M in M_SWEEP}
    log("[bench] 4096x2048 outliers, 64 copies: " + " ".join(f"M={M} {t[M]:.2f}us" for M in M_SWEEP))
    big = (33, 48, 64, 128, 256)
    t, _ = time_config(P, torch, np, synthgen, dev, 4096, 2048, list(big), copies, reps)
    d = {}
    for M in big:
        e = entry(4096, 2048, M, t[M])
        tf = 2.0 * M * 4096 * 2048 / (t[M] * 1e-6) / 1e12
        e.update({"TFLOP_s": round(tf, 2), "pct_fp8_mfma_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2)})
        d[str(M)] = e
    res["beyond_small_m_4096x2048"] = d
    log("[bench] 4096x2048 M>32: " + " ".join(f"M={M} {t[M]:.2f}us" for M in big))
    res["beyond_small_m_4096x2048_two_launch"] = two_launch_beyond(P, torch, np, synthgen, dev, copies, reps, big)
    res["beyond_small_m_crossover"] = crossover_beyond(P, torch, np, synthgen, dev, copies, reps)
    for N, K in ((4096, 2048), (2048, 4096)):
        ms = [1, 8, 32]
        tf, yf = time_config(P, torch, np, synthgen, dev, N, K, ms, copies, reps)
        te, ye = time_config(P, torch, np, synthgen, dev, N, K, ms, copies, reps, e8m0=True)
        d = {}
        for M in ms:
            rel = float(((ye[M] - yf[M]).abs().max() / yf[M].abs().max()).item())
            d[str(M)] = {"fp32_scales": entry(N, K, M, tf[M], floor=tf["floor"]),
                         "e8m0_scales": entry(N, K, M, te[M], True, floor=te["floor"]),
                         "max_abs_diff_over_max_abs": round(rel, 5)}
        res[f"e8m0_vs_fp32_{N}x{K}"] = d
        log(f"[bench] {N}x{K} e8m0 vs fp32: " + " ".join(f"M={M} {te[M]:.2f}/{tf[M]:.2f}us" for M in ms))
    res.update(producer_pipeline(P, torch, np, synthgen, dev, copies, reps))
    res.update(moe_sweeps(P, torch, np, synthgen, dev, reps))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=COPIES)
    ap.add_argument("--N", type=int, default=N_DEFAULT)
    ap.add_argument("--K", type=int, default=K_DEFAULT)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' timings")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="target seconds per CPU leg")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per M for the per-M breakdown")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times): the "
                         "reference kernel for scaling HBM byte counters, then exit")
    ap.add_argument("--beyond-only", action="store_true",
                    help="only time the paths past 32 rows on the pages' shapes (fused chunks against quant + "
                         "tiled GEMM) and print them as JSON")
    ap.add_argument("--only-m", type=int, default=0,
                    help="profiling runs: time this one M of the sweep only (no configs, no CPU leg)")
    ap.add_argument("--moe-only", action="store_true",
                    help="only time the MoE layers (as in the other workloads) and print them as JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import precision_gemm_x128_amd as P
    import synthgen

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calib_copy_mib} MiB three times")
        return
    N, K, copies = args.N, args.K, args.copies
    global M_SWEEP
    if args.only_m:
        M_SWEEP = (args.only_m,)
        args.no_configs = args.no_cpu = True
    P.lib()
    if args.moe_only:
        print(json.dumps({"moe": moe_sweeps(P, torch, np, synthgen, dev, max(1, args.reps))}))
        return
    if args.beyond_only:
        print(json.dumps({"beyond_small_m_crossover": crossover_beyond(P, torch, np, synthgen, dev, copies,
                                                                         max(1, args.reps))}))
        return

    # ---- inputs: 24 cold weight copies, quantised and packed on the device (load-time work) ----
    t0 = time.time()
    wps, sws = [], []
    for i in range(copies):
        w = torch.from_numpy(synthgen.gen_w(N, K, seed=0, copy=i)).to(dev)
        w8, sw = P.smallm_fp8bs_quant_weight(w)
        wps.append(P.smallm_fp8bs_pack_weight(w8))
        sws.append(sw)
        del w, w8
    torch.cuda.synchronize()
    log(f"[bench] prepared {copies} weight copies {N}x{K} in {time.time() - t0:.1f}s")
    xs = {M: torch.from_numpy(synthgen.gen_x(M, K, seed=0).view(np.int16).copy()).to(dev).view(torch.bfloat16)
          for M in M_SWEEP}
    ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in M_SWEEP}

    # ---- one graph of `copies` calls per M ----
    graphs = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for M in M_SWEEP:
            for i in range(copies):
                P.smallm_fp8bs_quant_gemm(xs[M], wps[i], sws[i], y=ys[M])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for M in M_SWEEP:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(copies):
                P.smallm_fp8bs_quant_gemm(xs[M], wps[i], sws[i], y=ys[M])
        graphs[M] = g
    # read floor: the library's plain streaming read over the same 24 weight buffers, one launch
    # per buffer in a graph (the achievable time for the weight bytes alone)
    gread = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gread):
        for i in range(copies):
            P.smallm_fp8bs_read_floor(wps[i])
    # launch floor: the same number of trivial launches in a graph
    tiny = torch.zeros(1, device=dev)
    gfloor = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gfloor):
        for i in range(copies):
            tiny.add_(1.0)
    torch.cuda.synchronize()

    def run_step():
        for M in M_SWEEP:
            graphs[M].replay()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps ----
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run_step()
    ev1.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    step_ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {step_ms:.4f} ms/step (wall {1e3 * (wall1 - wall0) / args.steps:.4f})")

    bytes_per_call = {M: P.algorithmic_bytes(M, N, K) for M in M_SWEEP}
    step_bytes = copies * sum(bytes_per_call.values())
    value = step_bytes / (step_ms * 1e-3) / 1e9

    # ---- per-M breakdown (each M's graph timed on its own, same stream) ----
    reps = max(1, args.reps)
    sweep = {}
    for M in M_SWEEP:
        graphs[M].replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            graphs[M].replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (reps * copies)
        gbs = bytes_per_call[M] / (us * 1e-6) / 1e9
        sweep[str(M)] = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1),
                         "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
                         "algorithmic_bytes": bytes_per_call[M], "kernel": P.kernel_name(M, N, K),
                         "plan": P.smallm_fp8bs_launch_plan(M, N, K)}
        log(f"[bench] M={M}: {us:.3f} us/call, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of peak)")
    gfloor.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gfloor.replay()
    b.record()
    torch.cuda.synchronize()
    floor_us = a.elapsed_time(b) * 1e3 / (reps * copies)
    log(f"[bench] trivial-kernel launch floor in a graph: {floor_us:.3f} us/launch")
    gread.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gread.replay()
    b.record()
    torch.cuda.synchronize()
    read_floor_us = a.elapsed_time(b) * 1e3 / (reps * copies)
    log(f"[bench] streaming-read floor of the {N}x{K} weight bytes: {read_floor_us:.3f} us/launch "
        f"({N * K / (read_floor_us * 1e-6) / 1e9:.0f} GB/s)")
    for M in M_SWEEP:
        sweep[str(M)]["time_over_read_floor"] = round(sweep[str(M)]["us_per_call"] / read_floor_us, 3)

    # ---- roofline of the dominant kernel instantiation (largest share of the step's time) ----
    by_kernel = {}
    for M in M_SWEEP:
        k = sweep[str(M)]["kernel"]
        d = by_kernel.setdefault(k, {"bytes": 0, "us": 0.0, "launches": 0})
        d["bytes"] += bytes_per_call[M]
        d["us"] += sweep[str(M)]["us_per_call"]
        d["launches"] += 1
    dom = max(by_kernel, key=lambda k: by_kernel[k]["us"])
    d = by_kernel[dom]
    achieved = (d["bytes"] / d["launches"]) / (d["us"] / d["launches"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(dom),
                "kernel": dom, "avg_launch_us": round(d["us"] / d["launches"], 3),
                "launch_ms": [m for m in M_SWEEP if sweep[str(m)]["kernel"] == dom],
                "floor_us": round(read_floor_us, 3),
                "frac_of_floor": round(read_floor_us / (d["us"] / d["launches"]), 4),
                "floor_kernel": "read_floor_kernel (library streaming read of the same weight bytes)"}

    # ---- pages' kernel on the same workload (same hardware): context ratio ----
    pages_step_us = sum(PAGES_FUSED_US[M] for M in M_SWEEP)
    pages_gbs = sum(bytes_per_call.values()) / (pages_step_us * 1e-6) / 1e9
    vs_baseline = round(value / pages_gbs, 3) if (N, K) == (5120, 4096) else None

    # ---- the other workloads (after the timed region; not part of `value`) ----
    configs = None
    if not args.no_configs:
        del graphs, wps, sws
        torch.cuda.empty_cache()
        configs = config_sweeps(P, torch, np, synthgen, dev, min(copies, COPIES), 10)

    # ---- CPU oracle baseline (rank 0, N=1 only), bounded sample ----
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(N, K, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs_baseline,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded N(0,1) x 2^U(-4,4) per 1x128 group activations; N(0,0.02) weights quantised per 128x128 block)",
        "config": {"workload": f"fused quant+fp8 block-scale GEMM N={N} K={K}, M sweep {list(M_SWEEP)}, "
                               f"{copies} cold weight copies rotated in a HIP graph",
                   "N": N, "K": K, "M": list(M_SWEEP), "weight_copies": copies,
                   "arithmetic": "e4m3 x e4m3 products, fp32 accumulation, bf16 activations in, bf16 out",
                   "calls_per_step": copies * len(M_SWEEP), "parallelism": "single GPU"},
        "sweep": sweep,
        "launch_floor_us": round(floor_us, 3),
        "read_floor_us": round(read_floor_us, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "configs": configs,
        "gpu": torch.cuda.get_device_name(0),
        "hip": torch.version.hip,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(N, K, target_s):
    """The oracle as it stands, on the host cores: quant + GEMM of the M sweep on weight copy 0,
    restricted to a column window sized to roughly `target_s` seconds per leg."""
    import numpy as np

    import oracle
    import synthgen

    cores = len(os.sched_getaffinity(0))
    t0 = time.time()
    w8, sw = oracle.quant_weight(synthgen.gen_w(N, K, seed=0, copy=0))
    log(f"[bench] oracle weight quant (untimed) {time.time() - t0:.1f}s")
    xs = {M: synthgen.gen_x(M, K, seed=0) for M in M_SWEEP}

    def run(ncols, threads):
        t = time.perf_counter()
        for M in M_SWEEP:
            oracle.quant_gemm(xs[M], w8, sw, n0=0, n1=ncols, threads=threads)
        return time.perf_counter() - t

    def sample_bytes(ncols):
        return sum(ncols * K + 4 * ((ncols + 127) // 128) * (K // 128) + 2 * M * K + 2 * M * ncols
                   for M in M_SWEEP)

    legs = {}
    for name, threads in (("all_cores", cores), ("single_thread", 1)):
        probe = 128
        tp = run(probe, threads)
        ncols = int(min(N, max(128, probe * (target_s / 3) / max(tp, 1e-3))) // 128 * 128)
        t = float(np.median([run(ncols, threads) for _ in range(3)]))
        legs[name] = {"GB_s": sample_bytes(ncols) / t / 1e9, "cols": ncols, "seconds": t, "threads": threads}
        log(f"[bench] oracle {name}: {ncols} columns, {t:.2f}s, {legs[name]['GB_s']:.4f} GB/s")
    model = ""
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True).stdout.splitlines():
            if line.startswith("Model name"):
                model = line.split(":", 1)[1].strip()
    except OSError:
        model = platform.processor()
    a = legs["all_cores"]
    return {"value": round(a["GB_s"], 5), "unit": "GB/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"quant+GEMM of the M sweep {list(M_SWEEP)} on weight copy 0, output columns "
                      f"[0, {a['cols']}) of {N} (algorithmic bytes of that window), median of runs",
            "single_thread": {"value": round(legs["single_thread"]["GB_s"], 5), "cores": 1,
                              "sample": f"output columns [0, {legs['single_thread']['cols']})"},
            "cpu_model": model}


if __name__ == "__main__":
    main()
