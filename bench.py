"""Benchmark of the block-quantized linear layer on one MI355X.

Headline step: one decode step of a quantized projection -- the fused
dequant-GEMV of a Q4K weight at the FFN up-projection shape (N = 14336,
K = 4096, M = 1 token), weights already quantized (ISQ) and resident in HBM.
`value` is quantized-weight GB/s: weight bytes per step / time per step.
Each step reads a different copy of the weights (enough copies to exceed
twice the 256 MiB Infinity Cache), so the bytes come from HBM.  Launches are
captured in a HIP graph (kernels are warmed before capture) so that host
launch cost does not enter a 4-microsecond kernel's time.

The same run also measures, as "parts": the Q8_0 variant of the headline
GEMV, batched decode (M = 4/16/64, K = 14336, N = 4096, Q4K with outliers),
prefill (M = 2048, K = 4096, N = 14336, Q8_0 weights) on the bf16 MFMA and
the int8 MFMA paths, ISQ of a 32-layer decoder to Q4K plus its 131072 x 5120
output head to Q6K, the output head GEMV at M = 1 and 8, and the equivalent
decode tokens/s of that decoder (all 224 projection GEMVs plus the head).
Parity with the CPU oracle is checked in the same run before timing.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0     # dense MFMA bf16, published
INT8_PEAK_TOPS = 5000.0       # dense MFMA int8, published
FP8_PEAK_TFLOPS = 5000.0      # dense MFMA fp8, published
MALL_BYTES = 256 << 20        # Infinity Cache


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--parts", default=None,
                    help="comma-separated parts measured after the headline: batched, glu, formats, fp8, prefill, isq "
                         "(default: all of them, none with --quick)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a buffer of BYTES bytes 10 times (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemv_q4k_14336x4096_m1_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "ggml_block_quant_amd", "csrc", f) for f in ("gemv.hip", "qlinear_internal.h")]


def measured_traffic():
    """HBM bytes per launch of the headline GEMV from the committed FETCH_SIZE /
    WRITE_SIZE counter record, scaled by the copy-probe factors it states; None
    when there is no record or the kernel's sources changed since it was taken."""
    import hashlib

    try:
        rec = {}
        for line in open(TRAFFIC_RECORD):
            if line.startswith("traffic_"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            h.update(open(f, "rb").read())
        if h.hexdigest() != rec["traffic_source_sha256"]:
            return None
        kib = (float(rec["traffic_fetch_kib_per_dispatch"]) * float(rec["traffic_fetch_scale"])
               + float(rec["traffic_write_kib_per_dispatch"]) * float(rec["traffic_write_scale"]))
        return int(round(kib * 1024))
    except (OSError, KeyError, ValueError):
        return None


def copies_for(nbytes: int) -> int:
    return max(2, math.ceil(2 * MALL_BYTES / nbytes))


class Timer:
    """HIP events on the current stream (the stream every launch uses)."""

    def __init__(self, torch):
        self.t = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.t.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.t.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def graph_of(torch, launch, n):
    """Capture n calls launch(i) in one HIP graph (after eager warm-up)."""
    launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                launch(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, calls_per_replay, warm_s=0.1):
    """Average time per call over `reps` replays, after replaying for at
    least `warm_s` seconds (the GPU clocks settle under sustained load)."""
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < warm_s:
        g.replay()
        torch.cuda.synchronize()
    with Timer(torch) as t:
        for _ in range(reps):
            g.replay()
    return t.ms / (reps * calls_per_replay)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(sharding is described in the design notes, not built). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import ggml_block_quant_amd as ql
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ql.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        a = torch.ones(args.copy_probe // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 10}))
        return
    result = {}

    def bf16_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------------
    # headline: Q4K GEMV, N=14336, K=4096, M=1, cold weights
    # ------------------------------------------------------------------
    N, K, M = 14336, 4096, 1
    log("headline: generating 14336x4096 weights and quantizing")
    w = synth.weights_bf16(synth.seed_for(2, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(2, 1), M, K)
    W = bf16_dev(w)
    X = bf16_dev(x)
    parts = {}
    head = {}
    for fmt in ("q4k", "q8_0"):
        blocks = ql.isq(fmt, W)
        nb = blocks.numel()
        R = copies_for(nb)
        copies = [blocks] + [blocks.clone() for _ in range(R - 1)]
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        # parity on the live buffers (oracle on 256 sampled rows)
        parity = check_gemv_parity(ql, fmt, w, x, blocks, Y, N)

        def launch(i, fmt=fmt, copies=copies, Y=Y):
            ql.qmatmul(fmt, copies[i % len(copies)], X, N, out=Y)

        steps = args.steps
        for i in range(args.warmup):
            launch(i)
        g = graph_of(torch, launch, steps)
        torch.cuda.synchronize()
        # the replay must reproduce the eager result (checked before timing)
        y_eager = Y.clone()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, y_eager), "graph replay differs from eager launch"
        ms = time_graph(torch, g, 1, steps)   # exactly `steps` launches timed
        ms_rep = time_graph(torch, g, 5, steps)
        wbytes = nb
        alg = nb + M * K * 2 + M * N * 4
        head[fmt] = dict(ms=ms, ms_5reps=ms_rep, weight_bytes=wbytes, alg_bytes=alg, copies=R,
                         weight_GBps=wbytes / (ms * 1e-3) / 1e9, alg_GBps=alg / (ms * 1e-3) / 1e9,
                         parity_max_err=parity)
        log(f"  {fmt} GEMV: {ms * 1e3:.2f} us/launch  {head[fmt]['weight_GBps']:.0f} GB/s weights  "
            f"(max err {parity:.1e}, {R} copies)")
        del copies, g, blocks
        torch.cuda.empty_cache()

    q4 = head["q4k"]
    result.update({
        "metric": "quantized GEMV weight GB/s (% HBM peak) + prefill qGEMM TOPS (% MFMA peak)",
        "value": round(q4["weight_GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": q4["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "q4k_decode_gemv", "N": N, "K": K, "M": M, "weights": "N(0,0.02) bf16 -> Q4K",
                   "activations": "N(0,1) bf16", "weight_copies_rotated": q4["copies"],
                   "launch": "HIP graph of `steps` launches"},
        "roofline": {"bound": "hbm", "achieved": round(q4["alg_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(q4["alg_GBps"] / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
                     "kernel": "gemv_lds_kernel<Q4K, M=1, CPT=2, R=2>", "alg_bytes_per_launch": q4["alg_bytes"]},
    })
    parts["gemv_q8_0_14336x4096_m1"] = {
        "us": round(head["q8_0"]["ms"] * 1e3, 3), "weight_GBps": round(head["q8_0"]["weight_GBps"], 1),
        "hbm_frac": round(head["q8_0"]["alg_GBps"] / HBM_PEAK_GBPS, 4), "parity_max_err": head["q8_0"]["parity_max_err"]}
    parts["gemv_q4k_14336x4096_m1"] = {
        "us": round(q4["ms"] * 1e3, 3), "weight_GBps": round(q4["weight_GBps"], 1),
        "hbm_frac": round(q4["alg_GBps"] / HBM_PEAK_GBPS, 4), "parity_max_err": q4["parity_max_err"]}
    del W

    which = set(args.parts.split(",")) if args.parts else (set() if args.quick else
                                                           {"batched", "glu", "formats", "fp8", "prefill", "isq"})
    if which:
        parts.update(bench_parts(torch, ql, synth, dev, bf16_dev, which))
    result["parts"] = parts
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(result), flush=True)


def check_gemv_parity(ql, fmt, w, x, blocks, Y, N):
    import torch

    import oracle

    ql.qmatmul(fmt, blocks, torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(blocks.device), N, out=Y)
    y = Y.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(1))
    rows = np.sort(rng.choice(N, 256, replace=False))
    K = w.shape[1]
    got = oracle.rows_of_buffer(fmt, blocks.cpu().numpy(), N, K, rows)
    f = oracle.quantize(fmt, w[rows])
    if not np.array_equal(got, oracle.pack(fmt, f, len(rows), K)):
        raise SystemExit(f"parity failure: {fmt} ISQ bytes differ from the oracle")
    Yr, den = oracle.matmul_a16(oracle.dequant(fmt, f, len(rows), K), x)
    e = oracle.normalized_error(y[:, rows], Yr, den).max()
    if e > 1e-3:
        raise SystemExit(f"parity failure: {fmt} GEMV error {e:.3e}")
    return float(e)


def bench_parts(torch, ql, synth, dev, bf16_dev, which):
    parts = {}

    def timed_calls(launch, n_calls, reps=3):
        for i in range(3):
            launch(i)
        g = graph_of(torch, launch, n_calls)
        return time_graph(torch, g, reps, n_calls)

    if "batched" in which:
        # batched decode: K=14336, N=4096, Q4K with outliers, M = 4, 16, 64
        log("batched decode 4096x14336 q4k")
        N, K = 4096, 14336
        w = synth.weights_bf16(synth.seed_for(3, 0), N, K, outliers=True)
        xs = synth.activations_bf16(synth.seed_for(3, 1), 64, K)
        blocks = ql.isq("q4k", bf16_dev(w))
        R = copies_for(blocks.numel())
        copies = [blocks] + [blocks.clone() for _ in range(R - 1)]
        for M in (4, 16, 64):
            X = bf16_dev(xs[:M])
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ms = timed_calls(lambda i: ql.qmatmul("q4k", copies[i % R], X, N, out=Y), 4 * R)
            fl = 2.0 * M * N * K
            parts[f"batched_q4k_m{M}"] = {
                "us": round(ms * 1e3, 3), "path": "gemv" if M <= 2 else "mfma_bf16",
                "weight_GBps": round(blocks.numel() / ms / 1e6, 1),
                "hbm_frac": round((blocks.numel() + M * K * 2 + M * N * 4) / ms / 1e6 / HBM_PEAK_GBPS, 4),
                "TFLOPs": round(fl / ms / 1e9, 2)}
            log(f"  M={M}: {ms * 1e3:.2f} us")
        # GEMV / MFMA crossover at this shape (sets the AUTO dispatch)
        cross = {}
        for M in range(1, 9):
            X = bf16_dev(xs[:M])
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            row = {}
            for path in ("gemv", "mfma_bf16"):
                ms = timed_calls(lambda i: ql.qmatmul("q4k", copies[i % R], X, N, out=Y, path=path), 2 * R)
                row[path] = round(ms * 1e3, 2)
            cross[str(M)] = row
        parts["crossover_q4k_4096x14336_us"] = cross
        log(f"  crossover: {cross}")
        del copies, blocks
        torch.cuda.empty_cache()

    if "glu" in which:
        # gated FFN projection, 14336 x 4096 gate and up (Q4K): one fused launch
        # against the two GEMVs it replaces (their outputs alone, no product)
        log("gated FFN 14336x4096 q4k: fused gate/up + SiLU vs two GEMVs")
        F, K = 14336, 4096
        wg = bf16_dev(synth.weights_bf16(synth.seed_for(2, 0), F, K))
        wu = synth.device_normal_bf16(9501, (F, K), synth.W_SIGMA)
        bg, bu = ql.isq("q4k", wg), ql.isq("q4k", wu)
        R = copies_for(2 * bg.numel())
        cg = [bg] + [bg.clone() for _ in range(R - 1)]
        cu = [bu] + [bu.clone() for _ in range(R - 1)]
        xs = synth.activations_bf16(synth.seed_for(2, 1), 2, K)
        for M in (1, 2):
            X = bf16_dev(xs[:M])
            H = torch.empty((M, F), dtype=torch.float32, device=dev)
            Y2 = torch.empty((M, F), dtype=torch.float32, device=dev)
            fused = timed_calls(lambda i: ql.qmatmul_glu("q4k", cg[i % R], cu[i % R], X, F, out=H), 2 * R)

            def two(i):
                ql.qmatmul("q4k", cg[i % R], X, F, out=Y2)
                ql.qmatmul("q4k", cu[i % R], X, F, out=H)

            sep = timed_calls(two, 2 * R)
            parts[f"glu_q4k_14336x4096_m{M}"] = {
                "fused_us": round(fused * 1e3, 2), "two_gemvs_us": round(sep * 1e3, 2),
                "fused_weight_GBps": round(2 * bg.numel() / fused / 1e6, 1),
                "hbm_frac": round(2 * bg.numel() / fused / 1e6 / HBM_PEAK_GBPS, 4)}
            log(f"  M={M}: fused {fused * 1e3:.2f} us, two GEMVs {sep * 1e3:.2f} us")
        del cg, cu, bg, bu, wg, wu
        torch.cuda.empty_cache()

    if "formats" in which:
        # the further formats on the generic kernels, at the 14336 x 4096 shape:
        # ISQ, one-token GEMV and a 16-token batch
        log("further formats 14336x4096: ISQ, GEMV M=1, MFMA M=16")
        N, K = 14336, 4096
        W = bf16_dev(synth.weights_bf16(synth.seed_for(2, 0), N, K))
        xs = bf16_dev(synth.activations_bf16(synth.seed_for(2, 1), 16, K))
        rows = {}
        for fmt in ("q5k", "q3k", "q2k", "q4_0", "q4_1", "q5_0", "q5_1"):
            blocks = ql.isq(fmt, W)
            nb = blocks.numel()
            R = copies_for(nb)
            copies = [blocks] + [blocks.clone() for _ in range(R - 1)]
            out = torch.empty_like(blocks)
            isq_ms = timed_calls(lambda i: ql.isq(fmt, W, out=out), 10)
            Y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
            g1 = timed_calls(lambda i: ql.qmatmul(fmt, copies[i % R], xs[:1], N, out=Y1), 2 * R)
            Y16 = torch.empty((16, N), dtype=torch.float32, device=dev)
            g16 = timed_calls(lambda i: ql.qmatmul(fmt, copies[i % R], xs, N, out=Y16), 2 * R)
            rows[fmt] = {"bytes": nb, "isq_us": round(isq_ms * 1e3, 1),
                         "isq_GBps": round((W.numel() * 2 + nb) / isq_ms / 1e6, 1),
                         "gemv_m1_us": round(g1 * 1e3, 2), "gemv_m1_weight_GBps": round(nb / g1 / 1e6, 1),
                         "m16_us": round(g16 * 1e3, 2), "m16_weight_GBps": round(nb / g16 / 1e6, 1)}
            log(f"  {fmt}: ISQ {isq_ms * 1e3:.0f} us, GEMV M=1 {g1 * 1e3:.2f} us ({nb / g1 / 1e6:.0f} GB/s), "
                f"M=16 {g16 * 1e3:.2f} us")
            del copies, blocks, out
        parts["further_formats_14336x4096"] = rows
        del W, xs
        torch.cuda.empty_cache()

    if "fp8" in which:
        # FP8 E4M3 with per-row scales: ISQ and W8A16 GEMV at 14336 x 4096, and
        # dynamic per-token W8A8 at the prefill shape on the FP8 MFMA path
        log("fp8: ISQ + W8A16 GEMV 14336x4096, W8A8 prefill 2048x4096x14336")
        N, K = 14336, 4096
        W = bf16_dev(synth.weights_bf16(synth.seed_for(4, 0), N, K))
        b8 = ql.isq("fp8", W)
        out = torch.empty_like(b8)
        isq_ms = timed_calls(lambda i: ql.isq("fp8", W, out=out), 10)
        R = copies_for(b8.numel())
        copies = [b8] + [b8.clone() for _ in range(R - 1)]
        x1 = bf16_dev(synth.activations_bf16(synth.seed_for(2, 1), 1, K))
        Y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        g1 = timed_calls(lambda i: ql.qmatmul("fp8", copies[i % R], x1, N, out=Y1), 2 * R)
        M = 2048
        X = bf16_dev(synth.activations_bf16(synth.seed_for(4, 1), M, K))
        ws = torch.empty(ql.workspace_bytes("fp8", "mfma_fp8", M, K), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        fl = 2.0 * M * N * K
        pf = timed_calls(lambda i: ql.qmatmul("fp8", copies[i % 2], X, N, out=Y, path="mfma_fp8", workspace=ws), 10)
        parts["fp8_e4m3_14336x4096"] = {
            "isq_us": round(isq_ms * 1e3, 1), "isq_GBps": round((W.numel() * 2 + b8.numel()) / isq_ms / 1e6, 1),
            "w8a16_gemv_m1_us": round(g1 * 1e3, 2), "w8a16_gemv_weight_GBps": round(b8.numel() / g1 / 1e6, 1),
            "w8a8_prefill_m2048_us": round(pf * 1e3, 1), "w8a8_TOPs": round(fl / pf / 1e9, 1),
            "w8a8_mfma_frac": round(fl / pf / 1e9 / FP8_PEAK_TFLOPS, 4),
            "includes": "per-token activation quantization"}
        log(f"  ISQ {isq_ms * 1e3:.0f} us, W8A16 GEMV M=1 {g1 * 1e3:.2f} us ({b8.numel() / g1 / 1e6:.0f} GB/s), "
            f"W8A8 prefill {pf * 1e3:.0f} us {fl / pf / 1e9:.0f} TFLOP/s")
        del copies, b8, out, W, X, ws, Y
        torch.cuda.empty_cache()

    if "prefill" in which:
        # prefill: M=2048, K=4096, N=14336, Q8_0; bf16 MFMA path and int8 path
        log("prefill 2048x4096x14336 q8_0")
        M, N, K = 2048, 14336, 4096
        w = synth.weights_bf16(synth.seed_for(4, 0), N, K)
        X = bf16_dev(synth.activations_bf16(synth.seed_for(4, 1), M, K))
        blocks = ql.isq("q8_0", bf16_dev(w))
        copies = [blocks, blocks.clone()]
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = torch.empty(ql.workspace_bytes("q8_0", "mfma_i8", M, K), dtype=torch.uint8, device=dev)
        fl = 2.0 * M * N * K
        ms = timed_calls(lambda i: ql.qmatmul("q8_0", copies[i % 2], X, N, out=Y, path="mfma_bf16"), 10)
        parts["prefill_q8_0_bf16_mfma"] = {"us": round(ms * 1e3, 2), "TFLOPs": round(fl / ms / 1e9, 1),
                                           "mfma_frac": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
        log(f"  bf16 path: {ms * 1e3:.1f} us {fl / ms / 1e9:.0f} TFLOP/s")
        ms = timed_calls(lambda i: ql.qmatmul("q8_0", copies[i % 2], X, N, out=Y, path="mfma_i8", workspace=ws), 10)
        parts["prefill_q8_0_int8_mfma"] = {"us": round(ms * 1e3, 2), "TOPs": round(fl / ms / 1e9, 1),
                                           "mfma_frac": round(fl / ms / 1e9 / INT8_PEAK_TOPS, 4),
                                           "includes": "activation quantization"}
        log(f"  int8 path: {ms * 1e3:.1f} us {fl / ms / 1e9:.0f} TOP/s")
        del copies, blocks, ws, Y, X
        torch.cuda.empty_cache()

    if "isq" in which:
        # ISQ of the 32-layer decoder (Q4K) and the output head (Q6K)
        log("decoder ISQ: 32 layers x 7 projections to q4k + 131072x5120 head to q6k")
        shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096),
                  (4096, 14336)]
        Wl, Bl = [], []
        read = write = 0
        for layer in range(32):
            for kind, (n, k) in enumerate(shapes):
                Wt = synth.device_normal_bf16(synth.decoder_seed(layer, kind), (n, k), synth.W_SIGMA)
                Wl.append(Wt)
                Bl.append(torch.empty(ql.blocks_bytes("q4k", n, k), dtype=torch.uint8, device=dev))
        Wh = synth.device_normal_bf16(synth.LM_HEAD_W_SEED, (131072, 5120), synth.W_SIGMA)
        Bh = torch.empty(ql.blocks_bytes("q6k", 131072, 5120), dtype=torch.uint8, device=dev)
        for Wt, Bt in zip(Wl, Bl):
            read += Wt.numel() * 2
            write += Bt.numel()
        read += Wh.numel() * 2
        write += Bh.numel()

        def isq_all():
            for Wt, Bt in zip(Wl, Bl):
                ql.isq("q4k", Wt, out=Bt)
            ql.isq("q6k", Wh, out=Bh)

        isq_all()
        torch.cuda.synchronize()
        with Timer(torch) as t:
            isq_all()
        parts["isq_decoder_32l_q4k_plus_head_q6k"] = {
            "ms": round(t.ms, 3), "read_bytes": read, "write_bytes": write,
            "GBps": round((read + write) / t.ms / 1e6, 1),
            "hbm_frac": round((read + write) / t.ms / 1e6 / HBM_PEAK_GBPS, 4)}
        log(f"  ISQ all: {t.ms:.2f} ms ({(read + write) / t.ms / 1e6:.0f} GB/s)")
        del Wl, Wh
        torch.cuda.empty_cache()

        # output head GEMV, M = 1 and M = 8 (Q6K)
        xh = synth.activations_bf16(synth.LM_HEAD_X_SEED, 8, 5120)
        Bh2 = [Bh, Bh.clone()]
        for M in (1, 8):
            X = bf16_dev(xh[:M])
            Y = torch.empty((M, 131072), dtype=torch.float32, device=dev)
            ms = timed_calls(lambda i: ql.qmatmul("q6k", Bh2[i % 2], X, 131072, out=Y), 8)
            parts[f"lm_head_q6k_m{M}"] = {"us": round(ms * 1e3, 2), "weight_GBps": round(Bh.numel() / ms / 1e6, 1),
                                          "hbm_frac": round((Bh.numel() + M * 5120 * 2 + M * 131072 * 4) / ms / 1e6 / HBM_PEAK_GBPS, 4)}
            log(f"  lm_head M={M}: {ms * 1e3:.1f} us")
        del Bh2

        # embedding lookup from the same Q6K table (a tied head): 2048 random ids
        ids = torch.randint(0, 131072, (2048,), generator=torch.Generator().manual_seed(9100),
                            dtype=torch.int32).to(dev)
        E = torch.empty((2048, 5120), dtype=torch.float32, device=dev)
        ms = timed_calls(lambda i: ql.embed("q6k", Bh, 131072, 5120, ids, out=E), 20)
        moved = 2048 * 5120 * 210 // 256 + E.numel() * 4
        parts["embed_q6k_131072x5120_2048ids"] = {"us": round(ms * 1e3, 2), "GBps": round(moved / ms / 1e6, 1),
                                                  "hbm_frac": round(moved / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                                  "bytes": moved, "note": "quantized rows read + fp32 rows written"}
        log(f"  embed 2048 ids: {ms * 1e3:.1f} us ({moved / ms / 1e6:.0f} GB/s)")
        del E

        # equivalent decode tokens/s: every projection GEMV of the 32 layers + head
        x1 = bf16_dev(synth.activations_bf16(9001, 1, 14336))
        Ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for (n, k) in shapes]
        Yh = torch.empty((1, 131072), dtype=torch.float32, device=dev)

        def token(_i):
            for j, Bt in enumerate(Bl):
                n, k = shapes[j % 7]
                ql.qmatmul("q4k", Bt, x1[:, :k], n, out=Ys[j % 7])
            ql.qmatmul("q6k", Bh, x1[:, :5120], 131072, out=Yh)

        token(0)
        g = graph_of(torch, token, 1)
        ms = time_graph(torch, g, 10, 1)
        total = sum(b.numel() for b in Bl) + Bh.numel()
        parts["equiv_decode_tok_s"] = {"tok_s": round(1000.0 / ms, 1), "ms_per_token": round(ms, 4),
                                       "weight_bytes_per_token": total,
                                       "weight_GBps": round(total / ms / 1e6, 1),
                                       "note": "225 quantized GEMVs per token (M=1); attention, norms, sampling excluded"}
        log(f"  decode token: {ms:.3f} ms -> {1000 / ms:.0f} tok/s")

        # the same token with each layer's gate and up projections fused with
        # SiLU * up into one launch (qmatmul_glu)
        Hf = torch.empty((1, 14336), dtype=torch.float32, device=dev)

        def token_fused(_i):
            for layer in range(32):
                for j in (0, 1, 2, 3, 6):
                    n, k = shapes[j]
                    ql.qmatmul("q4k", Bl[7 * layer + j], x1[:, :k], n, out=Ys[j])
                ql.qmatmul_glu("q4k", Bl[7 * layer + 4], Bl[7 * layer + 5], x1[:, :4096], 14336, out=Hf)
            ql.qmatmul("q6k", Bh, x1[:, :5120], 131072, out=Yh)

        token_fused(0)
        g = graph_of(torch, token_fused, 1)
        ms = time_graph(torch, g, 10, 1)
        parts["equiv_decode_tok_s_fused_ffn"] = {
            "tok_s": round(1000.0 / ms, 1), "ms_per_token": round(ms, 4), "weight_GBps": round(total / ms / 1e6, 1),
            "note": "per layer q, k, v, o, down GEMVs + one fused gate/up SiLU launch (193 launches per token)"}
        log(f"  decode token, fused gate/up: {ms:.3f} ms -> {1000 / ms:.0f} tok/s")
    return parts


def _oracle_gemv_rate(w, x, seconds):
    """GB/s of quantized weights through the oracle's GEMV (unpack + exact
    dequant + fp64 matmul) over whole matrices, repeated for `seconds`."""
    import oracle

    N, K = w.shape
    f = oracle.quantize("q4k", w)
    buf = oracle.pack("q4k", f, N, K)
    reps, t0 = 0, time.perf_counter()
    while True:
        g = oracle.unpack("q4k", buf, N, K)
        Wd = oracle.dequant("q4k", g, N, K)
        oracle.matmul_a16(Wd, x)
        reps += 1
        el = time.perf_counter() - t0
        if el > seconds or reps >= 1000:
            break
    return buf.size * reps / el / 1e9, reps, el


_ONE_CORE = """
import sys, json, numpy as np
sys.path.insert(0, {root!r})
import bench
d = np.load({path!r})
r, reps, el = bench._oracle_gemv_rate(d["w"], d["x"], 8.0)
print(json.dumps({{"value": round(r, 3), "reps": reps, "el": el}}))
"""


def cpu_baseline(w, x):
    """The oracle's quantized GEMV on the host cores, over whole 14336x4096
    Q4K matrices, repeated for ~12 s; then the same on one core in a child
    process whose thread counts are pinned to 1 (the child never touches the
    GPU)."""
    import subprocess
    import tempfile

    rate, reps, el = _oracle_gemv_rate(w, x, 12.0)
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    out = {"value": round(rate, 3), "unit": "GB/s", "cores": min(cores, threads), "kind": "oracle",
           "sample": f"{reps} full {w.shape[0]}x{w.shape[1]} Q4K GEMVs (M=1): unpack + fp64 dequant + fp64 matmul, "
                     f"{el:.1f} s"}
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "wx.npz")
        np.savez(path, w=w, x=x)
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
                   HIP_VISIBLE_DEVICES="")
        res = subprocess.run([sys.executable, "-c", _ONE_CORE.format(root=ROOT, path=path)], env=env,
                             capture_output=True, text=True, timeout=300)
    if res.returncode == 0 and res.stdout.strip():
        one = json.loads(res.stdout.strip().splitlines()[-1])
        out["one_core"] = {"value": one["value"], "unit": "GB/s", "cores": 1,
                           "sample": f"{one['reps']} full {w.shape[0]}x{w.shape[1]} Q4K GEMVs (M=1), {one['el']:.1f} s"}
    else:
        out["one_core"] = {"value": None, "error": (res.stderr or "no output")[-300:]}
    return out


if __name__ == "__main__":
    main()
