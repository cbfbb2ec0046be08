"""Benchmark of the block-quantized linear layer on one MI355X.

Headline (the largest configuration): the quantized GEMV of the output head of
a 32-layer decoder -- a 131072 x 5120 weight, promoted from the model's Q4K to
Q6K by the sensitive-tensor policy (page "Quantization types", section
"Sensitive tensor precision") -- for one token, after ISQ of the whole
decoder to Q4K and of the head to Q6K.  One step is one launch of that GEMV
with its blocks resident in HBM; two copies alternate, and at 550 MB each is
larger than the 256 MiB Infinity Cache, so every step streams its weights
from HBM.  value = weight bytes per step / time per step (GB/s).

The same run measures, each with its own roofline block:
  * the Q8_0 GEMV 1024 x 1024 (latency; cache-resident), the Q4K and Q8_0
    GEMVs at 14336 x 4096 (one token);
  * batched decode, Q4K 4096 x 14336 with 1 % outliers, 4 / 16 / 64 tokens;
  * prefill 2048 x 4096 x 14336 with Q8_0 weights on the bf16 MFMA path and
    on the int8 path (activation quantization included), and FP8 W8A8 at the
    same shape;
  * ISQ of the whole decoder and head; the head GEMV for eight tokens;
  * the further formats and FP8 at 14336 x 4096 (ISQ, one-token GEMV,
    16-token MFMA path);
  * equivalent decode tokens/s of the decoder (every projection GEMV of the
    32 layers plus the head, with q/k/v as one concatenated launch and
    gate/up as one fused SiLU launch);
  * two ceilings: a streaming read of a buffer read once per launch, and an
    MFMA-only loop.
Timing (page "Quantization types", section "NVFP4": kernels warmed up before
graph capture, outputs checked, median latency reported): parity with the
CPU oracle first (codes bit-exact, outputs within 1e-3 of sum |w||x| on
sampled outputs); W untimed launches; then a HIP graph of the launches,
replayed at least 10 times, each replay timed with HIP events on the stream
the launches go to; median, p10 and p90 per launch.  The oracle is also
timed on the host cores (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R]
                       [--parts list] [--quick] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
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

HEAD_N, HEAD_K = 131072, 5120
DECODER_SHAPES = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096),
                  (4096, 14336)]  # q, k, v, o, gate, up, down: [out][in]
ALL_PARTS = ("gemv", "batched", "prefill", "model", "ceilings", "crossover", "glu", "formats")

TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemv_q6k_131072x5120_m1_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "ggml_block_quant_amd", "csrc", f) for f in ("gemv.hip", "qlinear_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="launches per timed graph replay (headline)")
    ap.add_argument("--warmup", type=int, default=5, help="untimed launches before capture")
    ap.add_argument("--reps", type=int, default=10, help="timed replays (at least 10)")
    ap.add_argument("--parts", default=None, help="comma-separated: " + ",".join(ALL_PARTS) + " (default: all)")
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a buffer of BYTES bytes 10 times (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters), then exit")
    a = ap.parse_args()
    a.reps = max(10, a.reps)
    return a


def measured_traffic():
    """HBM bytes per launch of the headline GEMV from the committed FETCH_SIZE /
    WRITE_SIZE counter record, scaled by the copy-probe factors it states; None
    when there is no record or the kernel's sources changed since it was taken."""
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
    """Distinct weight copies rotated so that each launch reads HBM, not the
    Infinity Cache (twice its size in total)."""
    return max(2, math.ceil(2 * MALL_BYTES / nbytes))


def stats(per_launch_ms):
    a = np.sort(np.asarray(per_launch_ms, np.float64))
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


class Runner:
    """Graph capture and timed replays on the current stream."""

    def __init__(self, torch, reps):
        self.t = torch
        self.reps = reps

    def graph(self, launch, n):
        torch = self.t
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

    def time(self, launch, n, warmup=3, settle_s=0.1):
        """Per-launch times (ms) of `reps` replays of a graph of n launches,
        after `warmup` eager launches and replays for `settle_s` seconds."""
        torch = self.t
        for i in range(warmup):
            launch(i)
        g = self.graph(launch, n)
        t0 = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > settle_s:
                break
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(self.reps)]
        s = torch.cuda.current_stream()
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(s)
            g.replay()
            b.record(s)
        torch.cuda.synchronize()
        return stats([a.elapsed_time(b) / n for a, b in evs])


def roof(bound, units, t, peak, unit, kernel, traffic=None, note=None):
    """Roofline block: `units` algorithmic bytes (GB/s) or FLOP/OP (TFLOP/s)
    per launch over the median launch time (ms)."""
    scale = 1e6 if unit == "GB/s" else 1e9
    ach = units / t["median"] / scale
    d = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
         "traffic": traffic, "kernel": kernel,
         ("alg_bytes_per_launch" if unit == "GB/s" else "alg_ops_per_launch"): int(units),
         "us_median": round(t["median"] * 1e3, 3), "us_p10": round(t["p10"] * 1e3, 3),
         "us_p90": round(t["p90"] * 1e3, 3), "replays": t["n"]}
    if note:
        d["note"] = note
    return d


def sample_rows(N, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, count), replace=False)]))


def check_gemv_rows(ql, fmt, w_rows, rows, blocks, N, K, x, y, label, isq_exact=True):
    """ISQ bytes of the sampled rows bit-exact and outputs within the bar."""
    import oracle

    f = oracle.quantize(fmt, w_rows)
    if isq_exact:
        got = oracle.rows_of_buffer(fmt, blocks.cpu().numpy(), N, K, rows)
        if not np.array_equal(got, oracle.pack(fmt, f, len(rows), K)):
            raise SystemExit(f"parity failure: {label}: ISQ bytes differ from the oracle")
    Yr, den = oracle.matmul_a16(oracle.dequant(fmt, f, len(rows), K), x)
    e = float(oracle.normalized_error(y[:, rows], Yr, den).max())
    if e > 1e-3:
        raise SystemExit(f"parity failure: {label}: error {e:.3e}")
    return e


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (how it would shard is "
              "described in the design notes, not built).  Run with --gpus 1.", file=sys.stderr)
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
    run = Runner(torch, args.reps)

    def bf16_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def host_rows(W, rows):
        return W[torch.from_numpy(rows).to(dev)].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    # ------------------------------------------------------------------
    # headline: the Q6K head GEMV, M = 1
    # ------------------------------------------------------------------
    log(f"headline: head {HEAD_N}x{HEAD_K} to q6k, GEMV M=1")
    Wh = synth.device_normal_bf16(synth.LM_HEAD_W_SEED, (HEAD_N, HEAD_K), synth.W_SIGMA)
    Bh = ql.isq("q6k", Wh)
    xh = synth.activations_bf16(synth.LM_HEAD_X_SEED, 8, HEAD_K)
    Xh = bf16_dev(xh)
    rows = sample_rows(HEAD_N, 256, 12)
    wrows = host_rows(Wh, rows)
    Y1 = torch.empty((1, HEAD_N), dtype=torch.float32, device=dev)
    ql.qmatmul("q6k", Bh, Xh[:1], HEAD_N, out=Y1)
    err_head = check_gemv_rows(ql, "q6k", wrows, rows, Bh, HEAD_N, HEAD_K, xh[:1], Y1.cpu().numpy(), "head M=1")
    Bh2 = [Bh, Bh.clone()]
    nb_head = Bh.numel()

    def head_launch(i):
        ql.qmatmul("q6k", Bh2[i % 2], Xh[:1], HEAD_N, out=Y1)

    for i in range(args.warmup):
        head_launch(i)
    g = run.graph(head_launch, args.steps)
    y_eager = Y1.clone()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(Y1, y_eager):
        raise SystemExit("parity failure: graph replay of the head GEMV differs from its eager launch")
    # replays until the clocks settle, then the timed region: `reps`
    # replays of exactly `steps` launches each
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        g.replay()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.reps)]
    s = torch.cuda.current_stream()
    for a, b in evs:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    th = stats([a.elapsed_time(b) / args.steps for a, b in evs])
    alg_head = nb_head + HEAD_K * 2 + HEAD_N * 4
    log(f"  head GEMV M=1: median {th['median'] * 1e3:.1f} us (p10 {th['p10'] * 1e3:.1f}, p90 {th['p90'] * 1e3:.1f}); "
        f"{nb_head / th['median'] / 1e6:.0f} GB/s of weights; max err {err_head:.1e}")
    del g

    result = {
        "metric": "quantized GEMV weight GB/s (% HBM peak) + prefill qGEMM TOPS (% MFMA peak)",
        "value": round(nb_head / th["median"] / 1e6, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": th["median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "output head GEMV of the 32-layer decoder (ISQ: layers Q4K, head promoted to Q6K)",
                   "N": HEAD_N, "K": HEAD_K, "M": 1, "format": "q6k", "weight_bytes": nb_head,
                   "weights": "N(0,0.02) bf16 (device generator, seed 5999)", "activations": "N(0,1) bf16",
                   "weight_copies_rotated": 2, "timing": f"{args.reps} replays of a HIP graph of {args.steps} "
                   "launches, HIP events on the launch stream, median per launch",
                   "arithmetic": "exact Q6K codes x fp16-scaled activations, fp32 sums"},
        "roofline": roof("hbm", alg_head, th, HBM_PEAK_GBPS, "GB/s",
                         "gemv_lds_kernel<Q6K, M=1, CPT=3, R=4, FS=160>", traffic=measured_traffic(),
                         note="achieved = (weight bytes + X + Y) per launch / median launch time; traffic = "
                              "FETCH_SIZE + WRITE_SIZE per dispatch scaled by a copy kernel of known size"),
    }
    parts = {"head_q6k_gemv_m1": {"parity_max_err": err_head, **result["roofline"]}}

    which = set() if args.quick else (set(args.parts.split(",")) if args.parts else set(ALL_PARTS))
    if "model" in which:
        parts.update(part_model(torch, ql, synth, run, dev, bf16_dev, host_rows, Wh, Bh2, Xh, xh))
    del Wh
    torch.cuda.empty_cache()
    if "gemv" in which:
        parts.update(part_gemv(torch, ql, synth, run, dev, bf16_dev))
    if "batched" in which:
        parts.update(part_batched(torch, ql, synth, run, dev, bf16_dev))
    if "crossover" in which:
        parts.update(part_crossover(torch, ql, synth, run, dev, bf16_dev))
    if "glu" in which:
        parts.update(part_glu(torch, ql, synth, run, dev, bf16_dev))
    if "prefill" in which:
        parts.update(part_prefill(torch, ql, synth, run, dev, bf16_dev))
    if "formats" in which:
        parts.update(part_formats(torch, ql, synth, run, dev, bf16_dev))
    if "ceilings" in which:
        parts.update(part_ceilings(torch, ql, run, dev))
    result["parts"] = parts
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------
# parts
# ----------------------------------------------------------------------

def part_model(torch, ql, synth, run, dev, bf16_dev, host_rows, Wh, Bh2, Xh, xh):
    """ISQ of the 32-layer decoder (Q4K) and the head (Q6K); the head GEMV for
    eight tokens; equivalent decode tokens/s."""
    import oracle

    parts = {}
    log("model: ISQ of 32 layers x 7 projections (q4k) + head (q6k)")
    Wl, Bl = [], []
    for layer in range(32):
        for kind, (n, k) in enumerate(DECODER_SHAPES):
            Wl.append(synth.device_normal_bf16(synth.decoder_seed(layer, kind), (n, k), synth.W_SIGMA))
            Bl.append(torch.empty(ql.blocks_bytes("q4k", n, k), dtype=torch.uint8, device=dev))
    Bh_out = torch.empty_like(Bh2[0])
    read = sum(w.numel() * 2 for w in Wl) + Wh.numel() * 2
    write = sum(b.numel() for b in Bl) + Bh_out.numel()

    def isq_all(_i):
        for Wt, Bt in zip(Wl, Bl):
            ql.isq("q4k", Wt, out=Bt)
        ql.isq("q6k", Wh, out=Bh_out)

    isq_all(0)
    torch.cuda.synchronize()
    # codes bit-exact: 8 sampled rows of every layer's tensors, 64 rows of the head
    for j in range(len(Wl)):
        n, k = DECODER_SHAPES[j % 7]
        rows = sample_rows(n, 8, 100 + j)
        w_rows = host_rows(Wl[j], rows)
        got = oracle.rows_of_buffer("q4k", Bl[j].cpu().numpy(), n, k, rows)
        if not np.array_equal(got, oracle.pack("q4k", oracle.quantize("q4k", w_rows), len(rows), k)):
            raise SystemExit(f"parity failure: decoder tensor {j} ISQ bytes")
    if not torch.equal(Bh_out, Bh2[0]):
        raise SystemExit("parity failure: head ISQ is not deterministic")
    t = run.time(isq_all, 1, warmup=1)
    parts["isq_decoder_32l_q4k_head_q6k"] = {
        **roof("hbm", read + write, t, HBM_PEAK_GBPS, "GB/s", "isq_q4k_kernel x224 + isq_q6k_kernel",
               note="bf16 read + blocks written, 225 launches per step"),
        "read_bytes": read, "write_bytes": write, "parity": "224 tensors x 8 sampled rows + the head: bit-exact"}
    log(f"  ISQ: {t['median']:.2f} ms ({(read + write) / t['median'] / 1e6:.0f} GB/s)")

    # head GEMV, eight tokens
    Y8 = torch.empty((8, HEAD_N), dtype=torch.float32, device=dev)
    ql.qmatmul("q6k", Bh2[0], Xh, HEAD_N, out=Y8)
    rows = sample_rows(HEAD_N, 128, 13)
    e8 = check_gemv_rows(ql, "q6k", host_rows(Wh, rows), rows, Bh2[0], HEAD_N, HEAD_K, xh, Y8.cpu().numpy(),
                         "head M=8", isq_exact=False)
    t = run.time(lambda i: ql.qmatmul("q6k", Bh2[i % 2], Xh, HEAD_N, out=Y8), 8)
    nb = Bh2[0].numel()
    parts["head_q6k_gemv_m8"] = {**roof("hbm", nb + 8 * HEAD_K * 2 + 8 * HEAD_N * 4, t, HBM_PEAK_GBPS, "GB/s",
                                        "AUTO (8 tokens)"), "parity_max_err": e8}
    log(f"  head GEMV M=8: {t['median'] * 1e3:.1f} us")

    # equivalent decode tokens/s: q/k/v concatenated into one [6144][4096]
    # weight per layer (rows are quantized independently, so its blocks are
    # those of the three tensors), gate/up fused with SiLU, o and down, head
    log("  equivalent decode: building the concatenated q/k/v weights")
    Bqkv = []
    for layer in range(32):
        Wc = torch.cat([Wl[7 * layer], Wl[7 * layer + 1], Wl[7 * layer + 2]], 0)
        Bqkv.append(ql.isq("q4k", Wc))
    del Wc
    x1 = bf16_dev(synth.activations_bf16(9001, 1, 14336))
    Yqkv = torch.empty((1, 6144), dtype=torch.float32, device=dev)
    Yo = torch.empty((1, 4096), dtype=torch.float32, device=dev)
    Hf = torch.empty((1, 14336), dtype=torch.float32, device=dev)
    Yh = torch.empty((1, HEAD_N), dtype=torch.float32, device=dev)
    # parity of the concatenated launch against the oracle (sampled rows over q, k and v)
    ql.qmatmul("q4k", Bqkv[0], x1[:, :4096], 6144, out=Yqkv)
    rows = np.unique(np.concatenate([sample_rows(6144, 64, 14), [4095, 4096, 5119, 5120]]))
    Wc_rows = torch.cat([Wl[0], Wl[1], Wl[2]], 0)
    eq = check_gemv_rows(ql, "q4k", host_rows(Wc_rows, rows), rows, Bqkv[0], 6144, 4096,
                         synth.activations_bf16(9001, 1, 14336)[:, :4096], Yqkv.cpu().numpy(), "qkv concatenated")
    del Wc_rows

    def token(_i):
        for layer in range(32):
            ql.qmatmul("q4k", Bqkv[layer], x1[:, :4096], 6144, out=Yqkv)
            ql.qmatmul("q4k", Bl[7 * layer + 3], x1[:, :4096], 4096, out=Yo)
            ql.qmatmul_glu("q4k", Bl[7 * layer + 4], Bl[7 * layer + 5], x1[:, :4096], 14336, out=Hf)
            ql.qmatmul("q4k", Bl[7 * layer + 6], x1[:, :14336], 4096, out=Yo)
        ql.qmatmul("q6k", Bh2[0], x1[:, :HEAD_K], HEAD_N, out=Yh)

    total = sum(b.numel() for b in Bl) + nb
    t = run.time(token, 1, warmup=1)
    parts["equiv_decode_tok_s"] = {
        "tok_s": round(1.0 / (t["median"] * 1e-3), 1), **roof("hbm", total, t, HBM_PEAK_GBPS, "GB/s",
                                                              "129 launches per token"),
        "qkv_parity_max_err": eq,
        "note": "per layer: q/k/v as one concatenated GEMV, o, gate/up fused with SiLU, down; then the Q6K head; "
                "attention, norms and sampling excluded; bound 1,787 tok/s at 8 TB/s"}
    log(f"  decode token: {t['median']:.3f} ms -> {1.0 / (t['median'] * 1e-3):.0f} tok/s")

    def token_plain(_i):
        for j, Bt in enumerate(Bl):
            n, k = DECODER_SHAPES[j % 7]
            ql.qmatmul("q4k", Bt, x1[:, :k], n, out=Yo if n == 4096 else Hf if n == 14336 else Yqkv[:, :n])
        ql.qmatmul("q6k", Bh2[0], x1[:, :HEAD_K], HEAD_N, out=Yh)

    t = run.time(token_plain, 1, warmup=1)
    parts["equiv_decode_tok_s_unfused"] = {
        "tok_s": round(1.0 / (t["median"] * 1e-3), 1), "ms_per_token": round(t["median"], 4),
        "note": "225 separate GEMV launches per token"}
    log(f"  decode token, 225 launches: {t['median']:.3f} ms")
    del Wl, Bl, Bqkv
    torch.cuda.empty_cache()
    return parts


def part_gemv(torch, ql, synth, run, dev, bf16_dev):
    """One-token GEMVs: Q8_0 1024 x 1024 (latency) and 14336 x 4096 Q4K / Q8_0."""
    parts = {}
    N, K = 1024, 1024
    w = synth.weights_bf16(synth.seed_for(1, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(1, 1), 1, K)
    B = ql.isq("q8_0", bf16_dev(w))
    X = bf16_dev(x)
    Y = torch.empty((1, N), dtype=torch.float32, device=dev)
    ql.qmatmul("q8_0", B, X, N, out=Y)
    rows = np.arange(N)
    e = check_gemv_rows(ql, "q8_0", w, rows, B, N, K, x, Y.cpu().numpy(), "q8_0 1024")
    hot = run.time(lambda i: ql.qmatmul("q8_0", B, X, N, out=Y), 100)
    R = copies_for(B.numel())
    cp = [B] + [B.clone() for _ in range(R - 1)]
    cold = run.time(lambda i: ql.qmatmul("q8_0", cp[i % R], X, N, out=Y), R)
    alg = B.numel() + K * 2 + N * 4
    parts["gemv_q8_0_1024x1024_m1"] = {
        **roof("latency", alg, hot, HBM_PEAK_GBPS, "GB/s", "gemv_lds_kernel<Q8_0, M=1, CPT=1, R=1>",
               note="cache-resident (1.1 MB): a latency figure, no roofline claim"),
        "cold_us_median": round(cold["median"] * 1e3, 3), "cold_copies": R, "parity_max_err": e}
    log(f"gemv 1024x1024 q8_0: hot {hot['median'] * 1e3:.2f} us, cold {cold['median'] * 1e3:.2f} us")
    del cp, B

    N, K = 14336, 4096
    w = synth.weights_bf16(synth.seed_for(2, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(2, 1), 1, K)
    W = bf16_dev(w)
    X = bf16_dev(x)
    rows = sample_rows(N, 256, 1)
    for fmt, kern in (("q4k", "gemv_lds_kernel<Q4K, M=1, CPT=2, R=2>"), ("q8_0", "gemv_lds_kernel<Q8_0, M=1, CPT=2, R=2>")):
        B = ql.isq(fmt, W)
        Y = torch.empty((1, N), dtype=torch.float32, device=dev)
        ql.qmatmul(fmt, B, X, N, out=Y)
        e = check_gemv_rows(ql, fmt, w[rows], rows, B, N, K, x, Y.cpu().numpy(), f"{fmt} 14336x4096")
        R = copies_for(B.numel())
        cp = [B] + [B.clone() for _ in range(R - 1)]
        t = run.time(lambda i: ql.qmatmul(fmt, cp[i % R], X, N, out=Y), R)
        parts[f"gemv_{fmt}_14336x4096_m1"] = {**roof("hbm", B.numel() + K * 2 + N * 4, t, HBM_PEAK_GBPS, "GB/s", kern),
                                             "weight_GBps": round(B.numel() / t["median"] / 1e6, 1),
                                             "copies": R, "parity_max_err": e}
        log(f"gemv 14336x4096 {fmt}: {t['median'] * 1e3:.2f} us")
        del cp, B
    torch.cuda.empty_cache()
    return parts


def part_batched(torch, ql, synth, run, dev, bf16_dev):
    """Batched decode: Q4K 4096 x 14336 (1 % outliers), 4 / 16 / 64 tokens on AUTO."""
    import oracle

    parts = {}
    N, K = 4096, 14336
    w = synth.weights_bf16(synth.seed_for(3, 0), N, K, outliers=True)
    xs = synth.activations_bf16(synth.seed_for(3, 1), 64, K)
    B = ql.isq("q4k", bf16_dev(w))
    rows = sample_rows(N, 128, 3)
    Wd = oracle.dequant("q4k", oracle.quantize("q4k", w[rows]), len(rows), K)
    R = copies_for(B.numel())
    cp = [B] + [B.clone() for _ in range(R - 1)]
    for M in (4, 16, 64):
        X = bf16_dev(xs[:M])
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ql.qmatmul("q4k", B, X, N, out=Y)
        Yr, den = oracle.matmul_a16(Wd, xs[:M])
        e = float(oracle.normalized_error(Y.cpu().numpy()[:, rows], Yr, den).max())
        if e > 1e-3:
            raise SystemExit(f"parity failure: batched M={M}: {e:.3e}")
        t = run.time(lambda i: ql.qmatmul("q4k", cp[i % R], X, N, out=Y), R)
        parts[f"batched_q4k_4096x14336_m{M}"] = {
            **roof("hbm", B.numel() + M * K * 2 + M * N * 4, t, HBM_PEAK_GBPS, "GB/s", "AUTO (bf16 MFMA)"),
            "TFLOPs": round(2.0 * M * N * K / t["median"] / 1e9, 2), "parity_max_err": e}
        log(f"batched M={M}: {t['median'] * 1e3:.2f} us")
    del cp, B
    torch.cuda.empty_cache()
    return parts


def part_crossover(torch, ql, synth, run, dev, bf16_dev):
    """GEMV against the MFMA path for 1..8 tokens at 4096 x 14336 (sets AUTO)."""
    N, K = 4096, 14336
    B = ql.isq("q4k", bf16_dev(synth.weights_bf16(synth.seed_for(3, 0), N, K, outliers=True)))
    xs = bf16_dev(synth.activations_bf16(synth.seed_for(3, 1), 8, K))
    R = copies_for(B.numel())
    cp = [B] + [B.clone() for _ in range(R - 1)]
    cross = {}
    for M in range(1, 9):
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        row = {}
        for path in ("gemv", "mfma_bf16", "auto"):
            t = run.time(lambda i: ql.qmatmul("q4k", cp[i % R], xs[:M], N, out=Y, path=path), R)
            row[path] = round(t["median"] * 1e3, 2)
        cross[str(M)] = row
    log(f"crossover 4096x14336 q4k (us): {cross}")
    del cp, B
    torch.cuda.empty_cache()
    return {"crossover_q4k_4096x14336_us": cross}


def part_glu(torch, ql, synth, run, dev, bf16_dev):
    """Gated FFN projection 14336 x 4096 Q4K: one fused launch against two GEMVs."""
    parts = {}
    F, K = 14336, 4096
    bg = ql.isq("q4k", bf16_dev(synth.weights_bf16(synth.seed_for(2, 0), F, K)))
    bu = ql.isq("q4k", synth.device_normal_bf16(9501, (F, K), synth.W_SIGMA))
    R = copies_for(2 * bg.numel())
    cg = [bg] + [bg.clone() for _ in range(R - 1)]
    cu = [bu] + [bu.clone() for _ in range(R - 1)]
    xs = bf16_dev(synth.activations_bf16(synth.seed_for(2, 1), 2, K))
    for M in (1, 2):
        H = torch.empty((M, F), dtype=torch.float32, device=dev)
        Y2 = torch.empty((M, F), dtype=torch.float32, device=dev)
        fused = run.time(lambda i: ql.qmatmul_glu("q4k", cg[i % R], cu[i % R], xs[:M], F, out=H), R)

        def two(i):
            ql.qmatmul("q4k", cg[i % R], xs[:M], F, out=Y2)
            ql.qmatmul("q4k", cu[i % R], xs[:M], F, out=H)

        sep = run.time(two, R)
        parts[f"glu_q4k_14336x4096_m{M}"] = {
            **roof("hbm", 2 * bg.numel() + M * K * 2 + M * F * 4, fused, HBM_PEAK_GBPS, "GB/s",
                   f"gemv_lds_kernel<Q4K, M={M}, GLU>"), "two_gemvs_us": round(sep["median"] * 1e3, 2)}
        log(f"glu M={M}: fused {fused['median'] * 1e3:.2f} us, two GEMVs {sep['median'] * 1e3:.2f} us")
    del cg, cu, bg, bu
    torch.cuda.empty_cache()
    return parts


def part_formats(torch, ql, synth, run, dev, bf16_dev):
    """The further formats (Q5K, Q3K, Q2K, Q4_0, Q4_1, Q5_0, Q5_1) and FP8
    (W8A16) at 14336 x 4096: ISQ, the one-token GEMV and the 16-token MFMA
    path, each output checked against the oracle on sampled rows."""
    import oracle

    parts = {}
    N, K = 14336, 4096
    w = synth.weights_bf16(synth.seed_for(2, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(2, 2), 16, K)
    W = bf16_dev(w)
    X = bf16_dev(x)
    rows = sample_rows(N, 128, 3)
    for fmt in oracle.MORE_FORMATS + ("fp8",):
        B = ql.isq(fmt, W)
        out = torch.empty_like(B)
        t_isq = run.time(lambda i: ql.isq(fmt, W, out=out), 4)
        if fmt == "fp8":
            Wd = oracle.dequant_fp8(oracle.quantize_fp8(w[rows]))
        else:
            Wd = oracle.dequant(fmt, oracle.quantize(fmt, w[rows]), len(rows), K)
        R = copies_for(B.numel())
        cp = [B] + [B.clone() for _ in range(R - 1)]
        entry = {"isq_us": round(t_isq["median"] * 1e3, 2),
                 "isq_GBps": round((2 * N * K + B.numel()) / t_isq["median"] / 1e6, 1), "weight_bytes": B.numel()}
        for M, path in ((1, "gemv"), (16, "mfma_bf16")):
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ql.qmatmul(fmt, B, X[:M], N, out=Y, path=path)
            Yr, den = oracle.matmul_a16(Wd, x[:M])
            e = float(oracle.normalized_error(Y.cpu().numpy()[:, rows], Yr, den).max())
            if e > 1e-3:
                raise SystemExit(f"parity failure: {fmt} {path} M={M}: {e:.3e}")
            t = run.time(lambda i: ql.qmatmul(fmt, cp[i % R], X[:M], N, out=Y, path=path), R)
            entry[f"m{M}"] = {**roof("hbm", B.numel() + M * K * 2 + M * N * 4, t, HBM_PEAK_GBPS, "GB/s",
                                     "gemv_fp8_kernel" if (fmt == "fp8" and M <= 2) else
                                     ("gemv_genx_kernel" if M == 1 else "gemm_gen_lds_kernel")),
                              "parity_max_err": e}
        parts[f"format_{fmt}_14336x4096"] = entry
        log(f"format {fmt}: ISQ {entry['isq_us']} us, GEMV M=1 {entry['m1']['us_median']} us, "
            f"MFMA M=16 {entry['m16']['us_median']} us")
        del cp, B, out
    torch.cuda.empty_cache()
    return parts


def part_prefill(torch, ql, synth, run, dev, bf16_dev):
    """Prefill 2048 x 4096 x 14336: Q8_0 on the bf16 MFMA and int8 paths, FP8 W8A8."""
    import oracle

    parts = {}
    M, N, K = 2048, 14336, 4096
    w = synth.weights_bf16(synth.seed_for(4, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(4, 1), M, K)
    X = bf16_dev(x)
    W = bf16_dev(w)
    fl = 2.0 * M * N * K
    rng = np.random.Generator(np.random.PCG64(11))
    mi, ni = rng.integers(0, M, 1024), rng.integers(0, N, 1024)
    rows, inv = np.unique(ni, return_inverse=True)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)

    B = ql.isq("q8_0", W)
    cp = [B, B.clone()]
    fw = oracle.quantize("q8_0", w[rows])
    ql.qmatmul("q8_0", B, X, N, out=Y, path="mfma_bf16")
    Yr, den = oracle.matmul_a16_pairs(oracle.dequant("q8_0", fw, len(rows), K), x, mi, inv)
    e = float(oracle.normalized_error(Y.cpu().numpy()[mi, ni], Yr, den).max())
    if e > 1e-3:
        raise SystemExit(f"parity failure: prefill bf16 {e:.3e}")
    t = run.time(lambda i: ql.qmatmul("q8_0", cp[i % 2], X, N, out=Y, path="mfma_bf16"), 4)
    parts["prefill_q8_0_2048x4096x14336_bf16_mfma"] = {
        **roof("mfma", fl, t, BF16_PEAK_TFLOPS, "TFLOP/s", "gemm_pf_kernel<Q8_0> (exact codes, running rescale)"),
        "parity_max_err": e}
    log(f"prefill q8_0 bf16 path: {t['median'] * 1e3:.1f} us")

    ws = torch.empty(ql.workspace_bytes("q8_0", "mfma_i8", M, K), dtype=torch.uint8, device=dev)
    ql.qmatmul("q8_0", B, X, N, out=Y, path="mfma_i8", workspace=ws)
    Y8, den8 = oracle.matmul_a8(fw, oracle.quantize("q8_0", x), M, len(rows), K, mi=mi, ni=inv)
    e = float(oracle.normalized_error(Y.cpu().numpy()[mi, ni], Y8, den8).max())
    if e > 1e-3:
        raise SystemExit(f"parity failure: prefill int8 {e:.3e}")
    t = run.time(lambda i: ql.qmatmul("q8_0", cp[i % 2], X, N, out=Y, path="mfma_i8", workspace=ws), 4)
    parts["prefill_q8_0_2048x4096x14336_int8_mfma"] = {
        **roof("mfma", fl, t, INT8_PEAK_TOPS, "TFLOP/s", "isq (activations) + gemm_i8_kernel",
               note="TOPS against the int8 peak; activation quantization included"), "parity_max_err": e}
    log(f"prefill q8_0 int8 path: {t['median'] * 1e3:.1f} us")
    del cp, B, ws

    B = ql.isq("fp8", W)
    cp = [B, B.clone()]
    ws = torch.empty(ql.workspace_bytes("fp8", "mfma_fp8", M, K), dtype=torch.uint8, device=dev)
    ql.qmatmul("fp8", B, X, N, out=Y, path="mfma_fp8", workspace=ws)
    Yf, denf = oracle.matmul_fp8(oracle.quantize_fp8(x), oracle.quantize_fp8(w[rows]), mi=mi, ni=inv)
    e = float(oracle.normalized_error(Y.cpu().numpy()[mi, ni], Yf, denf).max())
    if e > 1e-3:
        raise SystemExit(f"parity failure: prefill fp8 {e:.3e}")
    t = run.time(lambda i: ql.qmatmul("fp8", cp[i % 2], X, N, out=Y, path="mfma_fp8", workspace=ws), 4)
    parts["prefill_fp8_2048x4096x14336_w8a8"] = {
        **roof("mfma", fl, t, FP8_PEAK_TFLOPS, "TFLOP/s", "isq_fp8 (activations) + gemm_fp8_tile_kernel",
               note="FP8 E4M3 weights (per-row scales), dynamic per-token activations; quantization included"),
        "parity_max_err": e}
    log(f"prefill fp8 w8a8: {t['median'] * 1e3:.1f} us")
    del cp, B, ws, W, X, Y
    torch.cuda.empty_cache()
    return parts


def part_ceilings(torch, ql, run, dev):
    """Measured ceilings: a streaming read of buffers read once per launch
    (550 MB, the head's size; 33 MB slices rotated past the Infinity Cache,
    the Q4K 14336 x 4096 size), and an MFMA-only bf16 loop."""
    parts = {}
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    big = torch.empty(2 * 550_502_400 // 16 * 16, dtype=torch.uint8, device=dev).fill_(1)
    half = big.numel() // 2
    views = [big[:half], big[half:]]
    t = run.time(lambda i: ql.probe_read(views[i % 2], sink), 4)
    parts["ceiling_read_550MB"] = roof("hbm", half, t, HBM_PEAK_GBPS, "GB/s", "read_probe_kernel",
                                       note="measured HBM read ceiling at the head's size")
    n33 = 33_030_144
    R = copies_for(n33)
    sl = [big[i * n33:(i + 1) * n33] for i in range(R)]
    t = run.time(lambda i: ql.probe_read(sl[i % R], sink), R)
    parts["ceiling_read_33MB"] = roof("hbm", n33, t, HBM_PEAK_GBPS, "GB/s", "read_probe_kernel",
                                      note="measured ceiling for one launch reading 33 MB (launch, ramp, drain)")
    log(f"ceilings: read 550 MB {parts['ceiling_read_550MB']['achieved']:.0f} GB/s, "
        f"33 MB {parts['ceiling_read_33MB']['achieved']:.0f} GB/s")
    del big, views, sl
    iters = 2000
    flops = ql.probe_mfma(iters, sink)
    t = run.time(lambda i: ql.probe_mfma(iters, sink), 2)
    parts["ceiling_mfma_bf16"] = roof("mfma", flops, t, BF16_PEAK_TFLOPS, "TFLOP/s", "mfma_probe_kernel",
                                      note="v_mfma_f32_32x32x16_bf16 chains, two waves per SIMD, no memory")
    log(f"ceilings: MFMA bf16 {parts['ceiling_mfma_bf16']['achieved']:.0f} TFLOP/s")
    # the same loop with 16 fp32 fmas per MFMA: MFMAs only, fmas only, and
    # both in one instruction stream, at 1, 2 and 8 waves per SIMD -- how far
    # VALU work hides behind MFMAs at a kernel's occupancy
    mixes = {}
    for wps in (1, 2, 8):
        mix, counts = {}, {}
        for mode, name in ((0, "mfma_only"), (1, "valu_only"), (2, "interleaved")):
            counts[name] = ql.probe_mix(iters // wps, mode, wps, sink)
            t = run.time(lambda i, mode=mode, wps=wps: ql.probe_mix(iters // wps, mode, wps, sink), 2)
            mix[name] = round(t["median"] * 1e3, 1)
        hidden = mix["mfma_only"] + mix["valu_only"] - mix["interleaved"]
        mixes[f"waves_per_simd_{wps}"] = {
            "us_median": mix, "mfma_flops": counts["mfma_only"][0], "valu_fma_insts": counts["valu_only"][1],
            "hidden_frac": round(hidden / min(mix["mfma_only"], mix["valu_only"]), 3)}
    parts["ceiling_mfma_valu_mix"] = {
        **mixes,
        "note": "mix_probe_kernel: v_mfma_f32_32x32x16_bf16 chains with 16 fp32 fmas per MFMA (the fmas take "
                "twice the MFMAs' time alone); hidden_frac = (t_mfma + t_valu - t_both) / min(t_mfma, t_valu), "
                "1 = full overlap, 0 = the two add"}
    log("ceilings: MFMA + VALU mix, hidden fraction at 1 / 2 / 8 waves per SIMD: "
        + " / ".join(str(v["hidden_frac"]) for v in mixes.values()))
    torch.cuda.empty_cache()
    return parts


# ----------------------------------------------------------------------
# the oracle on the host cores
# ----------------------------------------------------------------------

def _oracle_gemv_rate(fmt, w, x, seconds):
    """GB/s of quantized weights through the oracle's GEMV (unpack + exact
    dequant + fp64 matmul), repeated for `seconds`."""
    import oracle

    N, K = w.shape
    buf = oracle.pack(fmt, oracle.quantize(fmt, w), N, K)
    reps, t0 = 0, time.perf_counter()
    while True:
        Wd = oracle.dequant(fmt, oracle.unpack(fmt, buf, N, K), N, K)
        oracle.matmul_a16(Wd, x)
        reps += 1
        el = time.perf_counter() - t0
        if el > seconds or reps >= 10000:
            break
    return buf.size * reps / el / 1e9, reps, el


def _oracle_isq_rate(fmt, w, seconds):
    import oracle

    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.quantize(fmt, w)
        reps += 1
        el = time.perf_counter() - t0
        if el > seconds:
            break
    return w.size * reps / el, reps, el


def _oracle_gemm_rate(w, x, seconds):
    import oracle

    Wd = oracle.dequant("q8_0", oracle.quantize("q8_0", w), *w.shape)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.matmul_a16(Wd, x)
        reps += 1
        el = time.perf_counter() - t0
        if el > seconds:
            break
    return 2.0 * x.shape[0] * w.shape[0] * w.shape[1] * reps / el / 1e9, reps, el


def _samples():
    import synth

    return {
        "head": (synth.weights_bf16(7001, 512, HEAD_K), synth.activations_bf16(7002, 1, HEAD_K)),
        "cfg1": (synth.weights_bf16(synth.seed_for(1, 0), 1024, 1024), synth.activations_bf16(synth.seed_for(1, 1), 1, 1024)),
        "cfg2": (synth.weights_bf16(synth.seed_for(2, 0), 2048, 4096), synth.activations_bf16(synth.seed_for(2, 1), 1, 4096)),
    }


_ONE_CORE = """
import sys, json
sys.path.insert(0, {root!r})
import bench
s = bench._samples()
out = {{}}
for name, fmt, sec in (("head", "q6k", 4.0), ("cfg1", "q8_0", 2.0), ("cfg2", "q4k", 3.0)):
    r, reps, el = bench._oracle_gemv_rate(fmt, s[name][0], s[name][1], sec)
    out[name] = {{"value": round(r, 4), "reps": reps, "el": round(el, 2)}}
print(json.dumps(out))
"""


def cpu_baseline():
    """The oracle on the host cores, on bounded samples of the workloads:
    headline unit (GB/s of Q6K head weights through the oracle's GEMV), ISQ
    per format, the fp64 GEMM at the prefill shape's inner dimensions; then
    one core (child process, thread counts 1, no GPU) for cfg1, cfg2 and the
    head."""
    import subprocess

    import synth

    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    s = _samples()
    rate, reps, el = _oracle_gemv_rate("q6k", s["head"][0], s["head"][1], 8.0)
    out = {"value": round(rate, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} one-token GEMVs over 512 rows x {HEAD_K} of a Q6K head (1/256 of the 131072 rows): "
                     f"unpack + exact fp64 dequant + fp64 matmul, {el:.1f} s; GB/s of quantized weights"}
    try:
        with open("/proc/cpuinfo") as f:
            out["cpu_model"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    w = synth.weights_bf16(7003, 1024, 4096)
    isq = {}
    for fmt in ("q8_0", "q4k", "q6k"):
        r, reps, el = _oracle_isq_rate(fmt, w, 2.0)
        isq[fmt] = {"elements_per_s": round(r, 1), "bf16_GBps": round(2 * r / 1e9, 4), "reps": reps}
    out["isq_1024x4096"] = isq
    xg = synth.activations_bf16(7004, 64, 4096)
    r, reps, el = _oracle_gemm_rate(synth.weights_bf16(7005, 512, 4096), xg, 4.0)
    out["gemm_fp64_64x512x4096"] = {"GFLOPs": round(r, 3), "reps": reps,
                                    "note": "the prefill GEMM's arithmetic on a 64-token x 512-row sample"}
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-c", _ONE_CORE.format(root=ROOT)], env=env, capture_output=True,
                         text=True, timeout=300)
    if res.returncode == 0 and res.stdout.strip():
        one = json.loads(res.stdout.strip().splitlines()[-1])
        out["one_core"] = {k: {"value": v["value"], "unit": "GB/s", "cores": 1, "reps": v["reps"]} for k, v in one.items()}
    else:
        out["one_core"] = {"error": (res.stderr or "no output")[-300:]}
    return out


if __name__ == "__main__":
    main()
