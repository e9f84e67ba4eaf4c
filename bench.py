#!/usr/bin/env python3
"""Benchmark of the 4-bit-weight GEMM hot path on one MI355X.

One step = one pass of the whole hot path over synthetic inputs:
  decode  : AWQ W4A16 g128 GEMV at M=1 over the Llama-2-7B layer set
            (QKV 4096x12288, O 4096x4096, gate/up 4096x22016, down 11008x4096);
            weights rotate through enough distinct copies (>= 512 MB) that every
            step streams them from HBM, not from the 256 MB Infinity Cache;
  prefill : AWQ W4A16 g128 GEMM at M=2048 over the Llama-3-8B layer set
            (QKV 4096x6144, O 4096x4096, gate/up 4096x28672, down 14336x4096);
  w4a8    : per-token activation quantisation + W4A8 GEMM on the QQQ shape
            N=8192, K=21760 at M=1 (rotating weights) and M=1024.
All inputs are resident in HBM before the timed region.  `value` is the decode
weight bandwidth (qweight + scales + qzeros bytes / GEMV kernel time); the
prefill TFLOP/s and the W4A8 figures are reported beside it.

Kernel durations come from HIP events recorded on the stream the kernels run
on (torch's current stream), around every launch inside the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_F16_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk (dense fp16/bf16; ~2.5 PF published)
MFMA_I8_PEAK_TOPS = 5033.2     # dense int8
METRIC = "W4A16 g128 GEMV weight GB/s at M=1 + GEMM TFLOP/s at M=2048 (%roofline)"

DECODE_LAYERS = [("qkv", 4096, 12288), ("o", 4096, 4096), ("gate_up", 4096, 22016), ("down", 11008, 4096)]
PREFILL_LAYERS = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
G = 128
M_DECODE, M_PREFILL = 1, 2048
W4A8_K, W4A8_N, W4A8_M = 21760, 8192, (1, 1024)
ROTATE_MB = 600


def w4a16_weight_bytes(K, N, G=G, sym=False):
    return K * N // 2 + (K // G) * N * 2 + (0 if sym else (K // G) * N // 2)


def w4a16_alg_bytes(M, K, N, G=G):
    return w4a16_weight_bytes(K, N, G) + M * K * 2 + M * N * 2


def w4a8_alg_bytes(M, K, N):
    return K * N // 2 + N * 2 + M * K + 4 * M + 2 * M * N


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = ["bit_weight_only_awq_amd/csrc/w4a16.hip", "bit_weight_only_awq_amd/csrc/device.hpp",
                  "bit_weight_only_awq_amd/csrc/api.cpp"]


def load_traffic(name, digest):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/*.json),
    used only if the kernel sources are unchanged since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{name}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_digest") != digest:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(budget_s: float):
    """The oracle on the decode workload (M=1 over the Llama-2-7B layer set), run
    on this host's cores until about budget_s seconds of work are done."""
    import oracle
    import synthgen
    orc = oracle.get()
    cores = len(os.sched_getaffinity(0))
    cases = [synthgen.w4a16_case(1, K, N, G) for _, K, N in DECODE_LAYERS]
    done_bytes, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for c in cases:
            orc.w4a16(c.x, c.qweight, c.scales, c.qzeros, G, nthreads=cores)
            done_bytes += w4a16_weight_bytes(c.K, c.N)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode M=1 Llama-2-7B layer set (4 layers, {sum(w4a16_weight_bytes(K, N) for _, K, N in DECODE_LAYERS) / 1e6:.1f} MB "
                      f"of weights) x {reps} passes in {dt:.1f} s, fp64 scalar oracle, {cores} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--phases", default="decode,prefill,w4a8")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the 4-bit GEMM hot path has no "
                                   "multi-GPU component here (see the sharding notes in DESIGN.md)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import bit_weight_only_awq_amd as awq
    import synthgen

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    phases = set(args.phases.split(","))
    stream = torch.cuda.current_stream(dev)

    # ---------------- inputs (resident in HBM before timing) ----------------
    decode_set_bytes = sum(w4a16_weight_bytes(K, N) for _, K, N in DECODE_LAYERS)
    n_copies = max(2, -(-ROTATE_MB * 10 ** 6 // decode_set_bytes))
    decode = []  # [copy][layer] -> tensors
    if "decode" in phases:
        for r in range(n_copies):
            row = []
            for li, (name, K, N) in enumerate(DECODE_LAYERS):
                c = synthgen.w4a16_case(M_DECODE, K, N, G, seed=synthgen.seed_for(f"bench|decode|{name}|{r}"))
                row.append((c.x.to(dev), c.qweight.to(dev), c.scales.to(dev), c.qzeros.to(dev),
                            torch.empty(M_DECODE, N, dtype=torch.float16, device=dev), K, N))
            decode.append(row)
    prefill = []
    if "prefill" in phases:
        for name, K, N in PREFILL_LAYERS:
            c = synthgen.w4a16_case(M_PREFILL, K, N, G, seed=synthgen.seed_for(f"bench|prefill|{name}"))
            prefill.append((c.x.to(dev), c.qweight.to(dev), c.scales.to(dev), c.qzeros.to(dev),
                            torch.empty(M_PREFILL, N, dtype=torch.float16, device=dev), K, N))
    w4a8 = []
    if "w4a8" in phases:
        w8_copies = max(2, -(-ROTATE_MB * 10 ** 6 // (W4A8_K * W4A8_N // 2)))
        bs = []
        for r in range(w8_copies):
            c = synthgen.w4a8_case(1, W4A8_K, W4A8_N, -1, seed=synthgen.seed_for(f"bench|w4a8|{r}"))
            bs.append((c.b.to(dev), c.s2.to(dev)))
        for M in W4A8_M:
            x = synthgen.activations(M, W4A8_K, seed=synthgen.seed_for(f"bench|w4a8x|{M}")).to(dev)
            a8 = torch.empty(M, W4A8_K, dtype=torch.int8, device=dev)
            s1 = torch.empty(M, dtype=torch.float32, device=dev)
            y = torch.empty(M, W4A8_N, dtype=torch.float16, device=dev)
            w4a8.append((M, x, a8, s1, y))
    # copy kernel of known size, used to calibrate HBM byte counters in profiling runs
    cal_src = torch.ones(64 * 2 ** 20 // 2, dtype=torch.float16, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run_step(step, rec):
        # decode: one GEMV per layer, weights from copy (step mod n_copies)
        if decode:
            for li, (x, qw, s, qz, y, K, N) in enumerate(decode[step % n_copies]):
                e0, e1 = ev(), ev()
                e0.record(stream)
                awq.gemv_w4a16(x, qw, s, qz, G, out=y)
                e1.record(stream)
                rec.append(("decode", li, e0, e1))
        for li, (x, qw, s, qz, y, K, N) in enumerate(prefill):
            e0, e1 = ev(), ev()
            e0.record(stream)
            awq.gemm_w4a16(x, qw, s, qz, G, out=y)
            e1.record(stream)
            rec.append(("prefill", li, e0, e1))
        if w4a8:
            b, s2 = bs[step % len(bs)]
            for mi, (M, x, a8, s1, y) in enumerate(w4a8):
                e0, e1, e2 = ev(), ev(), ev()
                e0.record(stream)
                awq.quant_act(x, a8, s1)
                e1.record(stream)
                awq.w4a8_gemm(a8, b, s1, s2, out=y)
                e2.record(stream)
                rec.append(("w4a8_quant", mi, e0, e1))
                rec.append(("w4a8_gemm", mi, e1, e2))

    for w in range(args.warmup):
        run_step(w, [])
    torch.cuda.synchronize()

    rec = []
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        run_step(args.warmup + s, rec)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    from collections import defaultdict
    tsum = defaultdict(float)
    for kind, li, a, b in rec:
        tsum[(kind, li)] += a.elapsed_time(b) / 1e3  # seconds
    K_ = args.steps

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_step, 4), "wall_s_timed": round(wall, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic"}

    digest = source_digest(KERNEL_SOURCES)
    if decode:
        t_dec = sum(tsum[("decode", li)] for li in range(len(DECODE_LAYERS)))
        wbytes = decode_set_bytes * K_
        abytes = sum(w4a16_alg_bytes(M_DECODE, K, N) for _, K, N in DECODE_LAYERS) * K_
        out["value"] = round(wbytes / t_dec / 1e9, 2)
        out["unit"] = "GB/s"
        per_layer = {}
        for li, (name, K, N) in enumerate(DECODE_LAYERS):
            t = tsum[("decode", li)] / K_
            per_layer[name] = {"K": K, "N": N, "us": round(t * 1e6, 3),
                               "weight_GBs": round(w4a16_weight_bytes(K, N) / t / 1e9, 1),
                               "frac_hbm": round(w4a16_alg_bytes(1, K, N) / t / 1e9 / HBM_PEAK_GBS, 4)}
        achieved = abytes / t_dec / 1e9
        traffic = load_traffic("gemv_w4a16_m1_llama2_7b", digest)
        out["roofline"] = {"kernel": "w4a16_skinny (decode GEMV, M=1, 4 Llama-2-7B layers)", "bound": "hbm",
                           "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                           "avg_launch_us": round(t_dec / (K_ * len(DECODE_LAYERS)) * 1e6, 3),
                           "per_layer": per_layer}
    if prefill:
        t_pre = sum(tsum[("prefill", li)] for li in range(len(PREFILL_LAYERS)))
        flops = sum(2 * M_PREFILL * N * K for _, K, N in PREFILL_LAYERS) * K_
        tf = flops / t_pre / 1e12
        per_layer = {}
        for li, (name, K, N) in enumerate(PREFILL_LAYERS):
            t = tsum[("prefill", li)] / K_
            per_layer[name] = {"K": K, "N": N, "us": round(t * 1e6, 2),
                               "TFLOPs": round(2 * M_PREFILL * N * K / t / 1e12, 1)}
        out["gemm_m2048"] = {"kernel": "w4a16_tiled (prefill GEMM, M=2048, 4 Llama-3-8B layers)", "bound": "mfma",
                             "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "per_layer": per_layer}
    if w4a8:
        res = {}
        for mi, (M, *_rest) in enumerate(w4a8):
            tq = tsum[("w4a8_quant", mi)] / K_
            tg = tsum[("w4a8_gemm", mi)] / K_
            ops = 2 * M * W4A8_N * W4A8_K
            r = {"quant_us": round(tq * 1e6, 2), "gemm_us": round(tg * 1e6, 2),
                 "gemm_TOPs": round(ops / tg / 1e12, 2),
                 "gemm_weight_GBs": round((W4A8_K * W4A8_N // 2 + 2 * W4A8_N) / tg / 1e9, 1),
                 "frac_hbm": round(w4a8_alg_bytes(M, W4A8_K, W4A8_N) / tg / 1e9 / HBM_PEAK_GBS, 4),
                 "frac_i8_mfma": round(ops / tg / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
            res[f"M={M}"] = r
        out["w4a8_n8192_k21760"] = res
    out["config"] = {"workload": "AWQ W4A16 g128: decode GEMV M=1 on the Llama-2-7B layer set "
                                 "(4096x12288, 4096x4096, 4096x22016, 11008x4096) + prefill GEMM M=2048 on "
                                 "the Llama-3-8B layer set (4096x6144, 4096x4096, 4096x28672, 14336x4096); "
                                 "QQQ W4A8 N=8192 K=21760 at M=1 and M=1024",
                     "group_size": G, "decode_weight_copies": n_copies if decode else 0,
                     "source_digest": digest}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
