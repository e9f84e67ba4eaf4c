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
All inputs are resident in HBM before the timed region.  Each phase of a step
is one HIP graph (captured once, replayed every step), so the GPU runs the
kernels back to back without waiting on host-side launches; HIP events on the
replay stream bracket every phase.  `value` is the decode weight bandwidth:
(qweight + scales + qzeros bytes of the 4 layers) / decode phase time.  The
prefill TFLOP/s and the W4A8 figures are reported beside it.
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
KERNEL_SOURCES = ["bit_weight_only_awq_amd/csrc/w4a16.hip", "bit_weight_only_awq_amd/csrc/gemm_w4a16.hip",
                  "bit_weight_only_awq_amd/csrc/w4a16_ops.hpp", "bit_weight_only_awq_amd/csrc/w4a8.hip",
                  "bit_weight_only_awq_amd/csrc/device.hpp", "bit_weight_only_awq_amd/csrc/api.cpp"]


def w4a16_weight_bytes(K, N, G=G, sym=False):
    return K * N // 2 + (K // G) * N * 2 + (0 if sym else (K // G) * N // 2)


def w4a16_alg_bytes(M, K, N, G=G):
    """Bytes the decode GEMV must move: packed weights, scales, zeros, X and Y."""
    return w4a16_weight_bytes(K, N, G) + M * K * 2 + M * N * 2


def w4a8_alg_bytes(M, K, N):
    return K * N // 2 + N * 2 + M * K + 4 * M + 2 * M * N


def source_digest(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, digest):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/<name>.traffic.json),
    used only while the kernel sources are unchanged since the counters were taken."""
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
    mb = sum(w4a16_weight_bytes(K, N) for _, K, N in DECODE_LAYERS) / 1e6
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"decode M=1 on the Llama-2-7B layer set (4 layers, {mb:.1f} MB of weights) x {reps} "
                      f"passes in {dt:.1f} s; fp64 scalar C oracle on {cores} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the 4-bit GEMM hot path has no "
                                   "multi-GPU component here (the sharding design is described in DESIGN.md)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import bit_weight_only_awq_amd as awq
    import synthgen

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # ---------------- inputs (resident in HBM before timing) ----------------
    decode_set_bytes = sum(w4a16_weight_bytes(K, N) for _, K, N in DECODE_LAYERS)
    n_copies = max(2, -(-ROTATE_MB * 10 ** 6 // decode_set_bytes))
    decode = []  # [copy][layer]
    for r in range(n_copies):
        row = []
        for name, K, N in DECODE_LAYERS:
            c = synthgen.w4a16_case(M_DECODE, K, N, G, seed=synthgen.seed_for(f"bench|decode|{name}|{r}"))
            row.append((c.x.to(dev), c.qweight.to(dev), c.scales.to(dev), c.qzeros.to(dev),
                        torch.empty(M_DECODE, N, dtype=torch.float16, device=dev)))
        decode.append(row)
    prefill = []
    for name, K, N in PREFILL_LAYERS:
        c = synthgen.w4a16_case(M_PREFILL, K, N, G, seed=synthgen.seed_for(f"bench|prefill|{name}"))
        prefill.append((c.x.to(dev), c.qweight.to(dev), c.scales.to(dev), c.qzeros.to(dev),
                        torch.empty(M_PREFILL, N, dtype=torch.float16, device=dev)))
    w8_copies = max(2, -(-ROTATE_MB * 10 ** 6 // (W4A8_K * W4A8_N // 2)))
    w8w = []
    for r in range(w8_copies):
        c = synthgen.w4a8_case(1, W4A8_K, W4A8_N, -1, seed=synthgen.seed_for(f"bench|w4a8|{r}"))
        w8w.append((c.b.to(dev), c.s2.to(dev)))
    w8a = []
    for M in W4A8_M:
        x = synthgen.activations(M, W4A8_K, seed=synthgen.seed_for(f"bench|w4a8x|{M}")).to(dev)
        w8a.append((M, x, torch.empty(M, W4A8_K, dtype=torch.int8, device=dev),
                    torch.empty(M, dtype=torch.float32, device=dev),
                    torch.empty(M, W4A8_N, dtype=torch.float16, device=dev)))
    # copy kernel of known size, used to calibrate HBM byte counters in profiling runs
    cal_src = torch.ones(64 * 2 ** 20 // 2, dtype=torch.float16, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)

    def run_decode(r, layers=None):
        for li in (layers if layers is not None else range(len(DECODE_LAYERS))):
            x, qw, s, qz, y = decode[r][li]
            awq.gemv_w4a16(x, qw, s, qz, G, out=y)

    def run_prefill(layers=None):
        for li in (layers if layers is not None else range(len(PREFILL_LAYERS))):
            x, qw, s, qz, y = prefill[li]
            awq.gemm_w4a16(x, qw, s, qz, G, out=y)

    def run_w4a8(r, which=None):
        b, s2 = w8w[r]
        for i in (which if which is not None else range(len(w8a))):
            M, x, a8, s1, y = w8a[i]
            awq.quant_act(x, a8, s1)
            awq.w4a8_gemm(a8, b, s1, s2, out=y)

    # every op once eagerly: allocates the shared workspace before capture
    run_decode(0)
    run_prefill()
    run_w4a8(0)
    torch.cuda.synchronize()

    cap = torch.cuda.Stream(dev)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        return g

    g_dec = [capture(lambda r=r: run_decode(r)) for r in range(n_copies)]
    g_pre = capture(run_prefill)
    g_w8 = [capture(lambda r=r: run_w4a8(r)) for r in range(w8_copies)]
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = torch.cuda.current_stream(dev)

    def step(i, rec):
        e = [ev() for _ in range(4)]
        e[0].record(stream)
        g_dec[i % n_copies].replay()
        e[1].record(stream)
        g_pre.replay()
        e[2].record(stream)
        g_w8[i % w8_copies].replay()
        e[3].record(stream)
        if rec is not None:
            rec.append(e)

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    rec = []
    t0, t1 = ev(), ev()
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, rec)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    K_ = args.steps
    t_dec = sum(e[0].elapsed_time(e[1]) for e in rec) / 1e3 / K_   # seconds per step
    t_pre = sum(e[1].elapsed_time(e[2]) for e in rec) / 1e3 / K_
    t_w8 = sum(e[2].elapsed_time(e[3]) for e in rec) / 1e3 / K_

    # per-layer / per-kernel times (outside the timed steps): one graph per
    # layer with launches over rotating weight copies, replayed a few times
    def per_launch(fn, launches, reps=4):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / (reps * launches)

    dec_layer = {}
    for li, (name, K, N) in enumerate(DECODE_LAYERS):
        t = per_launch(lambda li=li: [run_decode(r, [li]) for r in range(n_copies)], n_copies)
        dec_layer[name] = {"K": K, "N": N, "us": round(t * 1e6, 3),
                           "weight_GBs": round(w4a16_weight_bytes(K, N) / t / 1e9, 1),
                           "frac_hbm": round(w4a16_alg_bytes(1, K, N) / t / 1e9 / HBM_PEAK_GBS, 4)}
    pre_layer = {}
    for li, (name, K, N) in enumerate(PREFILL_LAYERS):
        t = per_launch(lambda li=li: run_prefill([li]), 1, reps=3)
        pre_layer[name] = {"K": K, "N": N, "us": round(t * 1e6, 2),
                           "TFLOPs": round(2 * M_PREFILL * N * K / t / 1e12, 1)}
    w8_res = {}
    for i, (M, *_r) in enumerate(w8a):
        tq = per_launch(lambda i=i: [awq.quant_act(w8a[i][1], w8a[i][2], w8a[i][3]) for _ in range(4)], 4)
        tg = per_launch(lambda i=i: [awq.w4a8_gemm(w8a[i][2], w8w[r][0], w8a[i][3], w8w[r][1], out=w8a[i][4])
                                     for r in range(w8_copies)], w8_copies)
        ops = 2 * M * W4A8_N * W4A8_K
        w8_res[f"M={M}"] = {"quant_us": round(tq * 1e6, 2), "gemm_us": round(tg * 1e6, 2),
                            "gemm_TOPs": round(ops / tg / 1e12, 2),
                            "gemm_weight_GBs": round((W4A8_K * W4A8_N // 2 + 2 * W4A8_N) / tg / 1e9, 1),
                            "frac_hbm": round(w4a8_alg_bytes(M, W4A8_K, W4A8_N) / tg / 1e9 / HBM_PEAK_GBS, 4),
                            "frac_i8_mfma": round(ops / tg / 1e12 / MFMA_I8_PEAK_TOPS, 4)}

    digest = source_digest()
    dec_alg = sum(w4a16_alg_bytes(M_DECODE, K, N) for _, K, N in DECODE_LAYERS)
    achieved = dec_alg / t_dec / 1e9
    pre_flops = sum(2 * M_PREFILL * N * K for _, K, N in PREFILL_LAYERS)
    tf = pre_flops / t_pre / 1e12
    out = {"metric": METRIC, "value": round(decode_set_bytes / t_dec / 1e9, 2), "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
           "wall_s_timed": round(wall, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "data": "synthetic",
           "config": {"workload": "AWQ W4A16 g128: decode GEMV M=1 on the Llama-2-7B layer set (4096x12288, "
                                  "4096x4096, 4096x22016, 11008x4096) + prefill GEMM M=2048 on the Llama-3-8B "
                                  "layer set (4096x6144, 4096x4096, 4096x28672, 14336x4096); QQQ W4A8 N=8192 "
                                  "K=21760 at M=1 and M=1024",
                      "group_size": G, "decode_weight_copies": n_copies, "source_digest": digest},
           "roofline": {"kernel": "w4a16_decode (decode GEMV, M=1, 4 Llama-2-7B layers back to back)",
                        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": load_traffic("w4a16_decode_m1_llama2_7b", digest),
                        "avg_launch_us": round(t_dec / len(DECODE_LAYERS) * 1e6, 3),
                        "per_layer": dec_layer},
           "gemm_m2048": {"kernel": "w4a16_gemm (prefill GEMM, M=2048, 4 Llama-3-8B layers back to back)",
                          "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "per_layer": pre_layer},
           "w4a8_n8192_k21760": w8_res,
           "phases_us": {"decode": round(t_dec * 1e6, 2), "prefill": round(t_pre * 1e6, 2),
                         "w4a8": round(t_w8 * 1e6, 2)}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
