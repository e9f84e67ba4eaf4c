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
All inputs are resident in HBM before the timed region.  The timed region runs
exactly K passes of each phase; each phase is one HIP graph holding its K passes
back to back (weights rotating through the copies), bracketed by HIP events on
the replay stream, so a graph's launch cost is paid once per phase rather than
once per pass.  `value` is the decode weight bandwidth: (qweight + scales +
qzeros bytes of the 4 layers) / decode time per pass.  The prefill TFLOP/s, the
W4A8 figures, per-layer times (graphs of one layer over rotating weights), the
read-only bandwidth probe at each decode layer's size and the stated target
shapes are reported beside it.
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
CAL_BYTES = 256 * 2 ** 20                       # calibration copy: bytes read and bytes written
PER_LAUNCH_MIN = 64   # launches per graph in the per-layer timings
TARGET_SHAPES = [(4096, 4096), (4096, 14336)]   # (K, N): the stated M=1 / M=2048 targets
M_TARGETS = (1, 2048)
ROTATE_MB = 600
KERNEL_SOURCES = ["bit_weight_only_awq_amd/csrc/w4a16.hip", "bit_weight_only_awq_amd/csrc/gemm_w4a16.hip",
                  "bit_weight_only_awq_amd/csrc/dequant.hip", "bit_weight_only_awq_amd/csrc/stream_w4a16.hip",
                  "bit_weight_only_awq_amd/csrc/w4a16_ops.hpp", "bit_weight_only_awq_amd/csrc/w4a8.hip",
                  "bit_weight_only_awq_amd/csrc/w4a8_fp8.hip",
                  "bit_weight_only_awq_amd/csrc/gemm_w4a8.hip", "bit_weight_only_awq_amd/csrc/stream.hip",
                  "bit_weight_only_awq_amd/csrc/device.hpp", "bit_weight_only_awq_amd/csrc/launch.hpp",
                  "bit_weight_only_awq_amd/csrc/api.cpp"]


def w4a16_weight_bytes(K, N, G=G, sym=False):
    return K * N // 2 + (K // G) * N * 2 + (0 if sym else (K // G) * N // 2)


def w4a16_alg_bytes(M, K, N, G=G):
    """Bytes the decode GEMV must move: packed weights, scales, zeros, X and Y."""
    return w4a16_weight_bytes(K, N, G) + M * K * 2 + M * N * 2


def w4a8_alg_bytes(M, K, N):
    return K * N // 2 + N * 2 + M * K + 4 * M + 2 * M * N


# sources the decode kernel is built from; its traffic counters stay valid while
# these and its launch plans for the decode layers (decode_digest) are unchanged
DECODE_SOURCES = ["bit_weight_only_awq_amd/csrc/w4a16.hip", "bit_weight_only_awq_amd/csrc/w4a16_ops.hpp",
                  "bit_weight_only_awq_amd/csrc/device.hpp"]


def decode_digest():
    """Digest of what the decode traffic depends on: the decode kernel's sources
    and the plans (grid, K split, chunking) of the four decode layers on a whole
    MI355X, so that planner changes elsewhere do not invalidate it."""
    import bit_weight_only_awq_amd as awq
    plans = [awq.plan_info(awq.AWQ_OP_GEMV_W4A16, M_DECODE, N, K, G, cu_count=256) for _, K, N in DECODE_LAYERS]
    h = hashlib.sha256(source_digest(DECODE_SOURCES).encode())
    h.update(json.dumps(plans, sort_keys=True).encode())
    return h.hexdigest()[:16]


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


def counter_rows(path):
    """{dispatch id: (kernel name, {counter: value})} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = out.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return dict(sorted(out.items()))


def pmc_summary(kernel, labels, paths):
    """CPU only: the counters of the last len(labels) `kernel` dispatches (the
    last repetition of a --profile run, one dispatch per label, in order) in
    rocprofv3 counter_collection.csv files (one per --pmc pass), summed over
    the chip; byte counters scaled by the calibration copy the --profile run
    launches first.  Prints one table per dispatch."""
    import csv
    out = [dict() for _ in labels]
    shape = [None] * len(labels)
    factors = {}
    for path in paths:
        with open(path) as f:
            rows = list(csv.DictReader(f))
        disp = {}
        for r in rows:
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                        "wg": int(r["Workgroup_Size"]), "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for d in disp.values():
            if "neg" in d["name"]:
                for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                    if ctr in d["c"]:
                        factors[ctr] = CAL_BYTES / (d["c"][ctr] * 1024.0)
        mine = [disp[i] for i in sorted(disp) if kernel in disp[i]["name"]][-len(labels):]
        if len(mine) != len(labels):
            raise SystemExit(f"{path}: {len(mine)} {kernel} dispatches, {len(labels)} labels")
        for k, d in enumerate(mine):
            out[k].update(d["c"])
            shape[k] = (d["name"].split("(")[0], d["grid"] // d["wg"], d["wg"])
    for lab, (name, wgs, wg), c in zip(labels, shape, out):
        print(f"{lab}: {name}  {wgs} workgroups x {wg} threads")
        for ctr in sorted(c):
            v = c[ctr]
            extra = ""
            if ctr in factors:
                extra = f"   ({v * 1024.0 * factors[ctr] / 1e6:.2f} MB after calibration x{factors[ctr]:.4f})"
            print(f"  {ctr:28s} {v:12.4e}{extra}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * c["GRBM_GUI_ACTIVE"] / 8)
            print(f"  matrix cores busy: {100 * busy:.1f} % of the cycles (1024 SIMDs, GRBM over 8 XCDs)")


def trace_summary(trace_csv):
    """CPU only: per-kernel and per-launch-shape durations from a rocprofv3
    --kernel-trace kernel_trace.csv (all dispatches of the run)."""
    import csv
    import statistics
    per_kernel, per_shape = {}, {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0][:60]
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            wg = (int(r["Workgroup_Size_X"]), int(r["Workgroup_Size_Y"]), int(r["Workgroup_Size_Z"]))
            grid = tuple(int(r[f"Grid_Size_{a}"]) // w for a, w in zip("XYZ", wg))
            per_kernel.setdefault(name, []).append(us)
            per_shape.setdefault((name, grid, wg[0] * wg[1] * wg[2]), []).append(us)
    total = sum(sum(v) for v in per_kernel.values())
    print(f"{'kernel':60s} {'calls':>7s} {'avg_us':>9s} {'pct':>7s}")
    for name, v in sorted(per_kernel.items(), key=lambda kv: -sum(kv[1])):
        print(f"{name:60s} {len(v):7d} {sum(v) / len(v):9.2f} {100 * sum(v) / total:7.2f}")
    print()
    print(f"{'kernel':48s} {'grid (wg x,y,z)':>16s} {'block':>6s} {'calls':>6s} {'median':>9s} {'min':>9s}")
    for (name, grid, blk), v in sorted(per_shape.items()):
        print(f"{name[:48]:48s} {','.join(map(str, grid)):>16s} {blk:6d} {len(v):6d} "
              f"{statistics.median(v):9.2f} {min(v):9.2f}")


def traffic_summary(fetch_csv, write_csv, kernel="w4a16_decode", name="w4a16_decode_m1_llama2_7b"):
    """HBM bytes per launch of `kernel` in a `--profile decode` run: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, one rocprofv3 pass each), each scaled by what
    the same counter reads for the calibration copy of CAL_BYTES read + CAL_BYTES
    written that the profile run launches first.  Writes
    profiles/<name>.traffic.json for bench.py's roofline object."""
    res = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = counter_rows(path)
        cal = [i for i, (k, _) in rows.items() if "neg" in k]
        if not cal:
            raise SystemExit(f"no calibration copy dispatch in {path}")
        cal_kib = rows[cal[-1]][1][ctr]
        factor = CAL_BYTES / (cal_kib * 1024.0)
        per_layer = {n: [] for n, _, _ in DECODE_LAYERS}
        launches = [(i, v) for i, (k, v) in rows.items() if i > cal[-1] and kernel in k]
        for n, (i, v) in enumerate(launches):
            per_layer[DECODE_LAYERS[n % len(DECODE_LAYERS)][0]].append(v[ctr] * 1024.0 * factor)
        res[ctr] = {"calibration_kib": cal_kib, "scale": round(factor, 5), "launches": len(launches),
                    "per_layer_bytes": {n: round(sum(b) / len(b)) for n, b in per_layer.items() if b}}
    layers = res["FETCH_SIZE"]["per_layer_bytes"]
    total = {n: layers[n] + res["WRITE_SIZE"]["per_layer_bytes"][n] for n in layers}
    alg = {n: w4a16_alg_bytes(1, K, N) for n, K, N in DECODE_LAYERS}
    out = {"kernel": kernel, "workload": "decode GEMV M=1, Llama-2-7B layer set, g128, weights rotated",
           "bytes_per_launch": round(sum(total.values()) / len(total)),
           "alg_bytes_per_launch": round(sum(alg.values()) / len(alg)),
           "per_layer": {n: {"hbm_bytes": total[n], "alg_bytes": alg[n], "ratio": round(total[n] / alg[n], 4)}
                         for n in total},
           "counters": res, "source_digest": decode_digest(),
           "command": ("rocprofv3 --pmc FETCH_SIZE -d gpurun_out/m/dfetch -o run --output-format csv "
                       "-- python3 bench.py --profile decode; "
                       "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/m/dwrite -o run --output-format csv "
                       "-- python3 bench.py --profile decode; "
                       "python3 bench.py --traffic gpurun_out/m/dfetch/run_counter_collection.csv "
                       "gpurun_out/m/dwrite/run_counter_collection.csv")}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}.traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(budget_s: float):
    """The oracle on the decode workload (M=1 over the Llama-2-7B layer set), run
    on this host's cores until about budget_s seconds of work are done; beside
    it, the oracle on the prefill workload (the Llama-3-8B layer set at M=2048)
    on a seeded subset of 256 of the 2048 rows (its time scaled to the full
    layer, labelled as scaled), and one decode pass on a single thread."""
    import torch

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
    out = {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"decode M=1 on the Llama-2-7B layer set (4 layers, {mb:.1f} MB of weights) x {reps} "
                     f"passes in {dt:.1f} s; fp64 scalar C oracle on {cores} threads"}
    # one decode pass, single-threaded
    t0 = time.perf_counter()
    for c in cases:
        orc.w4a16(c.x, c.qweight, c.scales, c.qzeros, G, nthreads=1)
    dt1 = time.perf_counter() - t0
    out["single_thread"] = {"value": round(mb / 1e3 / dt1, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"one decode pass (4 layers) in {dt1:.1f} s"}
    # prefill: 256 of the 2048 rows of each layer, time scaled by 2048 / 256
    rows, flops, tg = 256, 0.0, 0.0
    for name, K, N in PREFILL_LAYERS:
        c = synthgen.w4a16_case(M_PREFILL, K, N, G, seed=synthgen.seed_for(f"bench|prefill|{name}"),
                                x_rows=M_PREFILL)
        g = torch.Generator().manual_seed(synthgen.seed_for(f"cpu|rows|{name}"))
        sel = torch.randperm(M_PREFILL, generator=g)[:rows].sort().values
        t0 = time.perf_counter()
        orc.w4a16(c.x[sel], c.qweight, c.scales, c.qzeros, G, nthreads=cores)
        tg += (time.perf_counter() - t0) * (M_PREFILL / rows)
        flops += 2.0 * M_PREFILL * N * K
    out["gemm_m2048"] = {"value": round(flops / tg / 1e9, 3), "unit": "GFLOP/s", "cores": cores, "scaled": True,
                         "sample": f"prefill GEMM M=2048 on the Llama-3-8B layer set, a seeded subset of {rows} "
                                   f"rows per layer; time scaled by {M_PREFILL // rows} to {tg:.1f} s for the "
                                   f"whole pass"}
    return out


def roof_frac(t, flops, alg_bytes, peak_t):
    """Fraction of the roofline: the time at min(MFMA peak, intensity x HBM) over the measured time."""
    t_roof = max(flops / (peak_t * 1e12), alg_bytes / (HBM_PEAK_GBS * 1e9))
    return round(t_roof / t, 4), ("mfma" if flops / (peak_t * 1e12) >= alg_bytes / (HBM_PEAK_GBS * 1e9) else "hbm")


def config_sweeps(awq, synthgen, torch, dev, per_launch, decode, n_copies, comparator):
    """Every configuration of the workloads beyond the headline step, timed per
    layer (graphs of one layer; weights rotated through >= ROTATE_MB of copies
    wherever the weights dominate the bytes, so they stream from HBM):
      cfg0: opt-125m fc1 (M=16, K=768, N=3072; fits in L2, absolute time);
      cfg1: decode GEMV M in {1, 2, 4, 8} on the Llama-2-7B layer set;
      cfg2: prefill GEMM M in {64, 256, 1024, 2048, 4096} on the Llama-3-8B
            layer set, with the dequantise + vendor dense GEMM route beside it
            for M >= 256;
      cfg3: K=4096, N=14336, M in {1, 512} x G in {32, 64, 128} x {fp16, bf16}
            x {zero point, symmetric};
      cfg4: W4A8 on the QQQ shape, M in {1, 16, 64, 256, 1024}, per-channel
            and g128 (whole layer: quantisation + GEMM; and the GEMM alone).
    Each entry carries the fraction of min(MFMA peak, intensity x HBM) it reaches."""
    f16 = torch.float16
    res = {}

    def rotate(tensors, nbytes):
        ncp = max(2, -(-ROTATE_MB * 10 ** 6 // nbytes))
        return [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(ncp - 1)]

    # cfg0
    c = synthgen.w4a16_case(16, 768, 3072, 128, seed=0)
    x0, q0, s0, z0 = (t.to(dev) for t in (c.x, c.qweight, c.scales, c.qzeros))
    y0 = torch.empty(16, 3072, dtype=f16, device=dev)
    t = per_launch(lambda: awq.gemm_w4a16(x0, q0, s0, z0, 128, out=y0), 1)
    res["cfg0_opt125m_fc1_M16"] = {"us": round(t * 1e6, 2), "TFLOPs": round(2 * 16 * 768 * 3072 / t / 1e12, 2),
                                   "note": "1.35 MB: served from L2, launch-latency bound; absolute time"}

    # cfg1: the decode copies already rotate the Llama-2-7B weights
    cfg1 = {}
    for M in (1, 2, 4, 8):
        for li, (name, K, N) in enumerate(DECODE_LAYERS):
            x = synthgen.activations(M, K, seed=synthgen.seed_for(f"bench|cfg1|{M}|{K}")).to(dev)
            y = torch.empty(M, N, dtype=f16, device=dev)
            t = per_launch(lambda x=x, y=y, li=li: [awq.gemv_w4a16(x, decode[r][li][1], decode[r][li][2],
                                                                   decode[r][li][3], G, out=y)
                                                    for r in range(n_copies)], n_copies)
            ab = w4a16_alg_bytes(M, K, N)
            fr, bound = roof_frac(t, 2 * M * N * K, ab, MFMA_F16_PEAK_TFLOPS)
            cfg1[f"M={M} {name} {K}x{N}"] = {"us": round(t * 1e6, 2),
                                             "weight_GBs": round(w4a16_weight_bytes(K, N) / t / 1e9, 1),
                                             "frac_roofline": fr, "bound": bound}
    res["cfg1_decode_llama2_7b"] = cfg1

    # cfg2
    cfg2 = {}
    xs = {K: synthgen.activations(4096, K, seed=synthgen.seed_for(f"bench|cfg2|x|{K}")).to(dev)
          for K in {K for _, K, _ in PREFILL_LAYERS}}
    for name, K, N in PREFILL_LAYERS:
        cw = synthgen.w4a16_case(1, K, N, G, seed=synthgen.seed_for(f"bench|cfg2|w|{name}"))
        base = tuple(t.to(dev) for t in (cw.qweight, cw.scales, cw.qzeros))
        copies = rotate(base, w4a16_weight_bytes(K, N))
        ybuf = torch.empty(4096, N, dtype=f16, device=dev)
        wd = awq.dequant_w4a16(*base, G) if comparator else None
        for M in (64, 256, 1024, 2048, 4096):
            x, y = xs[K][:M], ybuf[:M]
            ncp = len(copies) if M <= 256 else 1
            t = per_launch(lambda x=x, y=y, ncp=ncp: [awq.gemm_w4a16(x, *copies[r], G, out=y) for r in range(ncp)],
                           ncp, reps=3)
            flops = 2 * M * N * K
            fr, bound = roof_frac(t, flops, w4a16_alg_bytes(M, K, N), MFMA_F16_PEAK_TFLOPS)
            e = {"us": round(t * 1e6, 2), "TFLOPs": round(flops / t / 1e12, 1), "frac_roofline": fr, "bound": bound,
                 "weights": "rotated" if ncp > 1 else "one copy (MFMA-bound)"}
            if comparator and M >= 256:
                tdq = per_launch(lambda: awq.dequant_w4a16(*base, G, out=wd), 1, reps=3)
                tmm = per_launch(lambda x=x, y=y: torch.matmul(x, wd, out=y), 1, reps=3)
                e["dequant_plus_dense"] = {"dequant_us": round(tdq * 1e6, 2), "dense_us": round(tmm * 1e6, 2),
                                           "total_us": round((tdq + tmm) * 1e6, 2),
                                           "dense_TFLOPs": round(flops / tmm / 1e12, 1),
                                           "speedup_of_fused": round((tdq + tmm) / t, 3)}
            cfg2[f"M={M} {name} {K}x{N}"] = e
        del copies, wd, ybuf
    del xs
    res["cfg2_prefill_llama3_8b"] = cfg2

    # cfg3
    cfg3 = {}
    K, N = 4096, 14336
    x1 = {dt: synthgen.activations(512, K, dtype=dt, seed=synthgen.seed_for(f"bench|cfg3|x|{dt}")).to(dev)
          for dt in ("f16", "bf16")}
    for Gv in (32, 64, 128):
        for sym in (False, True):
            cw = synthgen.w4a16_case(1, K, N, Gv, sym=sym, seed=synthgen.seed_for(f"bench|cfg3|{Gv}|{sym}"))
            qw = cw.qweight.to(dev)
            qz = None if sym else cw.qzeros.to(dev)
            wb = w4a16_weight_bytes(K, N, Gv, sym)
            for dt in ("f16", "bf16"):
                sc = cw.scales.to(torch.bfloat16 if dt == "bf16" else f16).to(dev)
                copies = rotate((qw, sc) + (() if sym else (qz,)), wb)
                for M in (1, 512):
                    x = x1[dt][:M]
                    y = torch.empty(M, N, dtype=x.dtype, device=dev)
                    fn = awq.gemv_w4a16 if M == 1 else awq.gemm_w4a16
                    ncp = len(copies) if M == 1 else 1
                    t = per_launch(lambda x=x, y=y, fn=fn, ncp=ncp, copies=copies:
                                   [fn(x, copies[r][0], copies[r][1], None if sym else copies[r][2], Gv, out=y)
                                    for r in range(ncp)], ncp, reps=3)
                    ab = wb + M * K * 2 + M * N * 2
                    fr, bound = roof_frac(t, 2 * M * N * K, ab, MFMA_F16_PEAK_TFLOPS)
                    cfg3[f"M={M} g{Gv} {dt} {'sym' if sym else 'zp'}"] = {
                        "us": round(t * 1e6, 2), "frac_roofline": fr, "bound": bound,
                        **({"weight_GBs": round(wb / t / 1e9, 1)} if M == 1 else
                           {"TFLOPs": round(2 * M * N * K / t / 1e12, 1)})}
                del copies
    del x1
    res["cfg3_variants_4096x14336"] = cfg3

    # cfg4
    cfg4 = {}
    K, N = W4A8_K, W4A8_N
    for Gv in (-1, 128):
        c8 = synthgen.w4a8_case(1, K, N, Gv, seed=synthgen.seed_for(f"bench|cfg4|w|{Gv}"))
        parts = (c8.b.to(dev), c8.s2.to(dev)) + (() if Gv < 0 else (c8.s3.to(dev),))
        copies = rotate(parts, K * N // 2)
        for M in (1, 16, 64, 256, 1024):
            x = synthgen.activations(M, K, seed=synthgen.seed_for(f"bench|cfg4|x|{M}")).to(dev)
            a8 = torch.empty(M, K, dtype=torch.int8, device=dev)
            s1 = torch.empty(M, dtype=torch.float32, device=dev)
            y = torch.empty(M, N, dtype=f16, device=dev)
            ncp = len(copies) if M <= 64 else 1

            def s3_of(r):
                return None if Gv < 0 else copies[r][2]
            tl = per_launch(lambda x=x, y=y, a8=a8, s1=s1, ncp=ncp:
                            [awq.linear_w4a8(x, copies[r][0], copies[r][1], s3_of(r), Gv, out=y, a8=a8, s1=s1)
                             for r in range(ncp)], ncp, reps=3)
            awq.quant_act(x, a8, s1)
            tg = per_launch(lambda y=y, a8=a8, s1=s1, ncp=ncp:
                            [awq.w4a8_gemm(a8, copies[r][0], s1, copies[r][1], s3_of(r), Gv, out=y)
                             for r in range(ncp)], ncp, reps=3)
            ops = 2 * M * N * K
            ab = w4a8_alg_bytes(M, K, N) + (0 if Gv < 0 else (K // Gv) * N * 2)
            fr, bound = roof_frac(tg, ops, ab, MFMA_I8_PEAK_TOPS)
            frl, _ = roof_frac(tl, ops, ab + 3 * M * K, MFMA_I8_PEAK_TOPS)
            cfg4[f"M={M} {'per-channel' if Gv < 0 else 'g128'}"] = {
                "layer_us": round(tl * 1e6, 2), "gemm_us": round(tg * 1e6, 2),
                "gemm_TOPs": round(ops / tg / 1e12, 1), "gemm_frac_roofline": fr, "layer_frac_roofline": frl,
                "bound": bound}
        del copies
    res["cfg4_w4a8_qqq_n8192_k21760"] = cfg4

    # INT4-FP8 W4A8 (E4M3 activations) on the QQQ shape and the target shapes:
    # quantisation and GEMM timed separately, and the whole layer through
    # w4a8_fp8_linear (one fused kernel for a single token); the GEMM's
    # roofline is the fp8 matrix-core peak (5033 TFLOP/s dense), weights
    # rotated at M <= 64
    fp8 = {}
    shapes = [(M, W4A8_K, W4A8_N) for M in (1, 16, 64, 256, 1024)] + \
             [(M, K, N) for K, N in TARGET_SHAPES for M in M_TARGETS]
    wsets = {}
    for M, K, N in shapes:
        if (K, N) not in wsets:
            c8 = synthgen.w4a8_case(1, K, N, -1, seed=synthgen.seed_for(f"bench|fp8|w|{K}|{N}"))
            wsets[(K, N)] = rotate((c8.b.to(dev), c8.s2.to(dev)), K * N // 2)
        copies = wsets[(K, N)]
        x = synthgen.activations(M, K, seed=synthgen.seed_for(f"bench|fp8|x|{M}|{K}")).to(dev)
        a, s1, asum = awq.quant_act_fp8(x)
        y = torch.empty(M, N, dtype=f16, device=dev)
        ncp = len(copies) if M <= 64 else 1
        tq = per_launch(lambda x=x, a=a, s1=s1, asum=asum: awq.quant_act_fp8(x, a, s1, asum), 1, reps=3)
        tg = per_launch(lambda a=a, s1=s1, asum=asum, y=y, ncp=ncp, copies=copies:
                        [awq.w4a8_fp8_gemm(a, copies[r][0], s1, asum, copies[r][1], out=y) for r in range(ncp)],
                        ncp, reps=3)
        tl = per_launch(lambda x=x, a=a, s1=s1, asum=asum, y=y, ncp=ncp, copies=copies:
                        [awq.linear_w4a8_fp8(x, copies[r][0], copies[r][1], out=y, a=a, s1=s1, asum=asum)
                         for r in range(ncp)], ncp, reps=3)
        flops = 2 * M * N * K
        ab = w4a8_alg_bytes(M, K, N) + 4 * M  # + asum
        fr, bound = roof_frac(tg, flops, ab, MFMA_I8_PEAK_TOPS)
        fp8[f"M={M} K={K} N={N}"] = {"quant_us": round(tq * 1e6, 2), "gemm_us": round(tg * 1e6, 2),
                                     "layer_us": round(tl * 1e6, 2), "fused_quant": M == 1,
                                     "gemm_TFLOPs": round(flops / tg / 1e12, 1), "gemm_frac_roofline": fr,
                                     "bound": bound}
    del wsets
    res["w4a8_int4_fp8"] = fp8

    # the read probe over 2 GiB: the asymptotic read rate of the device
    big = torch.empty(2 ** 31 // 2, dtype=f16, device=dev)
    big.fill_(1.0)
    sink = torch.empty(awq.ops.STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    t = per_launch(lambda: awq.stream_read(big, sink), 1, reps=3)
    res["stream_read_2GiB"] = {"us": round(t * 1e6, 1), "GBs": round(2 ** 31 / t / 1e9, 1),
                               "frac_hbm": round(2 ** 31 / t / 1e9 / HBM_PEAK_GBS, 4)}
    del big
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparator", action="store_true", help="skip the dense fp16 GEMM comparator")
    ap.add_argument("--no-sweeps", action="store_true", help="skip the per-configuration sweeps")
    ap.add_argument("--profile", choices=["decode", "prefill", "w4a8", "targets"], default=None,
                    help="no timing: run one phase eagerly --profile-reps times (for rocprofv3 counter passes), "
                         "after a 256 MiB device copy of known size that calibrates the byte counters")
    ap.add_argument("--profile-reps", type=int, default=3)
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="CPU only: summarise the two counter passes of `--profile decode` into "
                         "profiles/w4a16_decode_m1_llama2_7b.traffic.json")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("KERNEL LABELS", "CSV"),
                    help="CPU only: print the counters of the last KERNEL dispatches, one per comma-separated "
                         "label, from counter CSVs of a --profile run (one per --pmc pass)")
    ap.add_argument("--trace-summary", metavar="TRACE_CSV",
                    help="CPU only: per-kernel and per-launch-shape durations from a rocprofv3 kernel_trace.csv")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic:
        traffic_summary(*args.traffic)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1].split(","), args.pmc_summary[2:])
        return
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
    # target shapes: W4A16 and W4A8 at M=1 (weights rotated through >= ROTATE_MB of
    # copies) and M=2048 on (4096, 4096) and (4096, 14336)
    tgt = []
    for K, N in TARGET_SHAPES:
        c = synthgen.w4a16_case(1, K, N, G, seed=synthgen.seed_for(f"bench|target|w4a16|{K}|{N}"))
        ncp = max(2, -(-ROTATE_MB * 10 ** 6 // w4a16_weight_bytes(K, N)))
        base = (c.qweight.to(dev), c.scales.to(dev), c.qzeros.to(dev))
        wcopies = [base] + [tuple(t.clone() for t in base) for _ in range(ncp - 1)]
        c8 = synthgen.w4a8_case(1, K, N, -1, seed=synthgen.seed_for(f"bench|target|w4a8|{K}|{N}"))
        b8 = (c8.b.to(dev), c8.s2.to(dev))
        w8copies = [b8] + [tuple(t.clone() for t in b8) for _ in range(ncp - 1)]
        xs = {M: synthgen.activations(M, K, seed=synthgen.seed_for(f"bench|target|x|{M}|{K}")).to(dev)
              for M in M_TARGETS}
        tgt.append({"K": K, "N": N, "w": wcopies, "w8": w8copies, "x": xs,
                    "y": {M: torch.empty(M, N, dtype=torch.float16, device=dev) for M in M_TARGETS},
                    "a8": {M: torch.empty(M, K, dtype=torch.int8, device=dev) for M in M_TARGETS},
                    "s1": {M: torch.empty(M, dtype=torch.float32, device=dev) for M in M_TARGETS}})
    sink = torch.empty(awq.ops.STREAM_SINK_WORDS, dtype=torch.int32, device=dev)

    def run_decode(r, layers=None):
        for li in (layers if layers is not None else range(len(DECODE_LAYERS))):
            x, qw, s, qz, y = decode[r][li]
            awq.gemv_w4a16(x, qw, s, qz, G, out=y)

    def run_prefill(layers=None):
        for li in (layers if layers is not None else range(len(PREFILL_LAYERS))):
            x, qw, s, qz, y = prefill[li]
            awq.gemm_w4a16(x, qw, s, qz, G, out=y)

    def run_w4a8(r, which=None):
        # the whole layer per call: per-token quantisation fused into the GEMM
        # at M = 1, quantisation then GEMM otherwise (w4a8_linear)
        b, s2 = w8w[r]
        for i in (which if which is not None else range(len(w8a))):
            M, x, a8, s1, y = w8a[i]
            awq.linear_w4a8(x, b, s2, out=y, a8=a8, s1=s1)

    def run_target(t, M, kind, r=0):
        x, y = t["x"][M], t["y"][M]
        if kind == "w4a16":
            qw, sc, qz = t["w"][r % len(t["w"])]
            (awq.gemv_w4a16 if M <= 8 else awq.gemm_w4a16)(x, qw, sc, qz, G, out=y)
        else:
            b, s2 = t["w8"][r % len(t["w8"])]
            awq.linear_w4a8(x, b, s2, out=y, a8=t["a8"][M], s1=t["s1"][M])

    def run_targets():
        for t in tgt:
            for M in M_TARGETS:
                for kind in ("w4a16", "w4a8"):
                    run_target(t, M, kind)

    # every op once eagerly: allocates the shared workspace before capture
    run_decode(0)
    run_prefill()
    run_w4a8(0)
    run_targets()
    torch.cuda.synchronize()

    if args.profile:
        # copy kernel of known size first (an elementwise negation: 256 MiB read,
        # 256 MiB written): the counters it produces calibrate the HBM byte
        # counts of the phase that follows
        cal_src = torch.ones(CAL_BYTES // 2, dtype=torch.float16, device=dev)
        cal_dst = torch.empty_like(cal_src)
        for _ in range(2):
            torch.neg(cal_src, out=cal_dst)
        torch.cuda.synchronize()
        del cal_src, cal_dst
        for rep in range(args.profile_reps):
            if args.profile == "decode":
                for r in range(n_copies):
                    run_decode(r)
            elif args.profile == "prefill":
                run_prefill()
            elif args.profile == "w4a8":
                run_w4a8(rep % w8_copies)
            else:
                run_targets()
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "reps": args.profile_reps, "decode_weight_copies": n_copies}))
        return

    cap = torch.cuda.Stream(dev)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn()
        return g

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    stream = torch.cuda.current_stream(dev)

    # warm-up passes, eagerly
    for i in range(args.warmup):
        run_decode(i % n_copies)
        run_prefill()
        run_w4a8(i % w8_copies)
    torch.cuda.synchronize()

    # Timed region: exactly K passes of each phase.  Each phase is one HIP graph
    # holding its K passes back to back (weights rotate through the copies), so
    # the per-graph launch cost is paid once per phase, not once per pass.
    K_ = args.steps
    g_dec = capture(lambda: [run_decode((args.warmup + i) % n_copies) for i in range(K_)])
    g_pre = capture(lambda: [run_prefill() for _ in range(K_)])
    g_w8 = capture(lambda: [run_w4a8((args.warmup + i) % w8_copies) for i in range(K_)])
    torch.cuda.synchronize()
    e = [ev() for _ in range(4)]
    wall0 = time.perf_counter()
    e[0].record(stream)
    g_dec.replay()
    e[1].record(stream)
    g_pre.replay()
    e[2].record(stream)
    g_w8.replay()
    e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    t_dec = e[0].elapsed_time(e[1]) / 1e3 / K_   # seconds per pass
    t_pre = e[1].elapsed_time(e[2]) / 1e3 / K_
    t_w8 = e[2].elapsed_time(e[3]) / 1e3 / K_
    ms_step = e[0].elapsed_time(e[3]) / K_
    del g_dec, g_pre, g_w8

    # per-layer / per-kernel times (outside the timed steps): one graph per
    # layer with launches over rotating weight copies, replayed a few times.
    # A graph holds at least PER_LAUNCH_MIN launches (the rotation repeated),
    # so that the replay's own start-up cost is spread thin.
    def per_launch(fn, launches, reps=4):
        inner = max(1, -(-PER_LAUNCH_MIN // launches))
        g = capture(lambda: [fn() for _ in range(inner)])
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / (reps * launches * inner)

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
    # comparator, not a library path: the vendor dense fp16 GEMM (hipBLASLt via
    # torch.matmul) on the same M=2048 shapes with weights already dequantised
    # to fp16 (4x the weight memory; the dequantisation is left out)
    dense = {}
    if not args.no_comparator:
        dshapes = [(name, K, N) for name, K, N in PREFILL_LAYERS] + \
                  [(f"target {K}x{N}", K, N) for K, N in TARGET_SHAPES]
        for name, K, N in dshapes:
            xd = synthgen.activations(M_PREFILL, K, seed=synthgen.seed_for(f"bench|dense|x|{K}")).to(dev)
            wd = (synthgen.activations(K, N, seed=synthgen.seed_for(f"bench|dense|w|{K}|{N}")) * 0.02).to(dev)
            yd = torch.empty(M_PREFILL, N, dtype=torch.float16, device=dev)
            torch.matmul(xd, wd, out=yd)
            t = per_launch(lambda xd=xd, wd=wd, yd=yd: torch.matmul(xd, wd, out=yd), 1, reps=3)
            dense[name] = {"K": K, "N": N, "us": round(t * 1e6, 2),
                           "TFLOPs": round(2 * M_PREFILL * N * K / t / 1e12, 1)}
            del xd, wd, yd
    # the vendor dense int8 GEMM (hipBLASLt via torch._int_mm, int32 out) on
    # the W4A8 shapes with weights already unpacked to int8 (2x the weight
    # memory; no scales applied): context for the W4A8 GEMM, not a library path
    dense8 = {}
    if not args.no_comparator:
        for M, K, N in [(1024, W4A8_K, W4A8_N)] + [(M_PREFILL, K, N) for K, N in TARGET_SHAPES]:
            name = f"M={M} K={K} N={N}"
            try:
                g8 = torch.Generator().manual_seed(synthgen.seed_for(f"bench|dense8|{M}|{K}|{N}"))
                a8d = torch.randint(-128, 128, (M, K), generator=g8, dtype=torch.int8).to(dev)
                w8d = torch.randint(-8, 8, (N, K), generator=g8, dtype=torch.int8).to(dev).t()
                torch._int_mm(a8d, w8d)
                t = per_launch(lambda a8d=a8d, w8d=w8d: torch._int_mm(a8d, w8d), 1, reps=3)
                dense8[name] = {"us": round(t * 1e6, 2), "TOPs": round(2 * M * N * K / t / 1e12, 1)}
                del a8d, w8d
            except RuntimeError as e:  # not every torch build has an int8 GEMM
                dense8[name] = {"error": str(e).splitlines()[0][:120]}
    def w4a8_times(M, x, a8, s1, y, s2s, fused):
        tq = per_launch(lambda: [awq.quant_act(x, a8, s1) for _ in range(4)], 4)
        tg = per_launch(lambda: [awq.w4a8_gemm(a8, w8w[r][0], s1, s2s[r], out=y) for r in range(w8_copies)],
                        w8_copies)
        tl = per_launch(lambda: [awq.linear_w4a8(x, w8w[r][0], s2s[r], out=y, a8=a8, s1=s1)
                                 for r in range(w8_copies)], w8_copies)
        ops = 2 * M * W4A8_N * W4A8_K
        return {"layer_us": round(tl * 1e6, 2), "fused_quant": fused,
                "quant_us": round(tq * 1e6, 2), "gemm_us": round(tg * 1e6, 2),
                "gemm_TOPs": round(ops / tg / 1e12, 2),
                "gemm_weight_GBs": round((W4A8_K * W4A8_N // 2 + 2 * W4A8_N) / tg / 1e9, 1),
                "frac_hbm": round(w4a8_alg_bytes(M, W4A8_K, W4A8_N) / tg / 1e9 / HBM_PEAK_GBS, 4),
                "frac_i8_mfma": round(ops / tg / 1e12 / MFMA_I8_PEAK_TOPS, 4)}

    w8_res = {f"M={M}": w4a8_times(M, x, a8, s1, y, [s2 for _, s2 in w8w], M == 1) for M, x, a8, s1, y in w8a}
    # the same layers with bf16 activations, scales and output
    s2_bf = [s2.to(torch.bfloat16) for _, s2 in w8w]
    w8_bf = {}
    for M, x, a8, s1, _y in w8a:
        w8_bf[f"M={M}"] = w4a8_times(M, x.to(torch.bfloat16), a8, s1,
                                     torch.empty(M, W4A8_N, dtype=torch.bfloat16, device=dev), s2_bf, M == 1)
    del s2_bf

    # achievable read rate at each decode layer's byte count: the bandwidth probe
    # streaming the same packed-weight tensors (same rotation)
    for li, (name, K, N) in enumerate(DECODE_LAYERS):
        t = per_launch(lambda li=li: [awq.stream_read(decode[r][li][1], sink) for r in range(n_copies)], n_copies)
        nb = K * N // 2
        dec_layer[name]["stream_read_us"] = round(t * 1e6, 3)
        dec_layer[name]["stream_read_GBs"] = round(nb / t / 1e9, 1)
        dec_layer[name]["frac_of_stream"] = round(dec_layer[name]["weight_GBs"] / (nb / t / 1e9), 4)

    targets = {}
    for t in tgt:
        K, N = t["K"], t["N"]
        for M in M_TARGETS:
            ncp = len(t["w"]) if M == 1 else 1
            for kind in ("w4a16", "w4a8"):
                tt = per_launch(lambda t=t, M=M, kind=kind, ncp=ncp: [run_target(t, M, kind, r) for r in range(ncp)],
                                ncp, reps=4 if M == 1 else 3)
                key = f"{kind} M={M} K={K} N={N}"
                ops = 2 * M * N * K
                if kind == "w4a16":
                    ab = w4a16_alg_bytes(M, K, N)
                    peak = MFMA_F16_PEAK_TFLOPS
                else:
                    ab = w4a8_alg_bytes(M, K, N) + 3 * M * K  # + the quant pass (reads x fp16, writes a8)
                    peak = MFMA_I8_PEAK_TOPS
                r = {"us": round(tt * 1e6, 2)}
                if M == 1:
                    r["alg_GBs"] = round(ab / tt / 1e9, 1)
                    r["frac_hbm"] = round(ab / tt / 1e9 / HBM_PEAK_GBS, 4)
                else:
                    r["T_per_s"] = round(ops / tt / 1e12, 1)
                    r["frac_mfma"] = round(ops / tt / 1e12 / peak, 4)
                targets[key] = r

    sweeps = None if args.no_sweeps else config_sweeps(awq, synthgen, torch, dev, per_launch, decode, n_copies,
                                                       not args.no_comparator)

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
                        "traffic": load_traffic("w4a16_decode_m1_llama2_7b", decode_digest()),
                        "avg_launch_us": round(t_dec / len(DECODE_LAYERS) * 1e6, 3),
                        "per_layer": dec_layer},
           "gemm_m2048": {"kernel": "w4a16_gemm (prefill GEMM, M=2048, 4 Llama-3-8B layers back to back)",
                          "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                          "per_layer_note": "each layer repeated alone in its graph: its weights and X stay in "
                                            "the 256 MB MALL between launches (cache-warm), so the per-layer "
                                            "times sum to less than the timed four-layer pass",
                          "per_layer": pre_layer},
           "w4a8_n8192_k21760": w8_res,
           "w4a8_bf16_n8192_k21760": w8_bf,
           "comparator_dense_fp16_m2048": {"note": "vendor dense fp16 GEMM (hipBLASLt via torch.matmul) on "
                                                   "pre-dequantised weights; context, not a library path",
                                           **dense},
           "comparator_dense_int8": {"note": "vendor dense int8 GEMM (torch._int_mm, int32 out) on weights "
                                             "pre-unpacked to int8, no scales; context, not a library path",
                                     **dense8},
           "targets": {"note": "W4A8 times are whole-layer calls (w4a8_linear): activation quantisation included, fused into the GEMM at M=1", **targets},
           "phases_us": {"decode": round(t_dec * 1e6, 2), "prefill": round(t_pre * 1e6, 2),
                         "w4a8": round(t_w8 * 1e6, 2)}}
    if sweeps is not None:
        out["configs"] = sweeps
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
