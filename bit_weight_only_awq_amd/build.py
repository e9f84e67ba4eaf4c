"""Build libawq4.so (gfx950) in-tree with hipcc.

Usage: python -m bit_weight_only_awq_amd.build   (or build() from Python).
Every source is compiled for gfx950 only; the result is placed next to this
file, where the ctypes binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libawq4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["pack.hip", "dequant.hip", "w4a16.hip", "stream_w4a16.hip", "gemm_w4a16.hip", "w4a8.hip", "w4a8_fp8.hip", "gemm_w4a8_fp8.hip", "gemm_w4a8.hip", "stream.hip", "api.cpp"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops (the host
# pass does not know the feature and warns; that is expected).
FLAGS = ["-O3", "--offload-arch=gfx950", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-fast-math"]


def build(verbose: bool = False) -> str:
    tmp = tempfile.mkdtemp(prefix="awq4_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                     text=True)))
        failed = []
        for src, cmd, p in procs:
            out, _ = p.communicate()
            msgs = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                failed.append((src, "\n".join(msgs)))
            elif verbose and msgs:
                print(f"[{src}]\n" + "\n".join(msgs))
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"== {s}\n{m}" for s, m in failed))
        tmp_lib = LIB + ".tmp"
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib], check=True,
                       capture_output=True, text=True)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
