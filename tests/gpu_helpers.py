"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

# Tolerances of the fp16 path (stated for this hot path): relative Frobenius
# error 2e-3 and max abs error 0.05 against the fp64 oracle.  bf16 output
# rounding alone is up to 2^-8 |y|, so bf16 gets rel-Frobenius 1e-2 and a
# per-element bound 0.05 + 2^-8 |y|.
F16_REL, F16_ABS = 2e-3, 0.05
BF16_REL = 1e-2

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def dev():
    return torch.device("cuda", 0)


def orc():
    return oracle.get()


def to_dev(*ts):
    return [None if t is None else t.to(dev()) for t in ts]


def check_fp(y_gpu: torch.Tensor, y64: np.ndarray, dtype: str = "f16", what: str = ""):
    """Compare a GPU fp16/bf16 result with the fp64 oracle; returns the metrics."""
    y = y_gpu.detach().float().cpu().double().numpy()
    assert y.shape == y64.shape, (y.shape, y64.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y - y64)
    nrm = np.linalg.norm(y64)
    rel = float(np.linalg.norm(y - y64) / nrm) if nrm > 0 else float(np.linalg.norm(y - y64))
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f16":
        assert rel <= F16_REL and mx <= F16_ABS, f"{what}: rel={rel:.3e} maxabs={mx:.3e}"
    else:
        bound = 0.05 + 2.0 ** -8 * np.abs(y64)
        worst = float((err - bound).max()) if err.size else -1.0
        assert rel <= BF16_REL and worst <= 0, f"{what}: rel={rel:.3e} maxabs={mx:.3e} bound excess={worst:.3e}"
    return rel, mx


def sample_rows(M: int, n: int = 12, seed: int = 0, tile: int = 256) -> np.ndarray:
    """Rows to check with the oracle at sizes it cannot do whole: the first and
    last rows of the matrix and of a 16-row tile boundary, one random row in
    every `tile`-row block (so no workgroup row tile goes unchecked), plus
    random ones."""
    if M <= n + 4:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, M // 2, M - 17, M - 2, M - 1]
    per_tile = [b + int(rng.integers(0, min(tile, M - b))) for b in range(0, M, tile)]
    rnd = rng.choice(M, size=n, replace=False)
    return np.unique(np.concatenate([fixed, per_tile, rnd]).clip(0, M - 1))
