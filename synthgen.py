"""Seeded synthetic inputs for the 4-bit-weight GEMM hot path.

This module serves both the GPU path and the CPU oracle.  It holds none of the
method's arithmetic: only random draws and dtype casts.  Packed words are drawn
directly as uniform random 32-bit integers -- eight independent uniform 4-bit
fields per word -- so no packing code is needed to make them.

Value distributions follow the workloads the pages measure on (Llama-2-7B,
Llama-3-8B, opt-125m layer shapes and the QQQ N=8192, K=21760 GEMM):
  * activations X ~ N(0, 1), cast to fp16 or bf16 (round to nearest even);
  * qweight / qzeros: uniform 4-bit fields 0..15 (AWQ) or -8..7 (W4A8,
    two's complement), i.e. uniform random int32 words;
  * scales ~ U[0.002, 0.02] cast to the activation dtype;
  * W4A8 per-group scales: integers 1..16 (stored as fp16), with the
    per-channel scale drawn as U[0.002, 0.02] / 16 so the output has the same
    magnitude as the per-channel case.
Seeds: 0 for the small opt-125m case, otherwise crc32 of a key naming the
shape, so every case is reproducible in isolation.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import torch

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def seed_for(key: str) -> int:
    """Stable 32-bit seed for a case key (crc32)."""
    return zlib.crc32(key.encode()) & 0xFFFFFFFF


def case_key(kind: str, M: int, K: int, N: int, G: int, dtype: str = "f16", sym: bool = False) -> str:
    return f"{kind}|{M}|{K}|{N}|{G}|{dtype}|{'sym' if sym else 'zp'}"


def _words(g: torch.Generator, shape) -> torch.Tensor:
    """Uniform random int32 words (eight uniform 4-bit fields each)."""
    return torch.randint(-(2 ** 31), 2 ** 31, shape, generator=g, dtype=torch.int64).to(torch.int32)


@dataclass
class W4A16Case:
    x: torch.Tensor        # [M, K] fp16/bf16
    qweight: torch.Tensor  # [K, N/8] int32
    qzeros: torch.Tensor | None  # [K/G, N/8] int32, None = symmetric
    scales: torch.Tensor   # [K/G, N] fp16/bf16
    M: int
    K: int
    N: int
    G: int
    dtype: str
    seed: int


def w4a16_case(M: int, K: int, N: int, G: int = 128, dtype: str = "f16", sym: bool = False,
               seed: int | None = None, x_rows: int | None = None) -> W4A16Case:
    """Inputs for Y = X . dequant(qweight, qzeros, scales).

    ``x_rows`` (default M) lets a caller draw the weights of a shape once and
    only a few activation rows (the weights do not depend on M)."""
    if seed is None:
        seed = seed_for(case_key("w4a16", M, K, N, G, dtype, sym))
    g = torch.Generator().manual_seed(seed)
    dt = _DT[dtype]
    qweight = _words(g, (K, N // 8))
    qzeros = None if sym else _words(g, (K // G, N // 8))
    scales = (0.002 + 0.018 * torch.rand(K // G, N, generator=g, dtype=torch.float32)).to(dt)
    x = torch.randn(M if x_rows is None else x_rows, K, generator=g, dtype=torch.float32).to(dt)
    return W4A16Case(x, qweight, qzeros, scales, M, K, N, G, dtype, seed)


def activations(M: int, K: int, dtype: str = "f16", seed: int = 0) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn(M, K, generator=g, dtype=torch.float32).to(_DT[dtype])


def activations_on(device, M: int, K: int, dtype: str = "f16", seed: int = 0) -> torch.Tensor:
    """Standard-normal activations drawn directly on `device` (for inputs too
    large to build on the host); the same seed gives the same tensor."""
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(M, K, generator=g, dtype=torch.float32, device=device).to(_DT[dtype])


@dataclass
class W4A8Case:
    x: torch.Tensor        # [M, K] fp16 / bf16 activations (quantised per token by the method)
    b: torch.Tensor        # [K/8, N] int32, K-packed two's-complement int4
    s2: torch.Tensor       # [N] per-output-channel scale, in the activation type
    s3: torch.Tensor | None  # [K/G, N] integer group scales 1..16 (activation type), None = per-channel
    M: int
    K: int
    N: int
    G: int
    seed: int
    dtype: str = "f16"


def w4a8_case(M: int, K: int, N: int, G: int = -1, seed: int | None = None,
              x_rows: int | None = None, dtype: str = "f16") -> W4A8Case:
    if seed is None:
        seed = seed_for(case_key("w4a8", M, K, N, G) if dtype == "f16" else case_key("w4a8", M, K, N, G, dtype))
    dt = _DT[dtype]
    g = torch.Generator().manual_seed(seed)
    b = _words(g, (K // 8, N))
    s = (0.002 + 0.018 * torch.rand(N, generator=g, dtype=torch.float32)).to(dt)
    if G > 0:
        s3 = torch.randint(1, 17, (K // G, N), generator=g, dtype=torch.int64).to(dt)
        s2 = s / 16  # a power-of-two division: exact in fp16 and bf16 for this range
    else:
        s3 = None
        s2 = s
    x = torch.randn(M if x_rows is None else x_rows, K, generator=g, dtype=torch.float32).to(dt)
    return W4A8Case(x, b, s2, s3, M, K, N, G, seed, dtype)
