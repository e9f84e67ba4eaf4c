"""CPU oracle for the AWQ W4A16 / QQQ W4A8 hot path (test infrastructure only).

This package is the plain reference that the GPU library is checked against.
Only the tests, the smoke check and the benchmark's ``cpu_baseline`` leg may
import it; the GPU library neither imports it nor shares any code with it.

The arithmetic lives in ``oracle.c`` (scalar C: integer bit work, int64 dot
products, IEEE double for floating point).  This module only compiles it with
gcc, loads it with ctypes and marshals numpy arrays.  Every function cites the
passage of the pages it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liborc.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-fno-fast-math", "-ffp-contract=off"]

F16, BF16 = 0, 1
_build_lock = threading.Lock()


def compile_oracle(src: str = SRC, out: str = LIB, defines=()) -> str:
    """Compile ``src`` with gcc into the shared library ``out``."""
    cmd = ["gcc", *GCC_FLAGS, *[f"-D{d}" for d in defines], src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


def build(force: bool = False) -> str:
    """Build liborc.so next to this file if it is missing or older than oracle.c."""
    with _build_lock:
        if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            compile_oracle()
    return LIB


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _u16(a) -> np.ndarray:
    """Accept a numpy uint16/float16 array or a torch fp16/bf16 CPU tensor; return raw bits."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        t = a.detach().cpu().contiguous()
        if t.dtype in (torch.float16, torch.bfloat16):
            t = t.view(torch.int16)
        a = t.numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a.view(np.uint16))


def _i32(a) -> np.ndarray:
    """Accept int32/uint32 numpy arrays or torch int32 tensors; return int32 words."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().numpy()
    a = np.asarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype != np.int32:
        a = a.astype(np.int32)
    return np.ascontiguousarray(a)


class Oracle:
    """ctypes binding of one compiled oracle library (the real one or a test mutant)."""

    def __init__(self, path: str | None = None):
        self.path = path or build()
        self.lib = ctypes.CDLL(self.path)
        L = self.lib
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_unpack_n8.argtypes = [vp, vp, i64, i64]
        L.orc_pack_n8.argtypes = [vp, vp, i64, i64, vp]
        L.orc_unpack_k8.argtypes = [vp, vp, i64, i64]
        L.orc_pack_k8.argtypes = [vp, vp, i64, i64, vp]
        L.orc_w4a16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, i32]
        L.orc_dequant.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp]
        L.orc_quant_act.argtypes = [vp, i64, i64, i32, vp, vp]
        L.orc_w4a8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, i32]
        L.orc_unpack_v2.argtypes = [vp, vp, i64, i64]
        L.orc_pack_v2.argtypes = [vp, vp, i64, i64, vp]
        L.orc_w4a16_v2.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = ctypes.c_double
        L.orc_f64_to_e4m3.argtypes = [ctypes.c_double]
        L.orc_f64_to_e4m3.restype = ctypes.c_uint8
        L.orc_quant_act_fp8.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.orc_w4a8_fp8.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        for f in ("orc_unpack_n8", "orc_pack_n8", "orc_unpack_k8", "orc_pack_k8", "orc_w4a16",
                  "orc_dequant", "orc_quant_act", "orc_w4a8", "orc_quant_act_fp8", "orc_w4a8_fp8",
                  "orc_unpack_v2", "orc_pack_v2", "orc_w4a16_v2"):
            getattr(L, f).restype = ctypes.c_int

    # -- scalar formats ------------------------------------------------------
    def f16_to_f64(self, bits: int) -> float:
        return self.lib.orc_f16_to_f64(int(bits) & 0xFFFF)

    def bf16_to_f64(self, bits: int) -> float:
        return self.lib.orc_bf16_to_f64(int(bits) & 0xFFFF)

    def f64_to_f16(self, v: float) -> int:
        return int(self.lib.orc_f64_to_f16(float(v)))

    def f64_to_bf16(self, v: float) -> int:
        return int(self.lib.orc_f64_to_bf16(float(v)))

    # -- packing ---------------------------------------------------------------
    def unpack_n8(self, packed) -> np.ndarray:
        p = _i32(packed)
        rows, wc = p.shape
        out = np.empty((rows, wc * 8), np.uint8)
        assert self.lib.orc_unpack_n8(_p(p), _p(out), rows, wc * 8) == 0
        return out

    def pack_n8(self, vals):
        v = np.ascontiguousarray(vals, dtype=np.uint8)
        rows, cols = v.shape
        out = np.empty((rows, cols // 8), np.int32)
        n_bad = ctypes.c_int64(0)
        rc = self.lib.orc_pack_n8(_p(v), _p(out), rows, cols, ctypes.byref(n_bad))
        if rc:
            raise ValueError("pack_n8: cols must be a multiple of 8")
        return out, int(n_bad.value)

    def unpack_k8(self, packed) -> np.ndarray:
        p = _i32(packed)
        kb, n = p.shape
        out = np.empty((kb * 8, n), np.int8)
        assert self.lib.orc_unpack_k8(_p(p), _p(out), kb * 8, n) == 0
        return out

    def pack_k8(self, vals):
        v = np.ascontiguousarray(vals, dtype=np.int8)
        k, n = v.shape
        out = np.empty((k // 8, n), np.int32)
        n_bad = ctypes.c_int64(0)
        rc = self.lib.orc_pack_k8(_p(v), _p(out), k, n, ctypes.byref(n_bad))
        if rc:
            raise ValueError("pack_k8: K must be a multiple of 8")
        return out, int(n_bad.value)

    # -- W4A16 -----------------------------------------------------------------
    def dequant(self, qweight, scales, qzeros, group_size: int, dtype: int = F16) -> np.ndarray:
        qw = _i32(qweight)
        K, wc = qw.shape
        N = wc * 8
        s = _u16(scales)
        qz = _i32(qzeros) if qzeros is not None else None
        out = np.empty((K, N), np.float64)
        rc = self.lib.orc_dequant(_p(qw), _p(s), _p(qz), N, K, group_size, dtype, _p(out))
        if rc:
            raise ValueError("dequant: bad shape")
        return out

    def w4a16(self, x, qweight, scales, qzeros, group_size: int, dtype: int = F16,
              nthreads: int = 1) -> np.ndarray:
        xb = _u16(x)
        qw = _i32(qweight)
        K, wc = qw.shape
        N = wc * 8
        M = xb.shape[0]
        assert xb.shape == (M, K), (xb.shape, K)
        s = _u16(scales)
        assert s.shape == (K // group_size, N)
        qz = _i32(qzeros) if qzeros is not None else None
        if qz is not None:
            assert qz.shape == (K // group_size, wc)
        y = np.empty((M, N), np.float64)
        rc = self.lib.orc_w4a16(_p(xb), _p(qw), _p(s), _p(qz), M, N, K, group_size, dtype,
                                _p(y), int(nthreads))
        if rc:
            raise ValueError("w4a16: bad shape")
        return y

    # -- W4A8 ------------------------------------------------------------------
    def quant_act(self, x, dtype: int = F16):
        """Per-token int8 quantisation of fp16 (dtype 0) or bf16 (dtype 1) activations."""
        xb = _u16(x)
        M, K = xb.shape
        a8 = np.empty((M, K), np.int8)
        s1 = np.empty((M,), np.float32)
        assert self.lib.orc_quant_act(_p(xb), M, K, int(dtype), _p(a8), _p(s1)) == 0
        return a8, s1

    def w4a8(self, a8, b_packed, s1, s2, s3=None, group_size: int = -1, nthreads: int = 1,
             want_y: bool = True, dtype: int = F16):
        a = np.ascontiguousarray(a8, dtype=np.int8)
        b = _i32(b_packed)
        M, K = a.shape
        kb, N = b.shape
        assert kb * 8 == K
        s1a = np.ascontiguousarray(s1, dtype=np.float32)
        s2a = _u16(s2)
        s3a = _u16(s3) if s3 is not None else None
        acc = np.empty((M, N), np.int64)
        y = np.empty((M, N), np.float64) if want_y else None
        rc = self.lib.orc_w4a8(_p(a), _p(b), _p(s1a), _p(s2a), _p(s3a), M, N, K,
                               int(group_size), int(dtype), _p(acc), _p(y), int(nthreads))
        if rc:
            raise ValueError("w4a8: bad shape or non-integer group scale")
        return acc, y


    # -- second AWQ packing -------------------------------------------------------
    def unpack_v2(self, packed, cols: int) -> np.ndarray:
        """Identity-order words [rows, ceil(cols/8)] -> values [rows, cols]."""
        p = _i32(packed)
        rows = p.shape[0]
        assert p.shape[1] == (cols + 7) // 8
        out = np.empty((rows, cols), np.uint8)
        assert self.lib.orc_unpack_v2(_p(p), _p(out), rows, cols) == 0
        return out

    def pack_v2(self, vals):
        v = np.ascontiguousarray(vals, dtype=np.uint8)
        rows, cols = v.shape
        out = np.empty((rows, (cols + 7) // 8), np.int32)
        n_bad = ctypes.c_int64(0)
        assert self.lib.orc_pack_v2(_p(v), _p(out), rows, cols, ctypes.byref(n_bad)) == 0
        return out, int(n_bad.value)

    def w4a16_v2(self, x, qweight, scales, qzeros, group_size: int, dtype: int = F16) -> np.ndarray:
        """Y64 from weights in the second AWQ packing (qweight [K, N/8] identity
        order, scales [K/G, N], qzeros [N, ceil(K/G/8)] or None)."""
        xb = _u16(x)
        qw = _i32(qweight)
        K, wc = qw.shape
        N = wc * 8
        M = xb.shape[0]
        s = _u16(scales)
        assert s.shape == (K // group_size, N)
        qz = _i32(qzeros) if qzeros is not None else None
        if qz is not None:
            assert qz.shape == (N, (K // group_size + 7) // 8)
        y = np.empty((M, N), np.float64)
        rc = self.lib.orc_w4a16_v2(_p(xb), _p(qw), _p(s), _p(qz), M, N, K, group_size, dtype, _p(y))
        if rc:
            raise ValueError("w4a16_v2: bad shape")
        return y

    # -- INT4-FP8 W4A8 -----------------------------------------------------------
    def e4m3_to_f64(self, code: int) -> float:
        return self.lib.orc_e4m3_to_f64(int(code) & 0xFF)

    def f64_to_e4m3(self, v: float) -> int:
        return int(self.lib.orc_f64_to_e4m3(float(v)))

    def quant_act_fp8(self, x, dtype: int = F16):
        """Per-token E4M3 quantisation -> (codes uint8 [M,K], s1 fp32 [M], asum fp32 [M])."""
        xb = _u16(x)
        M, K = xb.shape
        a = np.empty((M, K), np.uint8)
        s1 = np.empty((M,), np.float32)
        asum = np.empty((M,), np.float32)
        assert self.lib.orc_quant_act_fp8(_p(xb), M, K, int(dtype), _p(a), _p(s1), _p(asum)) == 0
        return a, s1, asum

    def w4a8_fp8(self, a, b_packed, s1, s2, dtype: int = F16, want_y: bool = True):
        """(acc fp64 [M,N] exact, Y64 fp64 [M,N]) of the INT4-FP8 W4A8 GEMM."""
        ac = np.ascontiguousarray(a, dtype=np.uint8)
        b = _i32(b_packed)
        M, K = ac.shape
        kb, N = b.shape
        assert kb * 8 == K
        s1a = np.ascontiguousarray(s1, dtype=np.float32)
        s2a = _u16(s2)
        acc = np.empty((M, N), np.float64)
        y = np.empty((M, N), np.float64) if want_y else None
        rc = self.lib.orc_w4a8_fp8(_p(ac), _p(b), _p(s1a), _p(s2a), M, N, K, int(dtype), _p(acc), _p(y))
        if rc:
            raise ValueError("w4a8_fp8: bad shape")
        return acc, y


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
