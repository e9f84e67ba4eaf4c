"""ctypes loader for libawq4.so (the C ABI in include/awq4.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libawq4.so")

AWQ_OK = 0
AWQ_EINVAL = -1
AWQ_EUNSUPPORTED = -2
AWQ_EWORKSPACE = -3
AWQ_EALIGN = -4
AWQ_EHIP = -5

AWQ_DTYPE_F16 = 0
AWQ_DTYPE_BF16 = 1
AWQ_LAYOUT_N8 = 0
W4A8_LAYOUT_K8 = 1
AWQ_LAYOUT_V2 = 2
AWQ_OP_GEMM_W4A16 = 0
AWQ_OP_GEMV_W4A16 = 1
AWQ_OP_W4A8_GEMM = 2
AWQ_OP_W4A8_FP8_GEMM = 3
AWQ_STATIC_SCRATCH_BYTES = 16 << 20

_lib = None


class PlanInfo(ctypes.Structure):
    """awq_plan_t: how the library would launch a call (awq_plan_info)."""
    _fields_ = [("kernel", ctypes.c_int), ("tiles_n", ctypes.c_int), ("tiles_m", ctypes.c_int),
                ("splits", ctypes.c_int), ("row_tiles", ctypes.c_int), ("ksplit", ctypes.c_int),
                ("cu_count", ctypes.c_int), ("workspace_bytes", ctypes.c_int64), ("tile_cols", ctypes.c_int)]


class AWQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {lib().awq_status_str(status).decode()}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_weight_only_awq_amd.build` "
                          "(hipcc, gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.awq_status_str.argtypes = [i32]
    L.awq_status_str.restype = ctypes.c_char_p
    L.awq_version.argtypes = []
    L.awq_version.restype = i32
    L.awq_pack.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.awq_unpack.argtypes = [vp, vp, i64, i64, i32, vp]
    L.awq_workspace_bytes.argtypes = [i32, i64, i64, i64, i32, i32]
    L.awq_workspace_bytes.restype = sz
    w4a16 = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp, sz, vp]
    L.awq_gemm_w4a16.argtypes = w4a16
    L.awq_gemv_w4a16.argtypes = w4a16
    L.awq_gemv_w4a16_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    L.awq_dequant_w4a16.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, vp]
    L.awq_repack_v2.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4a8_fp8_quant_act.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    L.w4a8_fp8_gemm.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    L.w4a8_fp8_linear.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
    L.w4a8_quant_act.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    L.w4a8_gemm.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    L.w4a8_linear.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp]
    L.awq_stream_read.argtypes = [vp, i64, vp, vp]
    L.awq_plan_info.argtypes = [i32, i64, i64, i64, i32, i32, i32, ctypes.POINTER(PlanInfo)]
    for f in ("awq_pack", "awq_unpack", "awq_gemm_w4a16", "awq_gemv_w4a16", "w4a8_quant_act", "w4a8_gemm", "w4a8_linear",
              "awq_stream_read", "awq_plan_info", "awq_gemv_w4a16_static",
              "awq_dequant_w4a16", "w4a8_fp8_quant_act", "w4a8_fp8_gemm", "w4a8_fp8_linear", "awq_repack_v2"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != AWQ_OK:
        raise AWQError(fn, status)
