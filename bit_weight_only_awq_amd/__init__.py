"""MI355X (gfx950) 4-bit-weight GEMM library: AWQ W4A16 GEMV/GEMM and QQQ-style W4A8.

The compute lives in libawq4.so (hand-written HIP, C ABI in include/awq4.h);
this package is its thin torch binding.  Importing the package does not need
a GPU; calling an op needs the built library and a gfx950 device.
"""
from ._lib import (AWQ_OP_GEMM_W4A16, AWQ_OP_GEMV_W4A16, AWQ_OP_W4A8_FP8_GEMM, AWQ_OP_W4A8_GEMM,  # noqa: F401
                   AWQError, lib)
from .ops import (dequant_w4a16, gemm_w4a16, gemv_w4a16, linear_w4a16, linear_w4a8, pack, plan_info, quant_act,  # noqa: F401
                  quant_act_fp8, repack_v2, stream_read, unpack, w4a8_fp8_gemm, linear_w4a8_fp8, w4a8_gemm,
                  workspace_bytes)

__all__ = ["AWQError", "lib", "dequant_w4a16", "gemm_w4a16", "gemv_w4a16", "linear_w4a16", "linear_w4a8", "pack", "plan_info",
           "quant_act", "stream_read", "unpack", "w4a8_gemm", "workspace_bytes", "AWQ_OP_GEMM_W4A16",
           "AWQ_OP_GEMV_W4A16", "AWQ_OP_W4A8_GEMM", "AWQ_OP_W4A8_FP8_GEMM", "quant_act_fp8", "w4a8_fp8_gemm", "linear_w4a8_fp8", "repack_v2"]
