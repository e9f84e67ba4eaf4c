"""Thin torch-facing binding of libawq4.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module
only checks tensor placement/dtypes, allocates outputs and the per-device
workspace through torch, and passes raw pointers and the current stream.
"""
from __future__ import annotations

import ctypes
import threading

import torch

from . import _lib as L

_F16 = {torch.float16: L.AWQ_DTYPE_F16, torch.bfloat16: L.AWQ_DTYPE_BF16}


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on a CUDA (HIP) device")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


# ----------------------------------------------------------------------------- workspace

class Workspace:
    """One zero-initialised workspace per (device, stream), grown on demand and
    shared by every call ordered on that stream (the library leaves its
    counters zero after each call).  Calls on different streams may overlap in
    time, so each stream gets its own buffer; a grown buffer is zero-filled on
    the stream that will use it, and the caching allocator keeps the old one
    alive until the work queued on that stream before the swap has run."""

    def __init__(self):
        self._bufs: dict[tuple[int, int], torch.Tensor] = {}
        self._lock = threading.Lock()

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        idx = device.index if device.index is not None else torch.cuda.current_device()
        stream = torch.cuda.current_stream(idx)
        key = (idx, stream.cuda_stream)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                size = max(nbytes, 2 * (buf.numel() if buf is not None else 0), 1 << 20)
                with torch.cuda.stream(stream):
                    buf = torch.zeros(size, dtype=torch.uint8, device=torch.device("cuda", idx))
                self._bufs[key] = buf
            return buf


WORKSPACE = Workspace()


def workspace_bytes(op: int, M: int, N: int, K: int, group_size: int, split_k: int = 0,
                    device: torch.device | None = None) -> int:
    """Workspace bytes of a call on `device` (the current device if None)."""
    if device is None:
        return int(L.lib().awq_workspace_bytes(op, M, N, K, group_size, split_k))
    with torch.cuda.device(device):
        return int(L.lib().awq_workspace_bytes(op, M, N, K, group_size, split_k))


def plan_info(op: int, M: int, N: int, K: int, group_size: int, split_k: int = 0, cu_count: int = 0) -> dict:
    """How the library would launch a call (awq_plan_info); cu_count 0 = the current device."""
    info = L.PlanInfo()
    L.check("awq_plan_info", L.lib().awq_plan_info(op, M, N, K, group_size, split_k, cu_count,
                                                   ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in L.PlanInfo._fields_}


# ----------------------------------------------------------------------------- packing

def pack(vals: torch.Tensor, layout: str = "n8", clamp_count: torch.Tensor | None = None) -> torch.Tensor:
    """Pack 4-bit values: layout "n8" (AWQ, uint8 [rows, cols] -> int32 [rows, cols/8]),
    "v2" (the newer AWQ packing, identity order, int32 [rows, ceil(cols/8)])
    or "k8" (W4A8, int8 [K, N] -> int32 [K/8, N])."""
    _need_cuda(vals, clamp_count)
    rows, cols = vals.shape
    if layout == "v2":
        out = torch.empty(rows, (cols + 7) // 8, dtype=torch.int32, device=vals.device)
        lay = L.AWQ_LAYOUT_V2
    elif layout == "n8":
        out = torch.empty(rows, cols // 8, dtype=torch.int32, device=vals.device)
        lay = L.AWQ_LAYOUT_N8
    else:
        out = torch.empty(rows // 8, cols, dtype=torch.int32, device=vals.device)
        lay = L.W4A8_LAYOUT_K8
    L.check("awq_pack", L.lib().awq_pack(_ptr(vals), _ptr(out), rows, cols, lay, _ptr(clamp_count),
                                         _stream(vals.device)))
    return out


def unpack(packed: torch.Tensor, layout: str = "n8", cols: int | None = None) -> torch.Tensor:
    """Inverse of pack; layout "v2" takes the number of values per row (default: all 8 per word)."""
    _need_cuda(packed)
    if layout == "v2":
        rows = packed.shape[0]
        cols = packed.shape[1] * 8 if cols is None else cols
        out = torch.empty(rows, cols, dtype=torch.uint8, device=packed.device)
        lay = L.AWQ_LAYOUT_V2
    elif layout == "n8":
        rows, cols = packed.shape[0], packed.shape[1] * 8
        out = torch.empty(rows, cols, dtype=torch.uint8, device=packed.device)
        lay = L.AWQ_LAYOUT_N8
    else:
        rows, cols = packed.shape[0] * 8, packed.shape[1]
        out = torch.empty(rows, cols, dtype=torch.int8, device=packed.device)
        lay = L.W4A8_LAYOUT_K8
    L.check("awq_unpack", L.lib().awq_unpack(_ptr(packed), _ptr(out), rows, cols, lay, _stream(packed.device)))
    return out


def repack_v2(qweight_v2: torch.Tensor, qzeros_v2: torch.Tensor | None, group_size: int = 128):
    """Weights in the newer AWQ packing -> (qweight, qzeros) in the format the
    GEMM / GEMV calls take (awq_repack_v2); scales are shared by both formats."""
    _need_cuda(qweight_v2, qzeros_v2)
    K, N = qweight_v2.shape[0], qweight_v2.shape[1] * 8
    qweight = torch.empty_like(qweight_v2)
    qzeros = None if qzeros_v2 is None else torch.empty(K // group_size, N // 8, dtype=torch.int32,
                                                        device=qweight_v2.device)
    L.check("awq_repack_v2", L.lib().awq_repack_v2(_ptr(qweight_v2), _ptr(qzeros_v2), _ptr(qweight), _ptr(qzeros),
                                                   N, K, group_size, _stream(qweight_v2.device)))
    return qweight, qzeros


# ----------------------------------------------------------------------------- W4A16

def _w4a16(fn_name: str, op: int, x, qweight, scales, qzeros, group_size, split_k, out):
    _need_cuda(x, qweight, scales, qzeros, out)
    if x.dtype not in _F16:
        raise ValueError("x must be fp16 or bf16")
    if scales.dtype != x.dtype:
        raise ValueError("scales must have the activation dtype")
    M, K = x.shape
    N = qweight.shape[1] * 8
    if out is None:
        out = torch.empty(M, N, dtype=x.dtype, device=x.device)
    need = workspace_bytes(op, M, N, K, group_size, split_k, x.device)
    ws = WORKSPACE.get(x.device, need)
    fn = getattr(L.lib(), fn_name)
    L.check(fn_name, fn(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(out), M, N, K, group_size,
                        _F16[x.dtype], split_k, _ptr(ws), 0 if ws is None else ws.numel(), _stream(x.device)))
    return out


def gemm_w4a16(x, qweight, scales, qzeros, group_size: int = 128, split_k: int = 0, out=None):
    """Y = X . dequant(qweight, qzeros, scales) (prefill path, any M)."""
    return _w4a16("awq_gemm_w4a16", L.AWQ_OP_GEMM_W4A16, x, qweight, scales, qzeros, group_size, split_k, out)


def gemv_w4a16(x, qweight, scales, qzeros, group_size: int = 128, split_k: int = 0, out=None):
    """Decode path, M <= 8."""
    return _w4a16("awq_gemv_w4a16", L.AWQ_OP_GEMV_W4A16, x, qweight, scales, qzeros, group_size, split_k, out)


def linear_w4a16(x, qweight, scales, qzeros, group_size: int = 128, out=None):
    """The AWQ linear-layer dispatch: more than 8 rows -> GEMM, else GEMV."""
    if x.shape[0] > 8:
        return gemm_w4a16(x, qweight, scales, qzeros, group_size, out=out)
    return gemv_w4a16(x, qweight, scales, qzeros, group_size, out=out)


def dequant_w4a16(qweight, scales, qzeros, group_size: int = 128, out=None):
    """Dense W = (q - z) * s, [K, N] in the scales' dtype (one rounding per
    element): the weight operand of a dense vendor GEMM, for comparison."""
    _need_cuda(qweight, scales, qzeros, out)
    if scales.dtype not in _F16:
        raise ValueError("scales must be fp16 or bf16")
    K, N = qweight.shape[0], qweight.shape[1] * 8
    if out is None:
        out = torch.empty(K, N, dtype=scales.dtype, device=qweight.device)
    L.check("awq_dequant_w4a16", L.lib().awq_dequant_w4a16(_ptr(qweight), _ptr(scales), _ptr(qzeros), _ptr(out), N,
                                                           K, group_size, _F16[scales.dtype],
                                                           _stream(qweight.device)))
    return out


# ----------------------------------------------------------------------------- W4A8

def quant_act(x: torch.Tensor, a8: torch.Tensor | None = None, s1: torch.Tensor | None = None):
    """Per-token int8 quantisation of fp16 or bf16 activations -> (a8 int8 [M,K], s1 fp32 [M])."""
    _need_cuda(x, a8, s1)
    if x.dtype not in _F16:
        raise ValueError("W4A8 activations must be fp16 or bf16")
    M, K = x.shape
    if a8 is None:
        a8 = torch.empty(M, K, dtype=torch.int8, device=x.device)
    if s1 is None:
        s1 = torch.empty(M, dtype=torch.float32, device=x.device)
    L.check("w4a8_quant_act", L.lib().w4a8_quant_act(_ptr(x), _ptr(a8), _ptr(s1), M, K, _F16[x.dtype],
                                                     _stream(x.device)))
    return a8, s1


def w4a8_gemm(a8, b, s1, s2, s3=None, group_size: int = -1, want_acc: bool = False, out=None):
    """y = act(acc * s1 * s2), acc = a8 . w8 (exact int32), in the dtype of s2
    (fp16 or bf16; s3 and y share it). Returns y or (y, acc)."""
    _need_cuda(a8, b, s1, s2, s3, out)
    if s2.dtype not in _F16 or (s3 is not None and s3.dtype != s2.dtype):
        raise ValueError("W4A8 scales must be fp16 or bf16, s2 and s3 alike")
    M, K = a8.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty(M, N, dtype=s2.dtype, device=a8.device)
    acc = torch.empty(M, N, dtype=torch.int32, device=a8.device) if want_acc else None
    need = workspace_bytes(L.AWQ_OP_W4A8_GEMM, M, N, K, group_size, 0, a8.device)
    ws = WORKSPACE.get(a8.device, need)
    L.check("w4a8_gemm", L.lib().w4a8_gemm(_ptr(a8), _ptr(b), _ptr(s1), _ptr(s2), _ptr(s3), _ptr(out), _ptr(acc),
                                           M, N, K, group_size, _F16[s2.dtype], _ptr(ws),
                                           0 if ws is None else ws.numel(), _stream(a8.device)))
    return (out, acc) if want_acc else out


def linear_w4a8(x, b, s2, s3=None, group_size: int = -1, want_acc: bool = False, out=None, a8=None, s1=None):
    """The whole W4A8 layer in one call (w4a8_linear): per-token quantisation of
    x, then the W4A8 GEMM, fused into one kernel for small batches.  Returns y,
    or (y, s1, acc) with want_acc.  `a8` is scratch for the two-step path."""
    _need_cuda(x, b, s2, s3, out, a8, s1)
    if x.dtype not in _F16 or s2.dtype != x.dtype or (s3 is not None and s3.dtype != x.dtype):
        raise ValueError("W4A8 activations and scales must be fp16 or bf16, all of one type")
    M, K = x.shape
    N = b.shape[1]
    if a8 is None:
        a8 = torch.empty(M, K, dtype=torch.int8, device=x.device)
    if s1 is None:
        s1 = torch.empty(M, dtype=torch.float32, device=x.device)
    if out is None:
        out = torch.empty(M, N, dtype=x.dtype, device=x.device)
    acc = torch.empty(M, N, dtype=torch.int32, device=x.device) if want_acc else None
    need = workspace_bytes(L.AWQ_OP_W4A8_GEMM, M, N, K, group_size, 0, x.device)
    ws = WORKSPACE.get(x.device, need)
    L.check("w4a8_linear", L.lib().w4a8_linear(_ptr(x), _ptr(a8), _ptr(s1), _ptr(b), _ptr(s2), _ptr(s3), _ptr(out),
                                               _ptr(acc), M, N, K, group_size, _F16[x.dtype], _ptr(ws),
                                               0 if ws is None else ws.numel(), _stream(x.device)))
    return (out, s1, acc) if want_acc else out


# ----------------------------------------------------------------------------- INT4-FP8 W4A8

def quant_act_fp8(x: torch.Tensor, a=None, s1=None, asum=None):
    """Per-token E4M3 quantisation -> (codes uint8 [M,K], s1 fp32 [M], asum fp32 [M])."""
    _need_cuda(x, a, s1, asum)
    if x.dtype not in _F16:
        raise ValueError("activations must be fp16 or bf16")
    M, K = x.shape
    a = torch.empty(M, K, dtype=torch.uint8, device=x.device) if a is None else a
    s1 = torch.empty(M, dtype=torch.float32, device=x.device) if s1 is None else s1
    asum = torch.empty(M, dtype=torch.float32, device=x.device) if asum is None else asum
    L.check("w4a8_fp8_quant_act", L.lib().w4a8_fp8_quant_act(_ptr(x), _ptr(a), _ptr(s1), _ptr(asum), M, K,
                                                             _F16[x.dtype], _stream(x.device)))
    return a, s1, asum


def w4a8_fp8_gemm(a, b, s1, asum, s2, want_acc: bool = False, out=None):
    """y = act(acc * s1 * s2), acc = sum_k e4m3(a) q (fp32 on the fp8 matrix
    cores), in the dtype of s2.  Returns y or (y, acc)."""
    _need_cuda(a, b, s1, asum, s2, out)
    if s2.dtype not in _F16:
        raise ValueError("s2 must be fp16 or bf16")
    M, K = a.shape
    N = b.shape[1]
    if out is None:
        out = torch.empty(M, N, dtype=s2.dtype, device=a.device)
    acc = torch.empty(M, N, dtype=torch.float32, device=a.device) if want_acc else None
    need = workspace_bytes(L.AWQ_OP_W4A8_FP8_GEMM, M, N, K, -1, 0, a.device)
    ws = WORKSPACE.get(a.device, need)
    L.check("w4a8_fp8_gemm", L.lib().w4a8_fp8_gemm(_ptr(a), _ptr(b), _ptr(s1), _ptr(asum), _ptr(s2), _ptr(out),
                                                   _ptr(acc), M, N, K, _F16[s2.dtype], _ptr(ws),
                                                   0 if ws is None else ws.numel(), _stream(a.device)))
    return (out, acc) if want_acc else out


def linear_w4a8_fp8(x, b, s2, want_acc: bool = False, out=None, a=None, s1=None, asum=None):
    """The whole INT4-FP8 layer in one call (w4a8_fp8_linear): per-token E4M3
    quantisation of x, then the GEMM, one kernel for a single token.  Returns
    y, or (y, s1, acc) with want_acc.  `a` and `asum` are scratch for the
    two-step path."""
    _need_cuda(x, b, s2, out, a, s1, asum)
    if x.dtype not in _F16 or s2.dtype != x.dtype:
        raise ValueError("activations and s2 must be fp16 or bf16, of one type")
    M, K = x.shape
    N = b.shape[1]
    a = torch.empty(M, K, dtype=torch.uint8, device=x.device) if a is None else a
    s1 = torch.empty(M, dtype=torch.float32, device=x.device) if s1 is None else s1
    asum = torch.empty(M, dtype=torch.float32, device=x.device) if asum is None else asum
    if out is None:
        out = torch.empty(M, N, dtype=x.dtype, device=x.device)
    acc = torch.empty(M, N, dtype=torch.float32, device=x.device) if want_acc else None
    need = workspace_bytes(L.AWQ_OP_W4A8_FP8_GEMM, M, N, K, -1, 0, x.device)
    ws = WORKSPACE.get(x.device, need)
    L.check("w4a8_fp8_linear", L.lib().w4a8_fp8_linear(_ptr(x), _ptr(a), _ptr(s1), _ptr(asum), _ptr(b), _ptr(s2),
                                                       _ptr(out), _ptr(acc), M, N, K, _F16[x.dtype], _ptr(ws),
                                                       0 if ws is None else ws.numel(), _stream(x.device)))
    return (out, s1, acc) if want_acc else out


# ----------------------------------------------------------------------------- measurement helper

STREAM_SINK_WORDS = 8192


def stream_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Read every byte of `src` once on the GPU (bandwidth probe; not part of the
    method).  Returns the int32 sink of per-wave checksums."""
    _need_cuda(src, sink)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(STREAM_SINK_WORDS, dtype=torch.int32, device=src.device)
    if not src.is_contiguous() or sink.numel() < STREAM_SINK_WORDS or sink.dtype != torch.int32:
        raise ValueError("stream_read needs a contiguous source and an int32 sink of STREAM_SINK_WORDS words")
    L.check("awq_stream_read", L.lib().awq_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(src.device)))
    return sink
