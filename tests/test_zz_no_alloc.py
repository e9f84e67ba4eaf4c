"""The no-allocation decode entry point (awq_gemv_w4a16_static) through the C
ABI: the same results as awq_gemv_w4a16 with a caller workspace, bit for bit,
on consecutive calls of shrinking size (the static scratch keeps the previous
call's contents only as the zeros the kernels leave behind), in fp16 and bf16;
sizes beyond the scratch are refused before anything is enqueued."""
import ctypes

import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from bit_weight_only_awq_amd import _lib as L
from gpu_helpers import THREADS, check_fp, dev, orc, to_dev

pytestmark = pytest.mark.gpu


def _static(x, qw, s, qz, G, out=None):
    M, K = x.shape
    N = qw.shape[1] * 8
    y = torch.empty(M, N, dtype=x.dtype, device=x.device) if out is None else out
    dt = L.AWQ_DTYPE_F16 if x.dtype == torch.float16 else L.AWQ_DTYPE_BF16
    rc = L.lib().awq_gemv_w4a16_static(x.data_ptr(), qw.data_ptr(), s.data_ptr(),
                                       None if qz is None else qz.data_ptr(), y.data_ptr(), M, N, K, G, dt,
                                       torch.cuda.current_stream(x.device).cuda_stream)
    L.check("awq_gemv_w4a16_static", rc)
    return y


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_static_matches_workspace_entry(dtype):
    """Two calls in a row, the second smaller, each against awq_gemv_w4a16
    (bit for bit) and the oracle."""
    seq = [(8, 11008, 4096, 128, False), (1, 4096, 4096, 128, False), (4, 4096, 1032, 64, True),
           (2, 4096, 12288, 32, False)]
    for M, K, N, G, sym in seq:
        c = synthgen.w4a16_case(M, K, N, G, dtype=dtype, sym=sym)
        x, qw, s, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
        y_static = _static(x, qw, s, qz, G)
        y_ws = awq.gemv_w4a16(x, qw, s, qz, G)
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), y_ws.view(torch.int16)), (M, K, N, G, dtype)
        y64 = orc().w4a16(c.x, c.qweight, c.scales, c.qzeros, G, 0 if dtype == "f16" else 1, nthreads=THREADS)
        check_fp(y_static.cpu(), y64, dtype, f"static gemv M={M} K={K} N={N} G={G} {dtype}")


def test_static_repeated_and_graph_replay():
    """Back-to-back calls leave the scratch clear; a captured call replays
    correctly with eager calls between the replays."""
    c = synthgen.w4a16_case(1, 4096, 4096, 128, seed=21)
    x, qw, s, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
    ref = _static(x, qw, s, qz, 128)
    torch.cuda.synchronize()
    c2 = synthgen.w4a16_case(3, 4096, 2048, 128, seed=22)
    x2, qw2, s2, qz2 = to_dev(c2.x, c2.qweight, c2.scales, c2.qzeros)
    ref2 = awq.gemv_w4a16(x2, qw2, s2, qz2, 128)
    y = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        _static(x, qw, s, qz, 128, out=y)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
        y2 = _static(x2, qw2, s2, qz2, 128)
        torch.cuda.synchronize()
        assert torch.equal(y2, ref2)


def test_static_refuses_what_does_not_fit():
    """A call whose split-K reduction needs more than the static scratch, or
    more than 8 rows, is refused before anything is enqueued."""
    M, K, N = 8, 16384, 32768
    info = awq.plan_info(awq.AWQ_OP_GEMV_W4A16, M, N, K, 128)
    assert info["workspace_bytes"] > L.AWQ_STATIC_SCRATCH_BYTES
    x = torch.zeros(M, K, dtype=torch.bfloat16, device=dev())
    qw = torch.zeros(K, N // 8, dtype=torch.int32, device=dev())
    s = torch.zeros(K // 128, N, dtype=torch.bfloat16, device=dev())
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev())
    rc = L.lib().awq_gemv_w4a16_static(x.data_ptr(), qw.data_ptr(), s.data_ptr(), None, y.data_ptr(), M, N, K, 128,
                                       L.AWQ_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == L.AWQ_EWORKSPACE
    rc = L.lib().awq_gemv_w4a16_static(x.data_ptr(), qw.data_ptr(), s.data_ptr(), None, y.data_ptr(), 9, 4096,
                                       4096, 128, L.AWQ_DTYPE_BF16, None)
    assert rc == L.AWQ_EUNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # nothing was written
