"""The workspace rule of awq_workspace_bytes: after every call the workspace is
zero again, whichever way the call reduced its K splits -- counting
accumulators (fp16 decode, skinny W4A8), partial tiles summed by the tile's
last workgroup, or partial tiles summed by a second kernel.  Each call runs on
the binding's shared workspace after the previous one (a different kind of
call each time), the whole buffer is checked for zero bytes after it, and the
call repeated must give the same bits."""
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from bit_weight_only_awq_amd import ops
from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu

# (op, M, K, N, G, dtype): each plan splits K
W16 = [
    (1, 4096, 4096, 128, "f16"),    # decode GEMV: counting accumulators
    (1, 4096, 4096, 128, "bf16"),   # decode GEMV: partial tiles, last workgroup
    (32, 4096, 4096, 128, "f16"),   # streaming kernel: partial quads, last workgroup
    (64, 4096, 1032, 32, "f16"),    # streaming kernel: a second kernel
    (100, 4096, 6144, 128, "f16"),  # LDS GEMM: a second kernel
    (96, 14336, 4096, 128, "bf16"),  # LDS GEMM, eight splits: a second kernel
]
W8 = [
    (16, 21760, 8192, -1),   # skinny: counting accumulators
    (48, 4096, 4096, 128),   # LDS GEMM from 33 rows: a second kernel
    (256, 4096, 4096, -1),   # LDS GEMM: a second kernel
]


def _buffer():
    d = dev()
    return ops.WORKSPACE._bufs[(d.index or 0, torch.cuda.current_stream(d).cuda_stream)]


def _assert_zero():
    torch.cuda.synchronize()
    buf = _buffer()
    assert int(torch.count_nonzero(buf)) == 0


def test_workspace_zero_after_every_split_call():
    torch.cuda.synchronize()
    for M, K, N, G, dt in W16:
        c = synthgen.w4a16_case(M, K, N, G, dtype=dt)
        x, qw, sc, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
        info = awq.plan_info(awq.AWQ_OP_GEMM_W4A16 if M > 8 else awq.AWQ_OP_GEMV_W4A16, M, N, K, G)
        assert info["splits"] > 1, (M, K, N, info)
        fn = awq.gemm_w4a16 if M > 8 else awq.gemv_w4a16
        y = fn(x, qw, sc, qz, G)
        _assert_zero()
        y2 = fn(x, qw, sc, qz, G)
        _assert_zero()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (M, K, N, dt)
    for M, K, N, G in W8:
        c = synthgen.w4a8_case(M, K, N, G)
        x, b, s2, s3 = to_dev(c.x, c.b, c.s2, c.s3)
        a8, s1 = awq.quant_act(x)
        info = awq.plan_info(awq.AWQ_OP_W4A8_GEMM, M, N, K, G)
        assert info["splits"] > 1, (M, K, N, info)
        y = awq.w4a8_gemm(a8, b, s1, s2, s3, G)
        _assert_zero()
        fa, fs1, fas = awq.quant_act_fp8(x)
        if G < 0:
            assert awq.plan_info(awq.AWQ_OP_W4A8_FP8_GEMM, M, N, K, -1)["splits"] > 1
            awq.w4a8_fp8_gemm(fa, b, fs1, fas, s2)
            _assert_zero()
        y2 = awq.w4a8_gemm(a8, b, s1, s2, s3, G)
        _assert_zero()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (M, K, N, G)
