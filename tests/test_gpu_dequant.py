"""GPU dense dequantisation (awq_dequant_w4a16) vs the oracle's fp64 W rounded
once to the activation type: bit-exact.  (q - z) * s is exact in fp64, so the
rounding is a plain type conversion, done here by numpy (fp16) and torch (bf16,
from an fp32 value that holds the product exactly)."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import orc, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N,G,dtype,sym", [(4096, 4096, 128, "f16", False), (4096, 14336, 64, "bf16", True),
                                             (256, 1032, 32, "f16", True), (384, 2056, 128, "bf16", False),
                                             (14336, 4096, 128, "f16", False), (64, 8, 32, "f16", False)])
def test_dequant_bit_exact(K, N, G, dtype, sym):
    c = synthgen.w4a16_case(1, K, N, G, dtype=dtype, sym=sym)
    qw, s, qz = to_dev(c.qweight, c.scales, c.qzeros)
    w = awq.dequant_w4a16(qw, s, qz, G)
    torch.cuda.synchronize()
    w64 = orc().dequant(c.qweight, c.scales, c.qzeros, G, 0 if dtype == "f16" else 1)
    if dtype == "f16":
        exp = torch.from_numpy(w64.astype(np.float16))
    else:
        w32 = w64.astype(np.float32)
        assert np.array_equal(w32.astype(np.float64), w64)  # the product fits fp32 exactly
        exp = torch.from_numpy(w32).to(torch.bfloat16)
    got = w.cpu()
    assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), int((got != exp).sum())


def test_dequant_matches_gemm_operand():
    """A dense GEMM on the dequantised W gives the W4A16 GEMM's result within
    the fp16 bar (both use the same once-rounded weights)."""
    c = synthgen.w4a16_case(64, 1024, 512, 128, seed=5)
    x, qw, s, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
    w = awq.dequant_w4a16(qw, s, qz, 128)
    y_dense = (x.float() @ w.float()).half()
    y = awq.gemm_w4a16(x, qw, s, qz, 128)
    torch.cuda.synchronize()
    err = (y.float() - y_dense.float()).abs().max().item()
    assert err <= 0.03, err
