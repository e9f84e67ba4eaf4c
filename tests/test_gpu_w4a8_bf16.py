"""GPU W4A8 with bf16 activations, scales and outputs vs the CPU oracle.

The QQQ page lists bf16 as not yet supported and names what it touches; this
library carries the fp16 recipe over (s1 rounded to bf16, s2 / s3 / y in
bf16).  The int8 activations, s1 and the int32 accumulators are checked bit
for bit; the bf16 output within the bf16 bound (relative Frobenius 1e-2, per
element 0.05 + 2^-8 |y|) of the fp64 result from the same quantised
activations."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import THREADS, check_fp, dev, orc, sample_rows, to_dev

pytestmark = pytest.mark.gpu

BF16 = 1


def _quant_check(x_cpu):
    assert x_cpu.dtype == torch.bfloat16
    a8, s1 = awq.quant_act(x_cpu.to(dev()))
    torch.cuda.synchronize()
    ea8, es1 = orc().quant_act(x_cpu, dtype=BF16)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    assert np.array_equal(a8.cpu().numpy(), ea8)
    return a8, s1, ea8, es1


@pytest.mark.parametrize("M,K", [(1, 21760), (16, 21760), (64, 4096), (3, 7), (5, 1000)])
def test_quant_act_bf16_bit_exact(M, K):
    x = synthgen.activations(M, K, "bf16", seed=M * 7 + K)
    x = x * torch.logspace(-6, 6, M).to(torch.bfloat16)[:, None]  # rows across magnitudes
    _quant_check(x.to(torch.bfloat16))


@pytest.mark.parametrize("K", [8192, 8200, 131072, 131080])
def test_quant_act_bf16_row_lengths(K):
    """Both register-resident widths and the two-pass kernel past them."""
    x = synthgen.activations(3, K, "bf16", seed=K)
    x = x * torch.tensor([1e-3, 1.0, 3e4], dtype=torch.bfloat16)[:, None]
    _quant_check(x)


def test_quant_act_bf16_edge_rows():
    """The worked examples of the bf16 recipe, a zero row, ties, and a row so
    small that s1 is a subnormal fp32 value (bf16 keeps binary32's range)."""
    rows = [[127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -127],
            [1.0, 0.5, -0.25, 0.75, 0, 0, 0, 0],
            [0.0] * 8,
            [2.0 ** -127, -(2.0 ** -127), 0, 0, 0, 0, 0, 0],
            [3.0e38, -3.0e38, 1, 2, 3, 4, 5, 6]]
    x = torch.tensor(rows, dtype=torch.float64).to(torch.bfloat16)
    a8, s1, _, _ = _quant_check(x)
    assert a8.cpu()[0].tolist() == [127, 2, 4, -2, -4, 0, 2, -127]
    assert a8.cpu()[1, :4].tolist() == [127, 64, -32, 95]
    assert float(s1.cpu()[2]) == 0.0
    assert a8.cpu()[3, :2].tolist() == [64, -64]


def _case_check(M, K, N, G):
    c = synthgen.w4a8_case(M, K, N, G, dtype="bf16")
    x, b, s2, s3 = to_dev(c.x, c.b, c.s2, c.s3)
    a8, s1 = awq.quant_act(x)
    y, acc = awq.w4a8_gemm(a8, b, s1, s2, s3, G, want_acc=True)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16
    ea8, es1 = orc().quant_act(c.x, dtype=BF16)
    assert np.array_equal(a8.cpu().numpy(), ea8)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    rows = np.arange(M) if M <= 16 else sample_rows(M, seed=M + 1)
    eacc, y64 = orc().w4a8(ea8[rows], c.b, es1[rows], c.s2, c.s3, G, nthreads=THREADS, dtype=BF16)
    gacc = acc.cpu().numpy()[rows].astype(np.int64)
    assert np.array_equal(gacc, eacc), f"acc mismatch at {np.argwhere(gacc != eacc)[:5]}"
    check_fp(y.cpu()[torch.as_tensor(rows)], y64, "bf16", f"w4a8 bf16 M={M} K={K} N={N} G={G}")


@pytest.mark.parametrize("G", [-1, 128])
@pytest.mark.parametrize("M", [1, 16, 64, 256, 1024])
def test_w4a8_bf16_qqq_shape(M, G):
    """The QQQ GEMM shape N=8192, K=21760 in bf16: every kernel (M <= 32,
    32 < M < 128, M >= 128)."""
    _case_check(M, 21760, 8192, G)


@pytest.mark.parametrize("G", [-1, 32, 64])
@pytest.mark.parametrize("M,K,N", [(2048, 4096, 4096), (1, 4096, 14336), (33, 4096, 520), (5, 64, 8),
                                   (129, 512, 1032)])
def test_w4a8_bf16_shapes(M, K, N, G):
    if G > 0 and K % G:
        pytest.skip("K not a multiple of G")
    _case_check(M, K, N, G)


@pytest.mark.parametrize("M", [1, 64, 300])
def test_linear_w4a8_bf16_matches_two_steps(M):
    """w4a8_linear on bf16 equals quant_act followed by w4a8_gemm, bit for bit."""
    c = synthgen.w4a8_case(M, 4096, 4096, -1, dtype="bf16")
    x, b, s2 = to_dev(c.x, c.b, c.s2)
    a8, s1 = awq.quant_act(x)
    y1, acc1 = awq.w4a8_gemm(a8, b, s1, s2, want_acc=True)
    y2, s1b, acc2 = awq.linear_w4a8(x, b, s2, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(acc1, acc2) and torch.equal(s1, s1b) and torch.equal(y1, y2)


@pytest.mark.parametrize("G", [-1, 128])
@pytest.mark.parametrize("scale", [1.0, 2.0 ** -124])
def test_linear_w4a8_bf16_fused_token(G, scale):
    """One bf16 token on the QQQ shape runs the fused quantise-and-GEMM
    kernel: a8 (read back through acc), s1 and y equal the two launches bit
    for bit, and s1 the oracle's.  At 2^-124 the row's s1 is a subnormal fp32
    value, which the fused kernel quantises through the divide."""
    c = synthgen.w4a8_case(1, 21760, 8192, G, dtype="bf16")
    xs = (c.x.double() * scale).to(torch.bfloat16)
    x, b, s2 = to_dev(xs, c.b, c.s2)
    s3 = None if c.s3 is None else to_dev(c.s3)[0]
    a8, s1 = awq.quant_act(x)
    y1, acc1 = awq.w4a8_gemm(a8, b, s1, s2, s3, G, want_acc=True)
    y2, s1b, acc2 = awq.linear_w4a8(x, b, s2, s3, G, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(s1, s1b) and torch.equal(acc1, acc2) and torch.equal(y1, y2)
    _, es1 = orc().quant_act(xs, dtype=BF16)
    assert np.array_equal(s1b.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    if scale != 1.0:
        assert 0.0 < float(s1b.cpu()[0]) < 2.0 ** -126


def test_w4a8_bf16_acc_equals_fp16():
    """The int32 accumulators do not depend on the scale type."""
    c = synthgen.w4a8_case(64, 4096, 1024, 64, dtype="bf16")
    x, b, s2, s3 = to_dev(c.x, c.b, c.s2, c.s3)
    a8, s1 = awq.quant_act(x)
    _, acc_b = awq.w4a8_gemm(a8, b, s1, s2, s3, 64, want_acc=True)
    _, acc_h = awq.w4a8_gemm(a8, b, s1, s2.to(torch.float16), s3.to(torch.float16), 64, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(acc_b, acc_h)
