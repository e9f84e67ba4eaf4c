"""GPU INT4-FP8 W4A8 vs the CPU oracle: the E4M3 activation codes, s1 and the
row sums bit-exact; the GEMM's fp32 sums within the bound of fp32 accumulation
and its fp16/bf16 output within the output bar of the fp64 result computed
from the same quantised activations."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import THREADS, check_fp, dev, orc, sample_rows, to_dev

pytestmark = pytest.mark.gpu

_T = {0: torch.float16, 1: torch.bfloat16}


def _quant_check(xb: torch.Tensor, dt: int):
    a, s1, asum = awq.quant_act_fp8(xb.to(dev()))
    torch.cuda.synchronize()
    ea, es1, esum = orc().quant_act_fp8(xb, dt)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    ga = a.cpu().numpy()
    assert np.array_equal(ga, ea), f"codes differ at {np.argwhere(ga != ea)[:5]}"
    assert np.array_equal(asum.cpu().numpy().view(np.uint32), esum.view(np.uint32))
    return a, s1, asum, ea, es1, esum


@pytest.mark.parametrize("dt", [0, 1])
def test_fp8_quant_every_value_per_binade(dt):
    """Rows made of every finite non-negative value of the activation type up
    to 2^e (and their negatives), one row per e: every quotient x / s1 the
    encoder can meet for s1 = act(2^e / 448) is checked against the oracle."""
    if dt == 0:
        vals = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
        exps = range(-14, 16)
    else:
        vals = torch.arange(0, 0x7F80, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().numpy()
        exps = list(range(-126, 128, 9)) + [127]
    rows = []
    for e in exps:
        v = vals[vals <= 2.0 ** e]
        rows.append(np.concatenate([v, -v]))
    K = max(len(r) for r in rows)
    K += (-K) % 8
    x = np.zeros((len(rows), K), np.float32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    _quant_check(torch.from_numpy(x).to(_T[dt]), dt)


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("M,K", [(1, 21760), (16, 4096), (64, 21760), (3, 7), (5, 1000), (2, 131072), (4, 32768), (2, 65536), (3, 8200)])
def test_fp8_quant_rows(M, K, dt):
    x = synthgen.activations(M, K, seed=M * 7 + K).float()
    x = x * torch.logspace(-4, 3, M)[:, None]
    if M >= 3:
        x[1] = 0
    _quant_check(x.to(_T[dt]), dt)


def _gemm_check(M, K, N, dt, rows=None):
    c = synthgen.w4a8_case(M, K, N, -1, dtype="f16" if dt == 0 else "bf16")
    x, b, s2 = to_dev(c.x, c.b, c.s2)
    a, s1, asum = awq.quant_act_fp8(x)
    y, acc = awq.w4a8_fp8_gemm(a, b, s1, asum, s2, want_acc=True)
    torch.cuda.synchronize()
    ea, es1, esum = orc().quant_act_fp8(c.x, dt)
    assert np.array_equal(a.cpu().numpy(), ea)
    rows = np.arange(M) if rows is None else rows
    eacc, y64 = orc().w4a8_fp8(ea[rows], c.b, es1[rows], c.s2, dt)
    # fp32 accumulation: every partial sum of sum_k a (q + 8) 2^-9 rounds with
    # a relative error of 2^-24, so the sum is off by at most about
    # K 2^-24 sum_k |a| 15 2^-9 (times 2^9 for acc), plus the roundings of
    # 8 asum and of the final difference
    av = np.abs(torch.from_numpy(ea[rows]).view(torch.float8_e4m3fn).double().numpy())
    bound = K * 2.0 ** -24 * 15 * av.sum(axis=1, keepdims=True) + 8 * np.abs(esum[rows, None]) * 2.0 ** -23 \
        + np.abs(eacc) * 2.0 ** -23
    gacc = acc.cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.abs(gacc - eacc) <= bound), float(np.max(np.abs(gacc - eacc) - bound))
    check_fp(y.cpu()[torch.as_tensor(rows)], y64, "f16" if dt == 0 else "bf16", f"fp8 M={M} K={K} N={N}")
    return y


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("M", [1, 16, 64, 256, 1024])
def test_fp8_qqq_shape(M, dt):
    """The QQQ GEMM shape N=8192, K=21760."""
    _gemm_check(M, 21760, 8192, dt, rows=None if M <= 64 else sample_rows(M, seed=M))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (2048, 4096, 4096), (1, 4096, 14336), (2048, 4096, 14336),
                                   (5, 128, 8), (17, 256, 136), (33, 384, 520), (65, 512, 264), (129, 512, 1032),
                                   (300, 4096, 1032), (7, 130944, 64)])
def test_fp8_shapes(M, K, N):
    rows = None if M <= 300 else sample_rows(M, seed=N)
    _gemm_check(M, K, N, 0, rows=rows)


def test_fp8_deterministic():
    c = synthgen.w4a8_case(4, 21760, 8192, -1)
    x, b, s2 = to_dev(c.x, c.b, c.s2)
    a, s1, asum = awq.quant_act_fp8(x)
    ys = [awq.w4a8_fp8_gemm(a, b, s1, asum, s2) for _ in range(4)]
    c2 = synthgen.w4a8_case(300, 4096, 1032, -1)
    x2, b2, s22 = to_dev(c2.x, c2.b, c2.s2)
    a2, s12, asum2 = awq.quant_act_fp8(x2)
    y2 = [awq.w4a8_fp8_gemm(a2, b2, s12, asum2, s22) for _ in range(3)]
    torch.cuda.synchronize()
    for yy in ys[1:]:
        assert torch.equal(yy.view(torch.int16), ys[0].view(torch.int16))
    for yy in y2[1:]:
        assert torch.equal(yy.view(torch.int16), y2[0].view(torch.int16))
