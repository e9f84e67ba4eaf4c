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
                                   (300, 4096, 1032), (7, 130944, 64),
                                   # the skinny kernel with one split (the atomic cap) and with five
                                   (64, 4096, 14336), (48, 4096, 4096),
                                   # the LDS GEMM's K splits: 8 of 14 stages, 4 of 8, 5 of 112 (uneven)
                                   (128, 14336, 4096), (256, 4096, 4096), (384, 14336, 4096)])
def test_fp8_shapes(M, K, N):
    rows = None if M <= 300 else sample_rows(M, seed=N)
    _gemm_check(M, K, N, 0, rows=rows)


def test_fp8_register_tiled_kernel_past_the_lds_offsets():
    """Activation codes of more than 2^31 bytes (M = 16401, K = 130944) run
    the register-tiled kernel, since the LDS GEMM addresses them with 32-bit
    offsets.  Activations drawn on the device from a seeded generator and
    quantised there; sampled rows (both ends, one per 256-row block) against
    the oracle: codes, s1 and row sums bit-exact, the sums within the fp32
    accumulation bound, the output within the fp16 bar."""
    M, K, N = 16401, 130944, 64
    info = awq.plan_info(awq.AWQ_OP_W4A8_FP8_GEMM, M, N, K, -1)
    assert info["kernel"] == 1, info
    gen = torch.Generator(device=dev()).manual_seed(16401)
    x = torch.randn((M, K), generator=gen, device=dev(), dtype=torch.float16)
    c = synthgen.w4a8_case(1, K, N, -1)
    b, s2 = to_dev(c.b, c.s2)
    a, s1, asum = awq.quant_act_fp8(x)
    y, acc = awq.w4a8_fp8_gemm(a, b, s1, asum, s2, want_acc=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, seed=6, tile=256)
    ridx = torch.as_tensor(rows, device=dev())
    xr, ar = x[ridx].cpu(), a[ridx].cpu().numpy()
    del x, a
    ea, es1, esum = orc().quant_act_fp8(xr, 0)
    assert np.array_equal(ar, ea)
    assert np.array_equal(s1.cpu().numpy()[rows].view(np.uint32), es1.view(np.uint32))
    assert np.array_equal(asum.cpu().numpy()[rows].view(np.uint32), esum.view(np.uint32))
    eacc, y64 = orc().w4a8_fp8(ea, c.b, es1, c.s2, 0)
    av = np.abs(torch.from_numpy(ea).view(torch.float8_e4m3fn).double().numpy())
    bound = K * 2.0 ** -24 * 15 * av.sum(axis=1, keepdims=True) + 8 * np.abs(esum[:, None]) * 2.0 ** -23 \
        + np.abs(eacc) * 2.0 ** -23
    gacc = acc.cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.abs(gacc - eacc) <= bound), float(np.max(np.abs(gacc - eacc) - bound))
    check_fp(y.cpu()[torch.as_tensor(rows)], y64, "f16", f"fp8 M={M} K={K} N={N}")


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


def _linear_check(M, K, N, dt, x=None, large=False):
    """w4a8_fp8_linear against the two launches and the oracle.  A single
    token runs the fused kernel: s1 identical to the quantiser's, acc within
    one fp32 rounding of the two-launch acc (the fused path forms acc once
    from the exact split-K sum, the two-launch path rounds t to fp32 first),
    y within one rounding of the activation type of it; more tokens run the
    two launches and must match them bit for bit."""
    c = synthgen.w4a8_case(M, K, N, -1, dtype="f16" if dt == 0 else "bf16")
    xs = c.x if x is None else x.to(_T[dt])
    xd, b, s2 = to_dev(xs, c.b, c.s2)
    y, s1, acc = awq.linear_w4a8_fp8(xd, b, s2, want_acc=True)
    a2, s12, asum2 = awq.quant_act_fp8(xd)
    y2, acc2 = awq.w4a8_fp8_gemm(a2, b, s12, asum2, s2, want_acc=True)
    torch.cuda.synchronize()
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s12.cpu().numpy().view(np.uint32))
    g, g2 = acc.cpu().numpy().astype(np.float64), acc2.cpu().numpy().astype(np.float64)
    yf, yf2 = y.cpu().double().numpy(), y2.cpu().double().numpy()
    if M > 1:
        assert np.array_equal(g, g2) and torch.equal(y.cpu(), y2.cpu())
    else:
        asum = np.abs(asum2.cpu().numpy().astype(np.float64))[:, None]
        # t rounded to fp32 (<= 512 |t| 2^-24 = (|acc| + 8 asum) 2^-24), asum rounded to
        # fp32 (8 asum 2^-24) and the FMA's rounding on the two-launch side, one
        # rounding on the fused side
        bound = (3 * np.abs(g2) + 16 * asum) * 2.0 ** -24 + 1e-30
        assert np.all(np.abs(g - g2) <= bound), float(np.max(np.abs(g - g2) - bound))
        ulp = 2.0 ** -10 if dt == 0 else 2.0 ** -7
        assert np.all(np.abs(yf - yf2) <= np.abs(yf2) * ulp + 2.0 ** -24), float(np.max(np.abs(yf - yf2)))
    # and against the oracle, from the codes the quantiser produces
    ea, es1, esum = orc().quant_act_fp8(xs, dt)
    eacc, y64 = orc().w4a8_fp8(ea, c.b, es1, c.s2, dt)
    av = np.abs(torch.from_numpy(ea).view(torch.float8_e4m3fn).double().numpy())
    bound = K * 2.0 ** -24 * 15 * av.sum(axis=1, keepdims=True) + 8 * np.abs(esum[:, None]) * 2.0 ** -23 \
        + np.abs(eacc) * 2.0 ** -23
    assert np.all(np.abs(g - eacc) <= bound), float(np.max(np.abs(g - eacc) - bound))
    if not large:
        check_fp(y.cpu(), y64, "f16" if dt == 0 else "bf16", f"fp8 linear M={M} K={K} N={N}")
    else:
        # outputs far from unit size: the absolute part of the output bar does
        # not apply.  Per element, acc is held to the fp32-accumulation bound
        # above (a few largest codes beside many small ones make that bound,
        # not the output rounding, the larger term); the output to the
        # relative bar.
        rel = float(np.linalg.norm(yf - y64) / np.linalg.norm(y64))
        assert np.all(np.isfinite(yf)) and rel <= 2e-3, rel


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("M,K,N", [(1, 21760, 8192), (1, 4096, 4096), (1, 4096, 14336), (1, 128, 8), (1, 256, 136),
                                   (1, 130944, 64), (3, 4096, 1032), (16, 21760, 8192)])
def test_fp8_linear(M, K, N, dt):
    _linear_check(M, K, N, dt)


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("row", ["zero", "tiny", "huge", "ties"])
def test_fp8_linear_edge_rows(row, dt):
    """The fused single-token path on the rows that take other branches of the
    quantiser: all zero (s1 = 0, codes 0), tiny (bf16: s1 below 2^-126, the
    exactly divided quotients), the largest finite value (s1 at its largest),
    and values that sit on E4M3 rounding ties after the division by s1 = 1."""
    K, N = 4096, 1032
    g = torch.Generator().manual_seed(11 + dt)
    if row == "zero":
        x = torch.zeros(1, K)
    elif row == "tiny":
        x = torch.randn(1, K, generator=g) * (2.0 ** -130 if dt == 1 else 2.0 ** -20)
    elif row == "huge":
        # four entries at the largest fp16 value (bf16: 1e34; its largest would
        # overflow y in fp32 on either path) set s1 = max / 448; the rest
        # quantise to small codes, so y stays finite
        big = 65504.0 if dt == 0 else 1e34
        x = torch.randn(1, K, generator=g) * 1e-3 * big
        x[0, torch.randperm(K, generator=g)[:4]] = torch.tensor([1.0, -1.0, 1.0, -1.0]) * big
    else:
        # s1 = 448 / 448 = 1: the codes of 1 + (2j + 1) / 16 sit halfway between E4M3 neighbours
        x = 1.0 + (2 * torch.randint(0, 8, (1, K), generator=g) + 1).float() / 16.0
        x[0, 0] = 448.0
    _linear_check(1, K, N, dt, x=x, large=row in ("huge", "ties"))
