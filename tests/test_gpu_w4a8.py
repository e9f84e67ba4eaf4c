"""GPU W4A8 (QQQ-style) vs the CPU oracle: activation quantisation and the int32
accumulators bit-exact, the fp16 output within the fp16 tolerance of the fp64
result computed from the same quantised activations."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import THREADS, check_fp, dev, orc, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _quant_check(x_cpu):
    a8, s1 = awq.quant_act(x_cpu.to(dev()))
    torch.cuda.synchronize()
    ea8, es1 = orc().quant_act(x_cpu)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    assert np.array_equal(a8.cpu().numpy(), ea8)
    return a8, s1, ea8, es1


@pytest.mark.parametrize("M,K", [(1, 21760), (16, 21760), (64, 21760), (256, 4096), (3, 7), (5, 1000)])
def test_quant_act_bit_exact(M, K):
    x = synthgen.activations(M, K, seed=M * 131 + K)
    x = x * torch.logspace(-4, 3, M).to(torch.float16)[:, None]  # rows across magnitudes
    _quant_check(x.to(torch.float16))


@pytest.mark.parametrize("K", [8192, 8200, 40968, 131072, 131080])
def test_quant_act_row_lengths(K):
    """Row lengths at the boundaries of the register-resident variants (and
    past them, where the two-pass kernel takes over)."""
    x = synthgen.activations(3, K, seed=K)
    x = x * torch.tensor([1e-3, 1.0, 30.0], dtype=torch.float16)[:, None]
    _quant_check(x.to(torch.float16))


@pytest.mark.parametrize("K", [4096, 21760])
def test_quant_act_ties(K):
    """Rows made of exact ties: amax 127 (s1 = 1) with half-integer values, and
    amax 63.5 (s1 = 0.5) with quarter-integer values."""
    g = torch.Generator().manual_seed(K)
    r1 = (torch.randint(-254, 255, (K,), generator=g).float() / 2)
    r2 = (torch.randint(-254, 255, (K,), generator=g).float() / 4)
    r1[0], r2[0] = 127.0, 63.5
    _quant_check(torch.stack([r1, r2]).to(torch.float16))


def test_quant_act_edge_rows():
    """Worked examples, a zero row, a subnormal-scale row (clamp active) and
    ties: bit-exact with the oracle."""
    rows = [[127, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -127],
            [0.0] * 8,
            [2.0 ** -14, -(2.0 ** -14), 0, 0, 2.0 ** -15, 0, 0, 0],
            [65504.0, -65504.0, 1, 2, 3, 4, 5, 6]]
    x = torch.tensor(rows, dtype=torch.float16)
    a8, s1, ea8, es1 = _quant_check(x)
    assert a8.cpu()[0].tolist() == [127, 2, 4, -2, -4, 0, 2, -127]
    assert a8.cpu()[2, :2].tolist() == [127, -128]
    assert float(s1.cpu()[1]) == 0.0


def _w4a8_case_check(M, K, N, G, full_rows=False):
    c = synthgen.w4a8_case(M, K, N, G)
    x, b, s2, s3 = to_dev(c.x, c.b, c.s2, c.s3)
    a8, s1 = awq.quant_act(x)
    y, acc = awq.w4a8_gemm(a8, b, s1, s2, s3, G, want_acc=True)
    torch.cuda.synchronize()
    ea8, es1 = orc().quant_act(c.x)
    assert np.array_equal(a8.cpu().numpy(), ea8)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), es1.view(np.uint32))
    rows = np.arange(M) if (full_rows or M <= 16) else sample_rows(M, seed=M)
    eacc, y64 = orc().w4a8(ea8[rows], c.b, es1[rows], c.s2, c.s3, G, nthreads=THREADS)
    assert np.abs(eacc).max() < 2 ** 31
    gacc = acc.cpu().numpy()[rows].astype(np.int64)
    assert np.array_equal(gacc, eacc), f"acc mismatch at {np.argwhere(gacc != eacc)[:5]}"
    check_fp(y.cpu()[torch.as_tensor(rows)], y64, "f16", f"w4a8 M={M} K={K} N={N} G={G}")


@pytest.mark.parametrize("G", [-1, 128])
@pytest.mark.parametrize("M", [1, 16, 64, 256, 1024])
def test_w4a8_qqq_shape(M, G):
    """The QQQ GEMM shape N=8192, K=21760 (per-channel and g128)."""
    _w4a8_case_check(M, 21760, 8192, G)


@pytest.mark.parametrize("G", [-1, 32, 64, 128])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 4096), (2048, 4096, 4096), (1, 4096, 14336), (2048, 4096, 14336),
                                   (300, 4096, 1032), (5, 64, 8),
                                   (17, 128, 136), (40, 256, 24), (129, 512, 1032), (33, 4096, 520),
                                   # 128 x 256 tiles with a ragged last row and column tile
                                   (2049, 256, 4104), (4000, 128, 2056),
                                   # one 128 x 256 tile per CU (K split inside the workgroup),
                                   # ragged, with an odd stage count
                                   (1000, 1088, 8184),
                                   # the skinny kernel where the atomic cap leaves one split
                                   # (48 and 64 rows on 4096 x 14336) or five (48 on 4096 x 4096)
                                   (48, 4096, 14336), (64, 4096, 14336), (48, 4096, 4096)])
def test_w4a8_shapes(M, K, N, G):
    if G > 0 and K % G:
        pytest.skip("K not a multiple of G")
    _w4a8_case_check(M, K, N, G)


def test_w4a8_group16_equals_channel():
    """Per-group with every s3 = 16 and s2/16 reproduces per-channel exactly."""
    c = synthgen.w4a8_case(37, 1024, 512, -1)
    x, b, s2 = to_dev(c.x, c.b, c.s2)
    a8, s1 = awq.quant_act(x)
    y1, acc1 = awq.w4a8_gemm(a8, b, s1, s2, None, -1, want_acc=True)
    s3 = torch.full((1024 // 64, 512), 16.0, dtype=torch.float16, device=dev())
    y2, acc2 = awq.w4a8_gemm(a8, b, s1, s2 / 16, s3, 64, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(acc2, 16 * acc1)
    assert torch.equal(y1, y2)


def test_w4a8_deterministic():
    c = synthgen.w4a8_case(1, 21760, 8192, -1)
    x, b, s2 = to_dev(c.x, c.b, c.s2)
    a8, s1 = awq.quant_act(x)
    ys = [awq.w4a8_gemm(a8, b, s1, s2) for _ in range(4)]
    torch.cuda.synchronize()
    for yy in ys[1:]:
        assert torch.equal(yy, ys[0])


@pytest.mark.parametrize("G", [-1, 128])
@pytest.mark.parametrize("M,K,N", [(1, 21760, 8192), (1, 4096, 4096), (1, 4096, 14336), (2, 16384, 4096),
                                   (3, 4096, 1032), (5, 64, 8), (16, 2048, 512), (16, 2112, 512),
                                   (2, 21760, 8192), (17, 128, 136), (300, 4096, 1032)])
def test_linear_matches_quant_then_gemm(M, K, N, G):
    """w4a8_linear (quantisation fused into the GEMM for M <= 16 and M*K <=
    32768, the two launches otherwise) gives y, s1 and the int32 accumulators
    bit for bit as w4a8_quant_act followed by w4a8_gemm; rows span magnitudes
    (a zero row and exact ties included) so every rounding case is met."""
    if G > 0 and K % G:
        pytest.skip("K not a multiple of G")
    c = synthgen.w4a8_case(M, K, N, G)
    xc = c.x.clone()
    xc = xc * torch.logspace(-3, 2, M).to(torch.float16)[:, None]
    if M >= 3:
        xc[1] = 0
        xc[2, : K // 2] = torch.arange(K // 2, dtype=torch.float32).remainder(255).sub(127).div(2).to(torch.float16)
        xc[2, 0] = 127
    x, b, s2, s3 = to_dev(xc.to(torch.float16), c.b, c.s2, c.s3)
    a8, s1 = awq.quant_act(x)
    y1, acc1 = awq.w4a8_gemm(a8, b, s1, s2, s3, G, want_acc=True)
    y2, s1b, acc2 = awq.linear_w4a8(x, b, s2, s3, G, want_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(s1b.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(acc2, acc1)
    assert torch.equal(y2.view(torch.int16), y1.view(torch.int16))
    # and against the oracle, from the oracle's own quantisation of x
    ea8, es1 = orc().quant_act(xc.to(torch.float16))
    rows = np.arange(M) if M <= 16 else sample_rows(M, seed=M)
    eacc, y64 = orc().w4a8(ea8[rows], c.b, es1[rows], c.s2, c.s3, G, nthreads=THREADS)
    assert np.array_equal(acc2.cpu().numpy()[rows].astype(np.int64), eacc)
    # the rows span five decades, so outputs reach the hundreds: y is one fp16
    # rounding of acc * s1 * s2 (fp32), i.e. within half an fp16 ulp of the
    # fp64 value (plus the fp32 product's own rounding)
    yg = y2.cpu()[torch.as_tensor(rows)].double().numpy()
    assert np.all(np.abs(yg - y64) <= 2.0 ** -11 * np.abs(y64) * (1 + 2.0 ** -20) + 2.0 ** -25), \
        f"w4a8_linear M={M} K={K} N={N} G={G}: y beyond one fp16 rounding of the exact value"


def test_linear_repeated_calls_and_split_workspace():
    """Back-to-back fused calls of different shapes share the split-K workspace
    and leave it re-armed; results stay identical to the two-step path."""
    for (M, K, N) in [(1, 21760, 8192), (1, 4096, 4096), (4, 8192, 14336), (1, 21760, 8192)]:
        c = synthgen.w4a8_case(M, K, N, -1)
        x, b, s2 = to_dev(c.x, c.b, c.s2)
        a8, s1 = awq.quant_act(x)
        y1 = awq.w4a8_gemm(a8, b, s1, s2)
        y2 = awq.linear_w4a8(x, b, s2)
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), y1.view(torch.int16)), (M, K, N)


# (M, K, N, G, expected plan: tiles_n, tiles_m, wave groups splitting K, K splits)
LDS_CASES = [
    (2048, 4096, 8192, -1, (32, 16, 1, 1)),   # 128 x 256 tiles (8 waves), two per CU
    (2048, 4096, 4096, -1, (16, 16, 2, 1)),   # one 128 x 256 tile per CU: K split inside the workgroup
    (1024, 4096, 4096, 128, (32, 8, 1, 1)),   # 128 x 128 tiles (4 waves), per group
    (256, 4096, 4096, -1, (32, 2, 1, 4)),     # few tiles: K split through int32 partial tiles
    (300, 4096, 1032, 64, (9, 3, 1, 4)),      # ragged rows and columns, split, per group
    (128, 4096, 14336, -1, (112, 1, 1, 2)),   # short K: the splits that fit whole (256 // 112)
    (384, 21760, 8192, -1, (64, 3, 1, 2)),    # long K: rounded up (192 tiles)
    (384, 4096, 14336, 128, (56, 3, 2, 1)),   # 168 wide tiles: more than half the CUs
]


@pytest.mark.parametrize("M,K,N,G,plan", LDS_CASES, ids=lambda v: str(v))
def test_lds_gemm_output_bit_exact(M, K, N, G, plan):
    """The LDS-pipelined W4A8 GEMM's fp16 output is one rounding of
    acc * s1 * s2: with power-of-two s1 and s2 and |acc| < 2^24 that product
    is exact in fp32, so y must equal the oracle's fp64 value rounded once,
    bit for bit (and acc exactly), on every tile configuration."""
    info = awq.plan_info(awq.AWQ_OP_W4A8_GEMM, M, N, K, G)
    if info["cu_count"] == 256:
        assert info["kernel"] == 2 and (info["tiles_n"], info["tiles_m"], info["ksplit"], info["splits"]) == plan, info
    g = torch.Generator().manual_seed(M + N + K)
    a8 = torch.randint(-128, 128, (M, K), generator=g, dtype=torch.int64).to(torch.int8)
    s1 = torch.pow(2.0, -torch.randint(5, 12, (M,), generator=g).to(torch.float32))
    c = synthgen.w4a8_case(1, K, N, G)
    s2 = torch.pow(2.0, -torch.randint(3, 9, (N,), generator=g).to(torch.float32)).to(torch.float16)
    y, acc = awq.w4a8_gemm(*to_dev(a8, c.b, s1, s2, c.s3), G, want_acc=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, seed=M, tile=128)
    eacc, y64 = orc().w4a8(a8.numpy()[rows], c.b, s1.numpy()[rows], s2, c.s3, G, nthreads=THREADS)
    assert np.abs(eacc).max() < 2 ** 24
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), eacc)
    exp = torch.from_numpy(y64).to(torch.float16)
    got = y.cpu()[torch.as_tensor(rows)]
    assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), int((got != exp).sum())


def test_register_tiled_kernel_past_the_lds_offsets():
    """Activation codes of more than 2^31 bytes (M = 16400, K = 131008: 2.1 GB)
    run the register-tiled kernel, since the LDS GEMM addresses them with
    32-bit offsets.  Codes drawn on the device from a seeded generator;
    sampled rows (both ends, one per 256-row block) against the oracle:
    accumulators exact, fp16 output bit for bit (power-of-two s1 and s2)."""
    M, K, N = 16400, 131008, 64
    info = awq.plan_info(awq.AWQ_OP_W4A8_GEMM, M, N, K, -1)
    assert info["kernel"] == 1, info
    gen = torch.Generator(device=dev()).manual_seed(16400)
    a8 = torch.randint(-128, 128, (M, K), generator=gen, device=dev(), dtype=torch.int8)
    g = torch.Generator().manual_seed(3)
    s1 = torch.pow(2.0, -torch.randint(5, 12, (M,), generator=g).to(torch.float32))
    s2 = torch.pow(2.0, -torch.randint(3, 9, (N,), generator=g).to(torch.float32)).to(torch.float16)
    c = synthgen.w4a8_case(1, K, N, -1)
    y, acc = awq.w4a8_gemm(a8, *to_dev(c.b, s1, s2), want_acc=True)
    torch.cuda.synchronize()
    rows = sample_rows(M, seed=5, tile=256)
    ra = a8[torch.as_tensor(rows, device=dev())].cpu().numpy()
    del a8
    eacc, y64 = orc().w4a8(ra, c.b, s1.numpy()[rows], s2, None, -1, nthreads=THREADS)
    assert np.abs(eacc).max() < 2 ** 24
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), eacc)
    exp = torch.from_numpy(y64).to(torch.float16)
    got = y.cpu()[torch.as_tensor(rows)]
    assert torch.equal(got.view(torch.int16), exp.view(torch.int16)), int((got != exp).sum())


def test_w4a8_largest_k_all_minimum():
    """K = 131008, the largest K the library accepts: a row of -2^-14 quantises
    to s1 = 2^-21 and a8 = -128 everywhere, and with every weight -8 the
    kernels' int32 sum of (-128) * (16 * -8) reaches 2^14 * K = 2146435072,
    just below 2^31.  The accumulators must come back exact (acc = 1024 K),
    through the two-step layer call and the separate calls alike."""
    M, K, N = 2, 131008, 64
    x = torch.full((M, K), -(2.0 ** -14), dtype=torch.float16)
    x[1] = synthgen.activations(1, K, seed=5)[0]
    b = torch.full((K // 8, N), -0x77777778, dtype=torch.int32)  # 0x88888888: every nibble -8
    s2 = (0.002 + 0.018 * torch.rand(N, generator=torch.Generator().manual_seed(1))).to(torch.float16)
    xd, bd, s2d = to_dev(x, b, s2)
    y1, s1b, acc1 = awq.linear_w4a8(xd, bd, s2d, want_acc=True)
    a8, s1 = awq.quant_act(xd)
    y2, acc2 = awq.w4a8_gemm(a8, bd, s1, s2d, want_acc=True)
    torch.cuda.synchronize()
    ea8, es1 = orc().quant_act(x)
    assert float(es1[0]) == 2.0 ** -21 and np.all(ea8[0] == -128)
    assert np.array_equal(a8.cpu().numpy(), ea8)
    eacc, y64 = orc().w4a8(ea8, b, es1, s2, nthreads=THREADS)
    assert eacc[0, 0] == 1024 * K
    for acc, y in ((acc1, y1), (acc2, y2)):
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), eacc)
        exp = torch.from_numpy(y64).to(torch.float16)
        assert torch.equal(y.cpu()[0], exp[0])  # acc * s1 * s2 with s1 a power of two: one rounding
        check_fp(y.cpu()[1:], y64[1:], "f16", "largest K, random row")
