"""GPU W4A16 GEMV / GEMM vs the fp64 CPU oracle.

Shapes are the workloads the pages measure on (opt-125m fc1; Llama-2-7B decode
layers; Llama-3-8B prefill layers; the K=4096, N=14336 group-size / dtype /
symmetric variants) plus ragged and degenerate edge cases.  Full-size prefill
cases are checked on sampled rows (every column tile is still covered)."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import THREADS, check_fp, dev, orc, sample_rows, to_dev

pytestmark = pytest.mark.gpu

F16, BF16 = 0, 1


def _run(case, entry="gemm", split_k=0, rows=None):
    x, qw, s, qz = to_dev(case.x, case.qweight, case.scales, case.qzeros)
    fn = awq.gemm_w4a16 if entry == "gemm" else awq.gemv_w4a16
    y = fn(x, qw, s, qz, case.G, split_k=split_k)
    torch.cuda.synchronize()
    xs = case.x if rows is None else case.x[torch.as_tensor(rows)]
    y64 = orc().w4a16(xs, case.qweight, case.scales, case.qzeros, case.G,
                      BF16 if case.dtype == "bf16" else F16, nthreads=THREADS)
    yg = y.cpu() if rows is None else y.cpu()[torch.as_tensor(rows)]
    return yg, y64, y


def test_opt125m_fc1_m16():
    """opt-125m fc1: M=16, K=768, N=3072, g128, seed 0 -- checked in full."""
    c = synthgen.w4a16_case(16, 768, 3072, 128, seed=0)
    yg, y64, _ = _run(c)
    check_fp(yg, y64, "f16", "opt125m fc1")


LLAMA2_7B = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]


@pytest.mark.parametrize("K,N", LLAMA2_7B)
@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_gemv_llama2_7b(M, K, N):
    c = synthgen.w4a16_case(M, K, N, 128)
    yg, y64, _ = _run(c, "gemv")
    check_fp(yg, y64, "f16", f"gemv M={M} K={K} N={N}")


LLAMA3_8B = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)]


@pytest.mark.parametrize("K,N", LLAMA3_8B)
@pytest.mark.parametrize("M", [64, 256, 1024, 2048, 4096])
def test_gemm_llama3_8b_sampled(M, K, N):
    c = synthgen.w4a16_case(M, K, N, 128)
    rows = sample_rows(M, seed=M + N)
    yg, y64, _ = _run(c, "gemm", rows=rows)
    check_fp(yg, y64, "f16", f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("K,N", [(4096, 4096), (4096, 14336)])
@pytest.mark.parametrize("M", [1, 2048])
def test_target_shapes(M, K, N):
    """The stated target shapes, at M=1 through the GEMV entry and at M=2048."""
    c = synthgen.w4a16_case(M, K, N, 128, x_rows=None)
    rows = None if M == 1 else sample_rows(M, seed=N)
    yg, y64, _ = _run(c, "gemv" if M == 1 else "gemm", rows=rows)
    check_fp(yg, y64, "f16", f"target M={M} K={K} N={N}")


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("M", [1, 512, 1024])
def test_group_dtype_sym_variants(M, G, dtype, sym):
    c = synthgen.w4a16_case(M, 4096, 14336, G, dtype=dtype, sym=sym)
    rows = None if M == 1 else sample_rows(M, seed=G)
    yg, y64, _ = _run(c, "gemv" if M == 1 else "gemm", rows=rows)
    check_fp(yg, y64, dtype, f"variant M={M} G={G} {dtype} sym={sym}")


def test_symmetric_equals_zero_point_8():
    """qzeros = NULL must equal qzeros filled with 0x88888888, bit for bit."""
    for M in (1, 40, 300):
        c = synthgen.w4a16_case(M, 1024, 2048, 64, sym=True)
        x, qw, s = to_dev(c.x, c.qweight, c.scales)
        z8 = torch.full((1024 // 64, 2048 // 8), -0x77777778, dtype=torch.int32, device=dev())
        a = awq.gemm_w4a16(x, qw, s, None, 64)
        b = awq.gemm_w4a16(x, qw, s, z8, 64)
        torch.cuda.synchronize()
        assert torch.equal(a, b), M


def test_exact_special_case_bit_identical():
    """z = 0, s = 2^-3, x in {-1,0,1}: every sum is an exact dyadic, so the fp16
    output must equal the rounded oracle value bit for bit (pins layout and
    indexing of every kernel variant)."""
    g = torch.Generator().manual_seed(3)
    for (M, K, N) in [(1, 128, 1024), (3, 256, 136), (8, 128, 4096), (16, 384, 512), (29, 256, 264),
                      (64, 256, 768), (200, 512, 520)]:
        X = torch.randint(-1, 2, (M, K), generator=g).to(torch.float16)
        qw = torch.randint(-(2 ** 31), 2 ** 31, (K, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
        qz = torch.zeros(K // 128, N // 8, dtype=torch.int32)
        s = torch.full((K // 128, N), 0.125, dtype=torch.float16)
        y64 = orc().w4a16(X, qw, s, qz, 128)
        exp = torch.from_numpy(y64).to(torch.float16)
        for entry in (("gemv", "gemm") if M <= 8 else ("gemm",)):
            fn = awq.gemv_w4a16 if entry == "gemv" else awq.gemm_w4a16
            for split in (0, 1, 3):
                if split > K // 32:
                    continue
                y = fn(*to_dev(X, qw, s, qz), 128, split_k=split)
                torch.cuda.synchronize()
                assert torch.equal(y.cpu(), exp), (M, K, N, entry, split)


# (M, K, N, split_k, expected plan: row tiles, wave groups splitting K, K
# splits, tile columns)
MAIN_TILE_CASES = [
    (2048, 4096, 8192, 0, (16, 1, 1, 256)),  # 256 tiles of 256 x 256: the large-M configuration
    (2200, 4096, 4384, 0, (16, 1, 1, 256)),  # the same, ragged: last row tile 152 rows, last column tile 32
    (2048, 4096, 4096, 0, (16, 2, 1, 128)),  # 256 tiles of 256 x 128: two wave groups split K in the workgroup
    (4096, 4096, 6144, 0, (16, 1, 1, 128)),  # 768 tiles of 256 x 128: more even over the CUs than 384 wide ones
    (2048, 4096, 8192, 2, (16, 1, 2, 128)),  # K split through partial tiles
    (2048, 4096, 4096, 3, (16, 1, 3, 128)),  # three splits, 64 stages (uneven)
    (1024, 4096, 4096, 0, (8, 2, 1, 128)),   # 128-row tiles where 256-row ones would leave CUs idle
    (512, 14336, 4096, 0, (8, 2, 2, 128)),   # K = 14336: K split and in-workgroup split together
    (768, 14336, 4096, 0, (8, 1, 4, 128)),   # long K on 128-row tiles: four single-group splits
    (384, 14336, 4096, 0, (8, 1, 8, 128)),   # eight single-group splits where two-group ones idle CUs
    (96, 14336, 4096, 0, (8, 2, 8, 128)),    # eight splits (two load batches in the last workgroup)
    (96, 4096, 4096, 0, (8, 2, 4, 128)),     # below 128 rows: 128-row tiles, K split both ways
    (100, 4096, 6144, 0, (8, 2, 4, 128)),    # the same with a ragged last row tile
    # K splits with a ragged last column tile (its quads past N never stored)
    (100, 4096, 4384, 0, (8, 2, 4, 128)),
    (700, 14336, 4384, 0, (8, 1, 3, 128)),   # single-group splits: 16 quads a lane, two chunks of 8
    (130, 4096, 4128, 0, (8, 2, 3, 128)),
]


@pytest.mark.parametrize("M,K,N,split,plan", MAIN_TILE_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_special_case_main_tiles(M, K, N, split, plan, dtype):
    """The bit-exact special case (z = 0, s = 2^-3, x in {-1, 0, 1}) at full
    size on every configuration of the LDS GEMM: the exact sums are multiples
    of 1/8 below 2^21, so the GPU's fp32 accumulation is exact and both sides
    round the same value once.  Checked on sampled rows (one in every 256-row
    tile), all columns."""
    info = awq.plan_info(awq.AWQ_OP_GEMM_W4A16, M, N, K, 128, split)
    if info["cu_count"] == 256:
        assert info["kernel"] == 3, info
        assert (info["row_tiles"], info["ksplit"], info["splits"], info["tile_cols"]) == plan, info
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    g = torch.Generator().manual_seed(M * 7 + N + split)
    X = torch.randint(-1, 2, (M, K), generator=g).to(tdt)
    qw = torch.randint(-(2 ** 31), 2 ** 31, (K, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
    qz = torch.zeros(K // 128, N // 8, dtype=torch.int32)
    s = torch.full((K // 128, N), 0.125, dtype=tdt)
    y = awq.gemm_w4a16(*to_dev(X, qw, s, qz), 128, split_k=split)
    torch.cuda.synchronize()
    rows = sample_rows(M, seed=M + N)
    y64 = orc().w4a16(X[torch.as_tensor(rows)], qw, s, qz, 128, F16 if dtype == "f16" else BF16, nthreads=THREADS)
    exp = torch.from_numpy(y64).to(tdt)
    got = y.cpu()[torch.as_tensor(rows)]
    assert torch.equal(got, exp), (M, K, N, split, dtype, int((got != exp).sum()))


# (M, K, N, G): the streaming kernel (8 < M <= 64): 1, 2 and 4 row tiles,
# 64-k and 32-k chunks, ragged last column tiles, one to fourteen chunks per
# wave (every path of the register ring), K splits from 1 to 8
STREAM_CASES = [(64, 4096, 4096, 128), (33, 4096, 4096, 128), (17, 11008, 4096, 128), (32, 14336, 4096, 128),
                (64, 4096, 1032, 32), (40, 640, 264, 64), (32, 4096, 14336, 128), (20, 4096, 6144, 64),
                (9, 4096, 4096, 128), (16, 11008, 4096, 128), (12, 640, 264, 32), (64, 14336, 4096, 128)]


def _stream_rows(M):
    return 1 if M <= 16 else 2 if M <= 32 else 4


@pytest.mark.parametrize("M,K,N,G", STREAM_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_special_case_stream(M, K, N, G, dtype):
    """The bit-exact special case on the streaming kernel, all rows: its exact
    (q - z) sums, per-chunk scale step, LDS tree and split-K exchange must
    reproduce the exact multiples of 1/8."""
    info = awq.plan_info(awq.AWQ_OP_GEMM_W4A16, M, N, K, G)
    assert info["kernel"] == 5 and info["row_tiles"] == _stream_rows(M), info
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    g = torch.Generator().manual_seed(M * 11 + N + K)
    X = torch.randint(-1, 2, (M, K), generator=g).to(tdt)
    qw = torch.randint(-(2 ** 31), 2 ** 31, (K, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
    qz = torch.zeros(K // G, N // 8, dtype=torch.int32)
    s = torch.full((K // G, N), 0.125, dtype=tdt)
    y = awq.gemm_w4a16(*to_dev(X, qw, s, qz), G)
    torch.cuda.synchronize()
    y64 = orc().w4a16(X, qw, s, qz, G, F16 if dtype == "f16" else BF16, nthreads=THREADS)
    exp = torch.from_numpy(y64).to(tdt)
    assert torch.equal(y.cpu(), exp), (M, K, N, G, dtype, int((y.cpu() != exp).sum()))


@pytest.mark.parametrize("M,K,N,G", STREAM_CASES, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("sym", [False, True])
def test_stream_random(M, K, N, G, dtype, sym):
    c = synthgen.w4a16_case(M, K, N, G, dtype=dtype, sym=sym)
    yg, y64, _ = _run(c)
    check_fp(yg, y64, dtype, f"streaming M={M} K={K} N={N} G={G} {dtype} sym={sym}")


@pytest.mark.parametrize("M,K,N,G,split", [(40, 640, 264, 64, 6), (12, 640, 264, 32, 7), (64, 4096, 4096, 128, 1),
                                           (24, 4096, 4096, 128, 13), (48, 11008, 4096, 128, 3),
                                           (16, 4096, 1032, 128, 20), (64, 4096, 1032, 32, 9)])
def test_stream_explicit_splits(M, K, N, G, split):
    """Explicit K splits on the streaming kernel, including splits that leave
    the last workgroups of a column tile without a chunk (640/64 = 10 chunks
    over 6 splits: ceil(10/6) = 2 each, the sixth empty) -- they still count
    in the split exchange --, the unsplit path, and more splits than the
    exchange loads in one batch (4 at 4 row tiles, 8 below; up to three
    batches); exact special case."""
    info = awq.plan_info(awq.AWQ_OP_GEMM_W4A16, M, N, K, G, split)
    assert info["kernel"] == 5 and info["splits"] == split, info
    g = torch.Generator().manual_seed(M + N + split)
    X = torch.randint(-1, 2, (M, K), generator=g).to(torch.float16)
    qw = torch.randint(-(2 ** 31), 2 ** 31, (K, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
    qz = torch.randint(0, 2 ** 31, (K // G, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
    s = torch.full((K // G, N), 0.25, dtype=torch.float16)
    y = awq.gemm_w4a16(*to_dev(X, qw, s, qz), G, split_k=split)
    torch.cuda.synchronize()
    exp = torch.from_numpy(orc().w4a16(X, qw, s, qz, G, F16, nthreads=THREADS)).to(torch.float16)
    assert torch.equal(y.cpu(), exp), (M, K, N, G, split, int((y.cpu() != exp).sum()))


def test_gemv_bf16_small_outputs():
    """bf16 decode outputs of about 1e-3 (scales near 1.5e-6): the split-K sum
    keeps bf16's relative precision at any magnitude (reading A8's relative
    bar), on the down layer's 43 K splits and the o layer's 32."""
    for M, K, N in ((1, 11008, 4096), (4, 4096, 4096), (8, 4096, 1032)):
        c = synthgen.w4a16_case(M, K, N, 128, dtype="bf16")
        g = torch.Generator().manual_seed(K + M)
        c.scales = (1e-6 + 1e-6 * torch.rand(c.scales.shape, generator=g, dtype=torch.float64)).to(torch.bfloat16)
        yg, y64, _ = _run(c, "gemv")
        rel, mx = check_fp(yg, y64, "bf16", f"bf16 small outputs M={M} K={K} N={N}")
        assert np.abs(y64).max() < 0.05 and rel <= 1e-2


def test_two_streams_unsynchronised():
    """Split-K calls on two streams with no synchronisation between them each
    get their own workspace (keyed by device and stream), and a later call on
    the first stream still finds its workspace clear."""
    cases = [synthgen.w4a16_case(1, 4096, 4096, 128, seed=11), synthgen.w4a16_case(64, 4096, 4096, 128, seed=12),
             synthgen.w4a16_case(2, 11008, 4096, 128, seed=13)]
    devs = [to_dev(c.x, c.qweight, c.scales, c.qzeros) for c in cases]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            outs.append(("a", awq.gemv_w4a16(*devs[0], 128)))
        with torch.cuda.stream(s2):
            outs.append(("b", awq.gemm_w4a16(*devs[1], 128)))
            outs.append(("c", awq.gemv_w4a16(*devs[2], 128)))
    with torch.cuda.stream(s1):
        outs.append(("c", awq.gemv_w4a16(*devs[2], 128)))
    torch.cuda.synchronize()
    ref = {k: orc().w4a16(c.x, c.qweight, c.scales, c.qzeros, 128, nthreads=THREADS)
           for k, c in zip("abc", cases)}
    first = {}
    for k, y in outs:
        check_fp(y.cpu(), ref[k], "f16", f"stream case {k}")
        first.setdefault(k, y)
        assert torch.equal(y, first[k]), k


@pytest.mark.parametrize("M,K,N,G", [(1, 32, 8, 32), (5, 96, 24, 32), (17, 64, 136, 64), (33, 128, 264, 128),
                                     (100, 192, 72, 64), (129, 256, 1032, 128), (2, 4096, 8, 128),
                                     (300, 128, 40, 32)])
def test_ragged_and_small_shapes(M, K, N, G):
    c = synthgen.w4a16_case(M, K, N, G)
    yg, y64, _ = _run(c)
    check_fp(yg, y64, "f16", f"ragged gemm {M}x{K}x{N} g{G}")
    if M <= 8:
        yg, y64, _ = _run(c, "gemv")
        check_fp(yg, y64, "f16", f"ragged gemv {M}x{K}x{N} g{G}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("M", [2, 5, 8])
def test_gemv_plans_by_rows_and_dtype(M, G, dtype):
    """The decode kernel's plans between one and eight rows: 8-wave workgroups
    (M >= 4 where their grid fits one round; bf16 at M <= 2 with 32- and 64-k
    groups), one 128-k group per wave (bf16 at M <= 2), on 11008 x 4104 --
    long K, many splits, a ragged last column tile."""
    c = synthgen.w4a16_case(M, 11008, 4104, G, dtype=dtype)
    yg, y64, _ = _run(c, "gemv")
    check_fp(yg, y64, dtype, f"gemv plans M={M} G={G} {dtype}")


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M", [1, 5])
def test_gemv_one_group_per_wave(M, dtype, sym):
    """A layer whose decode grid would not stay resident at 64-k chunks
    (Llama-3-8B gate_up, N = 28672): each wave then covers one 128-k group."""
    c = synthgen.w4a16_case(M, 4096, 28672, 128, dtype=dtype, sym=sym)
    yg, y64, _ = _run(c, "gemv")
    check_fp(yg, y64, dtype, f"gemv 128-k chunks M={M} {dtype} sym={sym}")


@pytest.mark.parametrize("M", [65535, 65536])
def test_gemm_activation_bytes_at_2_31(M):
    """X of just under 2^31 bytes runs the LDS GEMM with copy offsets close to
    2^31; at exactly 2^31 bytes the planner hands the call to the tiled kernel.
    Checked on sampled rows, the last ones included."""
    K, N, G = 16384, 32, 128
    c = synthgen.w4a16_case(1, K, N, G)
    x = synthgen.activations_on(dev(), M, K, seed=synthgen.seed_for(f"x-2^31|{M}"))
    qw, s, qz = to_dev(c.qweight, c.scales, c.qzeros)
    y = awq.gemm_w4a16(x, qw, s, qz, G)
    torch.cuda.synchronize()
    rows = torch.tensor(sorted(set(sample_rows(M, seed=3).tolist()) | {M - 1, M - 2, 0}))
    xs = x[rows.to(x.device)].cpu()
    del x
    y64 = orc().w4a16(xs, c.qweight, c.scales, c.qzeros, G, F16, nthreads=THREADS)
    check_fp(y.cpu()[rows], y64, "f16", f"gemm M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,G,split", [(200, 1216, 256, 64, 0), (200, 1216, 256, 64, 3), (130, 1216, 384, 32, 0),
                                           (256, 1152, 4096, 128, 0), (513, 4096, 1032, 128, 0), (300, 640, 640, 64, 0),
                                           # 128-row tiles above M = 128, 65 stages, with and without K splits
                                           (300, 4160, 1032, 64, 0), (300, 4160, 1032, 64, 2)])
def test_gemm_few_tiles(M, K, N, G, split):
    """Layers with no more tiles than CUs: the workgroup's two wave groups
    split its K stages, odd stage counts included (19 stages over 4 splits:
    5 per workgroup, so one group idles through a barrier)."""
    c = synthgen.w4a16_case(M, K, N, G)
    yg, y64, _ = _run(c, split_k=split)
    check_fp(yg, y64, "f16", f"few-tile gemm {M}x{K}x{N} g{G} split={split}")


@pytest.mark.parametrize("split", [1, 2, 3, 7, 16, 128])
def test_explicit_split_k(split):
    c = synthgen.w4a16_case(4, 4096, 1024, 128)
    yg, y64, _ = _run(c, "gemv", split_k=split)
    check_fp(yg, y64, "f16", f"gemv split={split}")
    c = synthgen.w4a16_case(96, 4096, 512, 128)
    yg, y64, _ = _run(c, "gemm", split_k=split)
    check_fp(yg, y64, "f16", f"gemm split={split}")


def test_deterministic_and_workspace_reuse():
    """Same inputs give the same bits; the shared workspace's counters are left
    re-armed, so back-to-back split-K calls stay correct."""
    c = synthgen.w4a16_case(1, 4096, 4096, 128)
    x, qw, s, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
    outs = [awq.gemv_w4a16(x, qw, s, qz, 128) for _ in range(5)]
    c2 = synthgen.w4a16_case(3, 4096, 4096, 128)
    o2 = awq.gemv_w4a16(*to_dev(c2.x, c2.qweight, c2.scales, c2.qzeros), 128)
    outs.append(awq.gemv_w4a16(x, qw, s, qz, 128))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    check_fp(outs[0].cpu(), orc().w4a16(c.x, c.qweight, c.scales, c.qzeros, 128, nthreads=THREADS), "f16")
    check_fp(o2.cpu(), orc().w4a16(c2.x, c2.qweight, c2.scales, c2.qzeros, 128, nthreads=THREADS), "f16")


def test_shared_workspace_across_shapes():
    """Calls of different shapes and tile counts share one workspace in turn
    (few tiles / many splits, then many tiles / few splits): each must find
    its split-K counters zero and be correct (regression test for a counter
    region whose size depended on the call)."""
    seq = [("gemv", 4, 4096, 1024), ("gemm", 64, 4096, 512), ("gemv", 8, 4096, 22016),
           ("gemm", 1024, 4096, 4096), ("gemv", 1, 4096, 4096), ("gemm", 512, 4096, 14336),
           ("gemv", 2, 11008, 4096)]
    for entry, M, K, N in seq:
        c = synthgen.w4a16_case(M, K, N, 128)
        rows = None if M <= 64 else sample_rows(M, seed=1)
        yg, y64, _ = _run(c, entry, rows=rows)
        check_fp(yg, y64, "f16", f"{entry} M={M} K={K} N={N}")


def test_output_guard_band():
    """The kernels write exactly M*N outputs: a sentinel band after y survives."""
    for (M, K, N) in [(1, 4096, 4096), (7, 1024, 1032), (70, 512, 776)]:
        c = synthgen.w4a16_case(M, K, N, 128)
        x, qw, s, qz = to_dev(c.x, c.qweight, c.scales, c.qzeros)
        buf = torch.full((M * N + 4096,), float("nan"), dtype=torch.float16, device=dev())
        y = buf[:M * N].view(M, N)
        (awq.gemv_w4a16 if M <= 8 else awq.gemm_w4a16)(x, qw, s, qz, 128, out=y)
        torch.cuda.synchronize()
        assert torch.isnan(buf[M * N:]).all()
        check_fp(y.cpu(), orc().w4a16(c.x, c.qweight, c.scales, c.qzeros, 128, nthreads=THREADS), "f16")


def test_linear_dispatch_rule():
    """More than 8 rows goes to the GEMM entry, up to 8 to the GEMV entry."""
    c = synthgen.w4a16_case(9, 512, 256, 128)
    y = awq.linear_w4a16(*to_dev(c.x, c.qweight, c.scales, c.qzeros), 128)
    torch.cuda.synchronize()
    check_fp(y.cpu(), orc().w4a16(c.x, c.qweight, c.scales, c.qzeros, 128), "f16")
    with pytest.raises(awq.AWQError):
        awq.gemv_w4a16(*to_dev(c.x, c.qweight, c.scales, c.qzeros), 128)
