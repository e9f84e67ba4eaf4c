"""The C ABI without a GPU: the library loads, exports every function that
include/awq4.h declares, and argument validation returns the documented status
codes before anything is enqueued (so these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

from bit_weight_only_awq_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ("awq_pack", "awq_unpack", "awq_gemm_w4a16", "awq_gemv_w4a16", "w4a8_quant_act", "w4a8_gemm",
              "w4a8_linear", "awq_workspace_bytes", "awq_status_str", "awq_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    lib = L.lib()
    for code in (L.AWQ_OK, L.AWQ_EINVAL, L.AWQ_EUNSUPPORTED, L.AWQ_EWORKSPACE, L.AWQ_EALIGN, L.AWQ_EHIP):
        s = lib.awq_status_str(code).decode()
        assert s.startswith("AWQ_")
    assert lib.awq_status_str(12345).decode() == "AWQ_UNKNOWN"
    assert lib.awq_version() == 102


# Fake "device" pointers: validation only looks at null-ness and alignment, and
# every call below is rejected before any launch.
A = 0x10000
MIS = 0x10002


def _w4a16(fn, x=A, qw=A, s=A, qz=A, y=A, M=1, N=4096, K=4096, G=128, dt=0, split=0, ws=None, wsb=0):
    return getattr(L.lib(), fn)(x, qw, s, qz, y, M, N, K, G, dt, split, ws, wsb, None)


def test_split_gemm_needs_workspace():
    """A K-split GEMM is refused without its workspace (before any launch)."""
    assert _w4a16("awq_gemm_w4a16", M=64, N=4096, K=4096) == L.AWQ_EWORKSPACE
    assert _w4a16("awq_gemm_w4a16", M=64, N=4096, K=4096, ws=A, wsb=1 << 10) == L.AWQ_EWORKSPACE


@pytest.mark.parametrize("fn", ["awq_gemm_w4a16", "awq_gemv_w4a16"])
def test_w4a16_validation(fn):
    E = L
    assert _w4a16(fn, x=None) == E.AWQ_EINVAL
    assert _w4a16(fn, qw=None) == E.AWQ_EINVAL
    assert _w4a16(fn, s=None) == E.AWQ_EINVAL
    assert _w4a16(fn, y=None) == E.AWQ_EINVAL
    assert _w4a16(fn, M=0) == E.AWQ_EINVAL
    assert _w4a16(fn, N=12) == E.AWQ_EINVAL          # N % 8
    assert _w4a16(fn, G=16) == E.AWQ_EINVAL          # unsupported group
    assert _w4a16(fn, G=256) == E.AWQ_EINVAL
    assert _w4a16(fn, K=4000) == E.AWQ_EINVAL        # K % G
    assert _w4a16(fn, dt=2) == E.AWQ_EINVAL
    assert _w4a16(fn, split=-1) == E.AWQ_EINVAL
    assert _w4a16(fn, split=129) == E.AWQ_EINVAL     # > K/32
    assert _w4a16(fn, K=16384, split=256) == E.AWQ_EINVAL  # > 255 splits
    assert _w4a16(fn, x=MIS) == E.AWQ_EALIGN
    assert _w4a16(fn, qz=MIS) == E.AWQ_EALIGN
    # a valid split-K request without workspace
    assert _w4a16(fn, M=1, split=8) == E.AWQ_EWORKSPACE
    assert _w4a16(fn, M=1, split=8, ws=A, wsb=16) == E.AWQ_EWORKSPACE


def test_gemv_rejects_more_than_8_rows():
    assert _w4a16("awq_gemv_w4a16", M=9) == L.AWQ_EUNSUPPORTED


def test_workspace_bytes():
    lib = L.lib()
    op_gemm, op_gemv, op8 = L.AWQ_OP_GEMM_W4A16, L.AWQ_OP_GEMV_W4A16, L.AWQ_OP_W4A8_GEMM
    # no split requested -> no workspace
    assert lib.awq_workspace_bytes(op_gemm, 2048, 4096, 4096, 128, 1) == 0
    # a M=1, N=4096 GEMV (32 K splits of 128 k, 16 column tiles): the larger of
    # one 64-bit counting accumulator per output element (fp16) and 16 tile
    # counters (256 bytes) + 32 fp32 partial rows (bf16)
    assert lib.awq_workspace_bytes(op_gemv, 1, 4096, 4096, 128, 8) == max(4096 * 8, 256 + 32 * 4096 * 4)
    # the tiled kernel with an explicit split: per-tile counters (16 tiles of
    # 64 rows x 256 columns, padded to 256 bytes), then 4 fp32 partial results
    assert lib.awq_workspace_bytes(op_gemm, 64, 4096, 4096, 128, 4) == 256 + 4 * 64 * 4096 * 4
    # the LDS GEMM with an explicit split: 8 x 32 tiles of 256 rows x 128
    # columns
    assert lib.awq_workspace_bytes(op_gemm, 2048, 4096, 4096, 128, 2) == 1024 + 2 * 2048 * 4096 * 4
    assert lib.awq_workspace_bytes(op8, 1, 8192, 21760, -1, 0) == 8192 * 8
    # one workgroup per tile without a K split: no workspace
    assert lib.awq_workspace_bytes(op_gemm, 2048, 6144, 4096, 128, 0) == 0
    # automatic split for decode needs a workspace
    assert lib.awq_workspace_bytes(op_gemv, 1, 4096, 4096, 128, 0) > 0
    # invalid shapes -> 0
    assert lib.awq_workspace_bytes(op_gemv, 9, 4096, 4096, 128, 0) == 0
    assert lib.awq_workspace_bytes(op_gemm, 1, 4095, 4096, 128, 0) == 0
    assert lib.awq_workspace_bytes(op8, 1, 8192, 21760, -1, 0) > 0
    assert lib.awq_workspace_bytes(op8, 1, 8192, 21700, -1, 0) == 0
    assert lib.awq_workspace_bytes(op8, 1, 64, 131072, -1, 0) == 0
    assert lib.awq_workspace_bytes(op8, 1, 64, 131008, -1, 0) > 0
    assert lib.awq_workspace_bytes(99, 1, 8192, 4096, 128, 0) == 0


def test_w4a8_validation():
    lib = L.lib()

    def g(a8=A, b=A, s1=A, s2=A, s3=None, y=A, acc=None, M=1, N=8192, K=21760, G=-1, dt=0, ws=None, wsb=0):
        return lib.w4a8_gemm(a8, b, s1, s2, s3, y, acc, M, N, K, G, dt, ws, wsb, None)

    assert g(a8=None) == L.AWQ_EINVAL
    assert g(s2=None) == L.AWQ_EINVAL
    assert g(N=12) == L.AWQ_EINVAL
    assert g(G=128) == L.AWQ_EINVAL            # grouped without s3
    assert g(s3=A) == L.AWQ_EINVAL             # per-channel with s3
    assert g(s3=A, G=48) == L.AWQ_EINVAL
    assert g(K=21700) == L.AWQ_EUNSUPPORTED    # K % 64
    assert g(K=262144) == L.AWQ_EUNSUPPORTED   # int32 accumulator bound
    assert g(K=131072) == L.AWQ_EUNSUPPORTED   # 2^14 * K would reach 2^31 exactly
    assert g(K=131008) == L.AWQ_EWORKSPACE     # the largest K: accepted (then needs its workspace)
    assert g(acc=MIS) == L.AWQ_EALIGN
    assert g() == L.AWQ_EWORKSPACE             # decode split needs a workspace
    assert g(dt=1) == L.AWQ_EWORKSPACE         # bf16 scales and output: same rules
    assert g(dt=2) == L.AWQ_EINVAL             # unknown dtype
    assert lib.w4a8_quant_act(None, A, A, 1, 16, 0, None) == L.AWQ_EINVAL
    assert lib.w4a8_quant_act(A, A, A, 0, 16, 0, None) == L.AWQ_EINVAL
    assert lib.w4a8_quant_act(A, A, A, 1, 16, 2, None) == L.AWQ_EINVAL
    assert lib.w4a8_quant_act(MIS, A, A, 1, 16, 0, None) == L.AWQ_EALIGN
    assert lib.w4a8_quant_act(MIS, A, A, 1, 16, 1, None) == L.AWQ_EALIGN


def test_w4a8_linear_validation():
    lib = L.lib()

    def f(x=A, a8=A, s1=A, b=A, s2=A, s3=None, y=A, acc=None, M=1, N=8192, K=21760, G=-1, dt=0, ws=None, wsb=0):
        return lib.w4a8_linear(x, a8, s1, b, s2, s3, y, acc, M, N, K, G, dt, ws, wsb, None)

    assert f(x=None) == L.AWQ_EINVAL
    assert f(a8=None) == L.AWQ_EINVAL          # scratch for the two-step path is required
    assert f(s1=None) == L.AWQ_EINVAL
    assert f(M=0) == L.AWQ_EINVAL
    assert f(N=12) == L.AWQ_EINVAL
    assert f(G=128) == L.AWQ_EINVAL            # grouped without s3
    assert f(s3=A, G=48) == L.AWQ_EINVAL
    assert f(K=21700) == L.AWQ_EUNSUPPORTED    # K % 64
    assert f(K=131072) == L.AWQ_EUNSUPPORTED   # int32 accumulator bound
    assert f(K=131008) == L.AWQ_EWORKSPACE
    assert f(x=MIS) == L.AWQ_EALIGN
    assert f(s1=MIS) == L.AWQ_EALIGN
    assert f() == L.AWQ_EWORKSPACE             # the decode split needs a workspace
    assert f(dt=1) == L.AWQ_EWORKSPACE
    assert f(dt=-1) == L.AWQ_EINVAL            # unknown dtype


def test_pack_validation():
    lib = L.lib()
    assert lib.awq_pack(A, A, 4, 12, L.AWQ_LAYOUT_N8, None, None) == L.AWQ_EINVAL
    assert lib.awq_pack(A, A, 12, 8, L.W4A8_LAYOUT_K8, None, None) == L.AWQ_EINVAL
    assert lib.awq_pack(A, A, 8, 8, 7, None, None) == L.AWQ_EINVAL
    assert lib.awq_pack(None, A, 8, 8, L.AWQ_LAYOUT_N8, None, None) == L.AWQ_EINVAL
    assert lib.awq_pack(MIS, A, 8, 8, L.AWQ_LAYOUT_N8, None, None) == L.AWQ_EALIGN
    assert lib.awq_pack(None, None, 0, 8, L.AWQ_LAYOUT_N8, None, None) == L.AWQ_OK  # empty: no-op
    assert lib.awq_unpack(A, A, 8, -8, L.AWQ_LAYOUT_N8, None) == L.AWQ_EINVAL
    assert lib.awq_unpack(None, None, 8, 0, L.W4A8_LAYOUT_K8, None) == L.AWQ_OK


def test_stream_read_validation():
    lib = L.lib()
    assert lib.awq_stream_read(None, 16, A, None) == L.AWQ_EINVAL
    assert lib.awq_stream_read(A, 0, A, None) == L.AWQ_EINVAL
    assert lib.awq_stream_read(A, 24, A, None) == L.AWQ_EINVAL
    assert lib.awq_stream_read(A, 16, None, None) == L.AWQ_EINVAL
    assert lib.awq_stream_read(MIS, 16, A, None) == L.AWQ_EALIGN


def _plan(op, M, N, K, G=128, split=0, cus=256):
    info = L.PlanInfo()
    rc = L.lib().awq_plan_info(op, M, N, K, G, split, cus, ctypes.byref(info))
    assert rc == L.AWQ_OK, rc
    return info


def test_plan_info_validation():
    lib = L.lib()
    info = L.PlanInfo()
    assert lib.awq_plan_info(L.AWQ_OP_GEMM_W4A16, 1, 4096, 4096, 128, 0, 256, None) == L.AWQ_EINVAL
    assert lib.awq_plan_info(L.AWQ_OP_GEMM_W4A16, 1, 4096, 4096, 128, 0, -1, ctypes.byref(info)) == L.AWQ_EINVAL
    assert lib.awq_plan_info(L.AWQ_OP_GEMV_W4A16, 9, 4096, 4096, 128, 0, 256, ctypes.byref(info)) == \
        L.AWQ_EUNSUPPORTED
    assert lib.awq_plan_info(L.AWQ_OP_W4A8_GEMM, 1, 4096, 21700, -1, 0, 256, ctypes.byref(info)) == \
        L.AWQ_EUNSUPPORTED
    assert lib.awq_plan_info(99, 1, 4096, 4096, 128, 0, 256, ctypes.byref(info)) == L.AWQ_EINVAL


def test_plan_matches_workspace_query():
    """awq_workspace_bytes (no device here: a whole MI355X) agrees with the plan at 256 CUs."""
    lib = L.lib()
    for op, M, N, K, G in ((L.AWQ_OP_GEMV_W4A16, 1, 4096, 4096, 128), (L.AWQ_OP_GEMM_W4A16, 64, 4096, 4096, 128),
                           (L.AWQ_OP_GEMM_W4A16, 2048, 4096, 14336, 128), (L.AWQ_OP_W4A8_GEMM, 1, 8192, 21760, -1),
                           (L.AWQ_OP_W4A8_GEMM, 256, 8192, 21760, 128)):
        assert _plan(op, M, N, K, G).workspace_bytes == lib.awq_workspace_bytes(op, M, N, K, G, 0)


def test_plan_sizes_grids_from_the_cu_count():
    """The planners size their grids from the device's compute units: a whole
    MI355X (256 CUs) and a quarter of one (64 CUs) get different plans, each
    filling its own device."""
    gemm, gemv, w8 = L.AWQ_OP_GEMM_W4A16, L.AWQ_OP_GEMV_W4A16, L.AWQ_OP_W4A8_GEMM
    # M = 1024 on 4096 x 4096: 128 tiles of 256 x 128 would leave half of 256
    # CUs idle, so 128-row tiles (256 of them, K split inside the workgroup);
    # on 64 CUs 256 x 256 tiles already give every CU one (64 of them)
    big, small = _plan(gemm, 1024, 4096, 4096, cus=256), _plan(gemm, 1024, 4096, 4096, cus=64)
    assert (big.kernel, small.kernel) == (3, 3)
    assert big.cu_count == 256 and small.cu_count == 64
    assert big.row_tiles == 8 and big.tile_cols == 128 and big.tiles_n * big.tiles_m == 256 and big.ksplit == 2
    assert small.row_tiles == 16 and small.tile_cols == 256 and small.tiles_n * small.tiles_m == 64
    assert small.ksplit == 1
    # M = 2048: 256 tiles of 256 x 128, one per CU on 256 CUs (two wave groups
    # split K inside each); on 64 CUs two tiles of 256 x 256 per CU
    big, small = _plan(gemm, 2048, 4096, 4096, cus=256), _plan(gemm, 2048, 4096, 4096, cus=64)
    assert big.row_tiles == 16 and big.ksplit == 2 and big.tile_cols == 128
    assert small.row_tiles == 16 and small.ksplit == 1 and small.tile_cols == 256
    # 256 x 256 tiles wherever more than half the CUs get one: (4096, 14336)
    # at M = 2048 has 448 of them; an explicit K split keeps 128 columns
    wide = _plan(gemm, 2048, 14336, 4096, cus=256)
    assert (wide.tile_cols, wide.tiles_n, wide.tiles_m, wide.splits, wide.ksplit) == (256, 56, 8, 1, 1)
    assert _plan(gemm, 2048, 14336, 4096, split=2).tile_cols == 128
    assert _plan(gemm, 4, 4096, 4096, cus=256).tile_cols == 0
    # decode GEMV at M = 1 on 4096 x 4096: 32-k chunks while they give at most
    # two workgroups per CU -- on 64 CUs the grid stays at 64-k chunks
    big, small = _plan(gemv, 1, 4096, 4096, cus=256), _plan(gemv, 1, 4096, 4096, cus=64)
    assert big.kernel == 0 and small.kernel == 0
    assert big.splits == 32 and small.splits == 16
    # W4A8 at M = 2048 on (4096, 4096): 256 tiles of 128 x 256, K split inside
    # the workgroup only when there are no more of them than CUs
    big, small = _plan(w8, 2048, 4096, 4096, -1, cus=256), _plan(w8, 2048, 4096, 4096, -1, cus=64)
    assert big.kernel == 2 and small.kernel == 2
    assert big.tiles_n * big.tiles_m == 256 and big.ksplit == 2
    assert small.tiles_n * small.tiles_m == 256 and small.ksplit == 1
    # every plan is valid at any CU count
    for cus in (8, 32, 64, 80, 128, 256, 304):
        for op, M, N, K, G in ((gemv, 1, 4096, 11008, 128), (gemv, 8, 22016, 4096, 64), (gemm, 16, 3072, 768, 128),
                               (gemm, 64, 6144, 4096, 128), (gemm, 4096, 28672, 4096, 128),
                               (gemm, 300, 136, 4096, 32), (w8, 1, 8192, 21760, -1), (w8, 64, 8192, 21760, 128),
                               (w8, 1024, 8192, 21760, -1)):
            p = _plan(op, M, N, K, G, cus=cus)
            assert 1 <= p.splits <= 255 and p.tiles_n >= 1 and p.tiles_m >= 1 and p.ksplit in (1, 2)
            assert (p.splits > 1) == (p.workspace_bytes > 0), (cus, op, M, N, K)


def test_gemm_k_split_rule():
    """The LDS GEMM's K split on a whole MI355X: about CUs / tiles splits of
    two-group workgroups, at most one per 16 stages and 8 in all; long K
    (>= 128 stages) on 128-row tiles with one tile per CU at most takes 3-4
    single-group splits; 256-row tiles at M = 2048 take none."""
    gemm = L.AWQ_OP_GEMM_W4A16
    want = {  # (M, N, K): (row tiles, tiles, splits, wave groups)
        (256, 6144, 4096): (8, 96, 2, 2),     # qkv: 96 tiles -> 2 splits
        (256, 4096, 4096): (8, 64, 4, 2),     # o: 64 tiles -> 4
        (256, 4096, 14336): (8, 64, 4, 2),    # down
        (96, 4096, 14336): (8, 32, 8, 2),     # down at 96 rows: 8, the cap
        (96, 6144, 4096): (8, 48, 4, 2),      # qkv at 96 rows: 5 capped at 64 / 16 stages
        (256, 28672, 4096): (16, 224, 1, 2),  # gate/up: more tiles than half the CUs, no split
        (768, 4096, 14336): (8, 192, 4, 1),   # long K, 192 tiles: 4 single-group splits
        (384, 4096, 14336): (8, 96, 8, 1),    # long K, 2 two-group splits would idle 64 CUs: 8 single-group
        (1024, 4096, 14336): (8, 256, 3, 1),  # long K, 256 tiles: 3
        (2048, 4096, 14336): (16, 256, 1, 2),  # 256-row tiles: none
    }
    for (M, N, K), (mt, tiles, s, ks) in want.items():
        p = _plan(gemm, M, N, K, 128, cus=256)
        assert (p.kernel, p.row_tiles, p.tiles_n * p.tiles_m, p.splits, p.ksplit) == (3, mt, tiles, s, ks), (M, N, K)
        assert p.workspace_bytes == (0 if s == 1 else L.lib().awq_workspace_bytes(gemm, M, N, K, 128, 0))


def test_gemm_wide_tile_rule():
    """256-column tiles for the LDS GEMM where they still give more than half
    the CUs a tile, without K splits or wave groups, unless the 128-column
    tiles spread over the CUs at least 1.25x more evenly."""
    gemm = L.AWQ_OP_GEMM_W4A16
    want = {  # (M, N, K): (tile columns, tiles, wave groups)
        (2048, 6144, 4096): (256, 192, 1),    # qkv: 192 wide tiles (0.75) against 384 (0.75)
        (4096, 6144, 4096): (128, 768, 1),    # qkv: 384 wide tiles (0.75) against 768 (1.0)
        (2048, 28672, 4096): (256, 896, 1),   # gate/up: 0.875 against 1.0, under 1.25x
        (4096, 28672, 4096): (256, 1792, 1),  # gate/up: even either way
        (4096, 4096, 4096): (256, 256, 1),    # o: one wide tile per CU
        (2048, 14336, 4096): (256, 448, 1),   # the (4096, 14336) target
        (2048, 4096, 4096): (128, 256, 2),    # o: 128 wide tiles would idle half the CUs
    }
    for (M, N, K), (cols, tiles, ks) in want.items():
        p = _plan(gemm, M, N, K, 128, cus=256)
        assert (p.kernel, p.row_tiles, p.splits) == (3, 16, 1), (M, N, K)
        assert (p.tile_cols, p.tiles_n * p.tiles_m, p.ksplit) == (cols, tiles, ks), (M, N, K)


def test_split_caps_of_the_atomic_kernels():
    """Kernels that reduce K splits through per-element counting atomics cap
    their splits as M grows: the skinny W4A8 kernels (int8 and INT4-FP8) at
    2^20 sqrt(K / 4096) / (M N), the decode GEMV with 8-wave workgroups at
    M >= 4 where that grid still runs in one round (half the splits)."""
    for op in (L.AWQ_OP_W4A8_GEMM, L.AWQ_OP_W4A8_FP8_GEMM):
        want = {  # (M, N, K): splits on a whole MI355X
            (1, 14336, 4096): 5, (32, 14336, 4096): 2, (48, 14336, 4096): 1, (64, 14336, 4096): 1,
            (32, 4096, 4096): 8, (16, 8192, 21760): 8, (32, 8192, 21760): 4,
        }
        for (M, N, K), s in want.items():
            p = _plan(op, M, N, K, -1, cus=256)
            assert (p.kernel, p.splits) == (0, s), (op, M, N, K, p.splits)
            assert p.workspace_bytes == (0 if s == 1 else M * N * 8)
        # from 33 rows the LDS GEMM wherever the skinny kernel would split K
        for M, N, K in ((48, 4096, 4096), (64, 4096, 4096), (64, 8192, 21760), (33, 4096, 14336)):
            assert _plan(op, M, N, K, -1, cus=256).kernel == 2, (op, M, N, K)
    gemv = L.AWQ_OP_GEMV_W4A16
    # Llama-2-7B qkv (4096 x 12288): 48 column tiles; 16 splits of 4 waves at
    # M = 1, 4 splits of 8 waves (128-k chunks) at M = 8; gate/up (4096 x
    # 22016) keeps 4 waves at M = 8 (8 waves would take two rounds)
    assert (_plan(gemv, 1, 12288, 4096, 128, cus=256).splits, _plan(gemv, 8, 12288, 4096, 128, cus=256).splits) == (16, 4)
    assert _plan(gemv, 8, 4096, 4096, 128, cus=256).splits == 8
    assert _plan(gemv, 8, 22016, 4096, 128, cus=256).splits == 8


def test_dequant_validation():
    lib = L.lib()
    assert lib.awq_dequant_w4a16(A, A, A, None, 4096, 4096, 128, 0, None) == L.AWQ_EINVAL   # no output
    assert lib.awq_dequant_w4a16(None, A, A, A, 4096, 4096, 128, 0, None) == L.AWQ_EINVAL
    assert lib.awq_dequant_w4a16(A, A, A, A, 4092, 4096, 128, 0, None) == L.AWQ_EINVAL      # N % 8
    assert lib.awq_dequant_w4a16(A, A, A, A, 4096, 4000, 128, 0, None) == L.AWQ_EINVAL      # K % G
    assert lib.awq_dequant_w4a16(A, A, A, A, 4096, 4096, 128, 5, None) == L.AWQ_EINVAL      # dtype
    assert lib.awq_dequant_w4a16(A, A, A, MIS, 4096, 4096, 128, 0, None) == L.AWQ_EALIGN


def test_fp8_validation():
    lib = L.lib()

    def g(a=A, b=A, s1=A, asum=A, s2=A, y=A, acc=None, M=1, N=8192, K=21760, dt=0, ws=None, wsb=0):
        return lib.w4a8_fp8_gemm(a, b, s1, asum, s2, y, acc, M, N, K, dt, ws, wsb, None)

    assert g(a=None) == L.AWQ_EINVAL
    assert g(asum=None) == L.AWQ_EINVAL
    assert g(N=12) == L.AWQ_EINVAL
    assert g(K=21760 + 64) == L.AWQ_EUNSUPPORTED   # K % 128
    assert g(K=131072) == L.AWQ_EUNSUPPORTED
    assert g(dt=2) == L.AWQ_EINVAL
    assert g(acc=MIS) == L.AWQ_EALIGN
    assert g() == L.AWQ_EWORKSPACE                  # split-K needs its workspace
    assert lib.awq_workspace_bytes(L.AWQ_OP_W4A8_FP8_GEMM, 1, 8192, 21760, -1, 0) == 8192 * 8
    assert lib.awq_workspace_bytes(L.AWQ_OP_W4A8_FP8_GEMM, 1, 8192, 21824, -1, 0) == 0
    # the kernels by M: skinny up to 64 rows (up to 32 where it would split
    # K), the LDS-pipelined GEMM (128 x 256 tiles) above, split only with
    # fewer tiles than CUs
    fp8 = L.AWQ_OP_W4A8_FP8_GEMM
    assert [_plan(fp8, M, 8192, 21760, -1).kernel for M in (32, 64, 65, 100, 128, 1024)] == [0, 2, 2, 2, 2, 2]
    # the register-tiled kernel only past the LDS GEMM's 32-bit offsets
    assert _plan(fp8, 16401, 64, 130944, -1).kernel == 1
    assert _plan(L.AWQ_OP_W4A8_GEMM, 16400, 64, 131008, -1).kernel == 1
    assert _plan(L.AWQ_OP_W4A8_GEMM, 100, 8192, 21760, -1).kernel == 2
    p = _plan(fp8, 1024, 8192, 21760, -1)
    assert (p.tiles_n, p.tiles_m, p.splits, p.workspace_bytes) == (32, 8, 1, 0)
    p = _plan(fp8, 256, 8192, 21760, -1)
    assert p.tiles_n * p.tiles_m == 64 and p.splits == 4
    # K splits: those that fit in one round, at most K / 1024, K / (4 M) and 8
    want = {(128, 4096, 4096): 4, (512, 4096, 4096): 2, (1024, 4096, 4096): 1, (128, 4096, 14336): 8,
            (384, 4096, 14336): 5, (128, 8192, 21760): 8, (768, 8192, 21760): 1, (256, 14336, 4096): 2}
    for (M, N, K), s in want.items():
        assert _plan(fp8, M, N, K, -1).splits == s, (M, N, K)
    assert p.workspace_bytes == lib.awq_workspace_bytes(fp8, 256, 8192, 21760, -1, 0) > 256 * 8192 * 4 * 4
    assert lib.w4a8_fp8_quant_act(None, A, A, A, 1, 16, 0, None) == L.AWQ_EINVAL
    assert lib.w4a8_fp8_quant_act(A, A, A, None, 1, 16, 0, None) == L.AWQ_EINVAL
    assert lib.w4a8_fp8_quant_act(A, A, A, A, 1, 16, 3, None) == L.AWQ_EINVAL
    assert lib.w4a8_fp8_quant_act(A, A, MIS, A, 1, 16, 0, None) == L.AWQ_EALIGN


def test_repack_v2_validation():
    lib = L.lib()
    assert lib.awq_repack_v2(None, A, A, A, 4096, 4096, 128, None) == L.AWQ_EINVAL
    assert lib.awq_repack_v2(A, A, A, None, 4096, 4096, 128, None) == L.AWQ_EINVAL  # zeros given, no output
    assert lib.awq_repack_v2(A, None, A, None, 4092, 4096, 128, None) == L.AWQ_EINVAL  # N % 8
    assert lib.awq_repack_v2(A, None, A, None, 4096, 4000, 128, None) == L.AWQ_EINVAL  # K % G
    assert lib.awq_repack_v2(A, None, A, None, 4096, 4096, 48, None) == L.AWQ_EINVAL
    assert lib.awq_repack_v2(MIS, None, A, None, 4096, 4096, 128, None) == L.AWQ_EALIGN
    # the newer layout takes any row length
    assert lib.awq_pack(None, None, 0, 43, L.AWQ_LAYOUT_V2, None, None) == L.AWQ_OK
    assert lib.awq_pack(MIS, A, 4, 43, L.AWQ_LAYOUT_V2, None, None) == L.AWQ_EALIGN
