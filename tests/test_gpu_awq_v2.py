"""The newer AWQ packing (identity order map, zero points packed per output
channel along the groups with the unused nibbles skipped): GPU pack / unpack
and the repack into the first-generation format bit-exact against the
oracle, and the GEMV / GEMM on repacked weights against the oracle's W4A16
computed straight from the newer packing."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import THREADS, check_fp, dev, orc, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(5, 43), (4096, 32), (8, 86), (1, 8), (3, 1), (0, 16), (11008, 17)])
def test_pack_v2_matches_oracle(rows, cols):
    g = torch.Generator().manual_seed(rows * 3 + cols)
    vals = torch.randint(0, 16, (rows, cols), generator=g, dtype=torch.uint8)
    if rows:
        vals[0, 0] = 200  # clamped and counted
    exp, bad = orc().pack_v2(vals.numpy())
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    got = awq.pack(vals.to(dev()), "v2", clamp_count=cnt)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)
    assert int(cnt.item()) == bad == (1 if rows else 0)
    back = awq.unpack(got, "v2", cols=cols)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), orc().unpack_v2(exp, cols))


def _v2_case(K, N, G, sym, seed):
    g = torch.Generator().manual_seed(seed)
    qw2 = torch.randint(-(2 ** 31), 2 ** 31, (K, N // 8), generator=g, dtype=torch.int64).to(torch.int32)
    groups = K // G
    zw = (groups + 7) // 8
    qz2 = None
    if not sym:
        # random words: the nibbles past the last group hold junk that must be ignored
        qz2 = torch.randint(-(2 ** 31), 2 ** 31, (N, zw), generator=g, dtype=torch.int64).to(torch.int32)
    return qw2, qz2


@pytest.mark.parametrize("K,N,G,sym", [(4096, 4096, 128, False), (11008, 4096, 128, False), (4096, 1032, 32, False),
                                       (640, 136, 64, True), (96, 8, 32, False)])
def test_repack_v2_bit_exact(K, N, G, sym):
    qw2, qz2 = _v2_case(K, N, G, sym, K + N)
    qw, qz = awq.repack_v2(*to_dev(qw2, qz2), G)
    torch.cuda.synchronize()
    exp_qw, _ = orc().pack_n8(orc().unpack_v2(qw2.numpy(), N))
    assert np.array_equal(qw.cpu().numpy(), exp_qw)
    if not sym:
        z = orc().unpack_v2(qz2.numpy(), K // G)  # [N, groups]
        exp_qz, _ = orc().pack_n8(np.ascontiguousarray(z.T))
        assert np.array_equal(qz.cpu().numpy(), exp_qz)
    else:
        assert qz is None


@pytest.mark.parametrize("M,K,N,G,sym", [(1, 4096, 4096, 128, False), (8, 11008, 4096, 128, False),
                                         (1, 4096, 14336, 32, True), (64, 4096, 1032, 64, False),
                                         (300, 4096, 4096, 128, False), (2048, 4096, 4096, 128, False)])
def test_gemm_on_repacked_weights(M, K, N, G, sym):
    qw2, qz2 = _v2_case(K, N, G, sym, M + K + N)
    c = synthgen.w4a16_case(M, K, N, G, sym=True)  # activations and scales only
    qw, qz = awq.repack_v2(*to_dev(qw2, qz2), G)
    x, s = to_dev(c.x, c.scales)
    y = awq.linear_w4a16(x, qw, s, qz, G)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 64 else sample_rows(M, seed=M)
    y64 = orc().w4a16_v2(c.x[torch.as_tensor(rows)], qw2, c.scales, qz2, G)
    check_fp(y.cpu()[torch.as_tensor(rows)], y64, "f16", f"v2 M={M} K={K} N={N} G={G} sym={sym}")
