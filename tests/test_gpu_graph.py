"""The ops under HIP graph capture: several replays, with eager work and
synchronisations between them, each bit-identical to the eager result.  The
library enqueues no memsets (split-K accumulators and partial tiles are
cleared by the kernel that sums them), so a captured graph can be replayed
any number of times."""
import pytest
import torch

import bit_weight_only_awq_amd as awq
import synthgen
from gpu_helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    d = dev()
    dec = synthgen.w4a16_case(1, 4096, 4096, 128)        # decode kernel, split-K
    mid = synthgen.w4a16_case(96, 4096, 512, 128)        # LDS GEMM, split-K summed by a second kernel
    big = synthgen.w4a16_case(256, 1024, 2048, 64)       # tiled kernel, no split
    w8 = synthgen.w4a8_case(1, 21760, 8192, -1)          # quant + W4A8 split-K
    w8g = synthgen.w4a8_case(64, 4096, 1024, 128)        # W4A8 LDS GEMM, per-group, split-K (second kernel)
    w8f = synthgen.w4a8_case(128, 4096, 4096, -1)        # INT4-FP8 LDS GEMM, split-K (second kernel)
    a = [to_dev(c.x, c.qweight, c.scales, c.qzeros) for c in (dec, mid, big)]
    x8, b8, s28 = to_dev(w8.x, w8.b, w8.s2)
    xg, bg, s2g, s3g = to_dev(w8g.x, w8g.b, w8g.s2, w8g.s3)
    outs = [torch.empty(c.M, c.N, dtype=torch.float16, device=d) for c in (dec, mid, big)]
    a8 = torch.empty(1, 21760, dtype=torch.int8, device=d)
    s1 = torch.empty(1, dtype=torch.float32, device=d)
    y8 = torch.empty(1, 8192, dtype=torch.float16, device=d)
    a8g = torch.empty(64, 4096, dtype=torch.int8, device=d)
    s1g = torch.empty(64, dtype=torch.float32, device=d)
    y8g = torch.empty(64, 1024, dtype=torch.float16, device=d)
    xf, bf, s2f = to_dev(w8f.x, w8f.b, w8f.s2)
    fa, fs1, fas = awq.quant_act_fp8(xf)
    yf = torch.empty(128, 4096, dtype=torch.float16, device=d)

    def work():
        awq.gemv_w4a16(*a[0], 128, out=outs[0])
        awq.gemm_w4a16(*a[1], 128, out=outs[1])
        awq.gemm_w4a16(*a[2], 64, out=outs[2])
        awq.quant_act(x8, a8, s1)
        awq.w4a8_gemm(a8, b8, s1, s28, out=y8)
        awq.quant_act(xg, a8g, s1g)
        awq.w4a8_gemm(a8g, bg, s1g, s2g, s3g, 128, out=y8g)
        awq.w4a8_fp8_gemm(fa, bf, fs1, fas, s2f, out=yf)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (*outs, y8, y8g, a8, s1, yf)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(d)
    with torch.cuda.graph(g, stream=s):
        work()
    for rep in range(4):
        for t in (*outs, y8, y8g, yf):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = [*outs, y8, y8g, a8, s1, yf]
        for i, (r, t) in enumerate(zip(ref, got)):
            assert torch.equal(r, t), (rep, i)
        # eager work between replays, on the same workspace
        other = synthgen.w4a16_case(3, 2048, 1024, 128)
        awq.gemv_w4a16(*to_dev(other.x, other.qweight, other.scales, other.qzeros), 128)
        torch.cuda.synchronize()
