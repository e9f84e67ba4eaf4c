"""GPU pack / unpack vs the oracle: bit-exact (both layouts)."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
from gpu_helpers import dev, orc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(768, 3072), (4096, 4096), (7, 8), (1, 136), (0, 64)])
def test_pack_n8_matches_oracle(rows, cols):
    g = torch.Generator().manual_seed(rows * 7 + cols)
    vals = torch.randint(0, 16, (rows, cols), generator=g, dtype=torch.uint8)
    exp, bad = orc().pack_n8(vals.numpy())
    assert bad == 0
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    got = awq.pack(vals.to(dev()), "n8", clamp_count=cnt)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)
    assert int(cnt.item()) == 0
    back = awq.unpack(got, "n8")
    assert torch.equal(back.cpu(), vals)


@pytest.mark.parametrize("rows,cols", [(21760, 64), (4096, 8192), (8, 8), (64, 24)])
def test_pack_k8_matches_oracle(rows, cols):
    g = torch.Generator().manual_seed(rows + cols)
    vals = torch.randint(-8, 8, (rows, cols), generator=g, dtype=torch.int8)
    exp, bad = orc().pack_k8(vals.numpy())
    assert bad == 0
    got = awq.pack(vals.to(dev()), "k8")
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)
    assert torch.equal(awq.unpack(got, "k8").cpu(), vals)


def test_unpack_random_words_matches_oracle():
    g = torch.Generator().manual_seed(5)
    words = torch.randint(-(2 ** 31), 2 ** 31, (300, 40), generator=g, dtype=torch.int64).to(torch.int32)
    words[0, :6] = torch.tensor([0, -(2 ** 31), -1, 2 ** 31 - 1, 0x12345678, -0x77777778], dtype=torch.int32)
    n8 = awq.unpack(words.to(dev()), "n8").cpu().numpy()
    k8 = awq.unpack(words.to(dev()), "k8").cpu().numpy()
    assert np.array_equal(n8, orc().unpack_n8(words.numpy()))
    assert np.array_equal(k8, orc().unpack_k8(words.numpy()))


def test_pack_clamps_and_counts():
    vals = torch.tensor([[16, 200, 3, 15, 0, 255, 7, 8]] * 5, dtype=torch.uint8)
    exp, bad = orc().pack_n8(vals.numpy())
    cnt = torch.zeros(1, dtype=torch.int32, device=dev())
    got = awq.pack(vals.to(dev()), "n8", clamp_count=cnt)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)
    assert int(cnt.item()) == bad == 15
    s = torch.tensor([-9, 8, -128, 127, 0, -8, 7, 1], dtype=torch.int8)[:, None].repeat(1, 16)
    exp, bad = orc().pack_k8(s.numpy())
    cnt.zero_()
    got = awq.pack(s.to(dev()), "k8", clamp_count=cnt)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), exp)
    assert int(cnt.item()) == bad == 64
