"""The bandwidth probe reads every byte: its per-wave XOR checksums fold to
the XOR of all 32-bit words of the buffer (checked on the CPU)."""
import numpy as np
import pytest
import torch

import bit_weight_only_awq_amd as awq
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16, 64 << 20])
def test_stream_read_touches_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev())
    sink = torch.zeros(awq.ops.STREAM_SINK_WORDS, dtype=torch.int32, device=dev())
    awq.stream_read(src, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
