"""GPU check of w4_stream_read, the plain-read measurement kernel: every
32-bit word of the buffer is read once (its XOR matches the host's)."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_amd as w4
from gpu_helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 35651584])
def test_stream_read_xor(nbytes):
    require_gpu()
    rng = np.random.default_rng(nbytes % 1000)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    acc = torch.zeros(w4.STREAM_READ_ACC_WORDS, dtype=torch.int32, device="cuda")
    announce("stream read", dict(nbytes=nbytes))
    w4.stream_read(buf, acc)
    got = acc.cpu().numpy().view(np.uint32)
    assert np.all(np.delete(got, np.arange(0, 449, 64)) == 0)  # only the eight fold words are written
    assert int(np.bitwise_xor.reduce(got[::64])) == int(np.bitwise_xor.reduce(words))
    w4.stream_read(buf, acc)  # a second pass cancels the first
    assert np.all(acc.cpu().numpy() == 0)
