"""GPU check of the streaming-read reference the bench measures the HBM read bandwidth with:
every 32-bit word of the buffer must be read once, which the XOR of all words shows exactly
(numpy computes the same XOR on the host copy).  Sizes span one 16-byte word, fewer words than
one workgroup's eight loads per thread, and ranges that split unevenly over the 512 workgroups
(each reads one contiguous range, with a ragged tail)."""

import numpy as np
import pytest
import torch

import expert_load_balancing_amd as elb

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words", [4, 4 * 1000 + 4, 4 * (2048 * 256 * 8) + 12, 4 * (2048 * 256 * 8 * 3) - 4,
                                     16 << 20])
def test_stream_xor_reads_every_word(n_words):
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 32, size=n_words, dtype=np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    out = elb.stream_xor(dev)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)


def test_stream_xor_accumulates_into_out_and_skips_empty():
    host = np.arange(64, dtype=np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    elb.stream_xor(dev, out=out)
    elb.stream_xor(dev[:0], out=out)
    torch.cuda.synchronize()
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host) ^ np.uint32(0x5A5A5A5A))
