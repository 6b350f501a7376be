"""tv_stream_read (the bandwidth measurement aid) reads every 16-byte piece
exactly once: the XOR of its per-workgroup words equals the XOR of every
32-bit word of the buffer, for sizes around the grid's stride."""

import numpy as np
import pytest
import torch

from tree_verification_attention_tv_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 4 * 2048 * 256 - 4, 4 * 2048 * 256 * 8 + 12, 3_000_004])
def test_stream_read_folds_every_word_once(words):
    print(f"[stream_read] {words} words", flush=True)
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**31 - 1, size=words, dtype=np.int64).astype(np.int32)
    x = torch.from_numpy(host).cuda()
    sink = torch.zeros(binding.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    binding.stream_read(x, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want
