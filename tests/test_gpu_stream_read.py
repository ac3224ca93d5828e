"""The streaming-read ceiling kernel reads every byte once: the XOR of its per-workgroup sink
words equals the XOR of all 32-bit words of the buffer (a sizes with a ragged tail included)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16 * 7, (64 << 20) + 16 * 123])
def test_stream_read_reads_every_byte_once(nbytes):
    rng = np.random.default_rng((444, 90, nbytes))
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(pa.load_library().pa_stream_read_sink_words(), dtype=torch.int32,
                       device="cuda")
    pa.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
