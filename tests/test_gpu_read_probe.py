"""spec_read_probe (the plain-read measurement aid): every chunk's largest 32-bit
word, against numpy, for buffers with partial last chunks and a tail shorter than
16 bytes, one buffer or two."""
import numpy as np
import pytest

import acceptance_row_softmax_amd as sv
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _expect(buf):
    n16 = (buf.size // 16) * 16          # a tail shorter than 16 bytes is not read
    words = buf[:n16].view(np.uint32)
    return [int(words[c * 2048:(c + 1) * 2048].max()) for c in range((n16 + 8191) // 8192)]


@pytest.mark.parametrize("sizes", [(8192, 0), (100_000, 0), (65_536, 24_583), (16, 8192 * 3 + 48)])
def test_read_probe_chunk_maxima(sizes):
    import torch
    rng = np.random.default_rng(sum(sizes))
    G.say(f"read probe: buffers of {sizes} bytes")
    host = [rng.integers(0, 256, size=n, dtype=np.uint8) for n in sizes]
    dev = [torch.from_numpy(h).cuda() if h.size else None for h in host]
    sink = sv.read_probe(dev[0], dev[1])
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = _expect(host[0]) + (_expect(host[1]) if host[1].size else [])
    assert got[:len(want)].tolist() == want
