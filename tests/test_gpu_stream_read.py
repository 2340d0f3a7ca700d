"""tv_stream_read, the plain-read yardstick that bench.py times next to the
decode kernel: every byte is read (the per-chunk XOR of 32-bit words equals
the host's, bit for bit), including a ragged last chunk and a one-piece
buffer."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CHUNK = 8192


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import paged_kv_cache_tv_amd as tv
    tv.lib()
    return torch.device("cuda:0")


def _host_xor(words: np.ndarray) -> np.ndarray:
    per = CHUNK // 4
    n = -(-words.size // per)
    padded = np.zeros(n * per, dtype=np.uint32)
    padded[:words.size] = words
    return np.bitwise_xor.reduce(padded.reshape(n, per), axis=1)


@pytest.mark.parametrize("nbytes", [16, CHUNK, 37 * CHUNK + 5 * 16, (1 << 26) + 48])
def test_stream_read_touches_every_byte(dev, nbytes):
    import torch
    import paged_kv_cache_tv_amd as tv
    rng = np.random.default_rng(nbytes % 1009)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    chunks = -(-nbytes // CHUNK)
    out = torch.full((chunks + 1,), -7, dtype=torch.int32, device=dev)
    tv.stream_read(buf, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:chunks], _host_xor(words))
    assert got[chunks] == np.uint32(-7 & 0xffffffff), "wrote past the last chunk"
