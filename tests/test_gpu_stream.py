"""The streaming-read measurement hook reads every byte once: the XOR of its
per-workgroup results equals the XOR of all 32-bit words of the buffer
(computed on the host), for sizes that leave a partial round and for an
empty buffer."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import mla_decode_attention_02_amd as m
    m.library()
    return m


@pytest.mark.parametrize("words,sink_len", [(0, 4), (4, 1), (1 << 20, 64), ((3 << 20) + 44, 2048)])
def test_stream_read_xor_matches_host(mla, words, sink_len):
    rng = np.random.default_rng(7000 + words % 97)
    host = rng.integers(-(1 << 31), 1 << 31, size=words, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda() if words else torch.empty(0, dtype=torch.int32, device="cuda")
    sink = torch.full((sink_len,), -1, dtype=torch.int32, device="cuda")
    mla.stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32)) if words else np.uint32(0)
    assert int(got) == int(want)
