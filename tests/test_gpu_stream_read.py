"""GPU check of the streaming-read probe (attn_stream_read): every 16-byte
chunk of the buffer is read exactly once, so the XOR of the per-thread sink
words equals the XOR of all 32-bit words of the buffer (computed on the
CPU), for several grid sizes and a ragged tail."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_fwd_amd as pa
    pa.load_library()


@pytest.mark.parametrize("depth", [4, 8])
@pytest.mark.parametrize("n_words,grid", [(4, 1), (4 * 1000 + 4, 3), (1 << 20, 512), ((1 << 22) + 12, 2048)])
def test_every_chunk_read_once(n_words, grid, depth):
    import paged_kv_gqa_fwd_amd as pa
    g = torch.Generator().manual_seed(n_words)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), dtype=torch.int64, generator=g).to(torch.int32)
    buf = host.cuda()
    sink = pa.stream_read(buf, grid, depth=depth)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink[: grid * 256].cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
