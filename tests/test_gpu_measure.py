"""The streaming-read measurement aid (GPU only): every 16-byte word of the buffer is read
exactly once, whatever the launch shape -- the XOR of the per-block checksums equals the
XOR of all the buffer's 32-bit words."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import speculative_verify_moe_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("words16,blocks,depth", [(1, 1, 4), (4096 * 37 + 5, 64, 8), (1 << 20, 1024, 16),
                                                  ((1 << 18) + 255, 8192, 4)])
def test_stream_read_reads_every_word_once(words16, blocks, depth):
    import speculative_verify_moe_amd as moe
    print(f"[case] stream_read words16={words16} blocks={blocks} depth={depth}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(words16)
    host = rng.integers(0, 2 ** 32, size=4 * words16, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = moe.moe_measure_stream_read(buf, blocks, depth)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
