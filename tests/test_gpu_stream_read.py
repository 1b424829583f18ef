"""The streaming-read kernel (nucleus_stream_read) reads every byte once:
its XOR checksum over the 256 sink words equals the host's XOR of the
buffer's 32-bit words and tail bytes, for sizes that fill whole blocks,
leave a ragged last block, and end in a partial 16-byte unit."""
import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu


def _host_xor(a: np.ndarray) -> int:
    n16 = a.size // 16
    words = a[: n16 * 16].view(np.uint32)
    acc = int(np.bitwise_xor.reduce(words)) if words.size else 0
    for byte in a[n16 * 16:]:
        acc ^= int(byte)
    return acc


@pytest.mark.parametrize("nbytes", [16, 17, 4096, 65536 * 16 + 48, 65536 * 3 + 31, 131334144 + 7])
def test_stream_read_checksum(nbytes):
    import torch

    import nucleus_sampling_amd as ns

    rng = np.random.default_rng(nbytes)
    a = rng.integers(0, 256, nbytes, dtype=np.uint8)
    say(f"stream_read over {nbytes} bytes")
    buf = torch.from_numpy(a).to("cuda:0")
    sink = torch.zeros(256, dtype=torch.int64, device="cuda:0")
    ns.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint64)))
    assert got == _host_xor(a)
