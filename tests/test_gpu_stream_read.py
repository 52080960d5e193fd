"""The streaming-read measurement helper (tq_stream_read, not part of the
method): its XOR of every 32-bit word equals numpy's, for lengths that leave
the grid-stride loop with and without a remainder, and it accumulates into the
sink (reading the same range twice XORs to zero)."""
import numpy as np
import pytest
import torch

from parity_util import tq

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("n16", [1, 7, 1024 * 256 * 4 + 3, 3_000_001])
def test_stream_read_xor_matches_numpy(n16):
    print(f"[stream read] {n16} x 16 bytes", flush=True)
    rng = np.random.default_rng(n16)
    host = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    tq.stream_read(src, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    tq.stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0
