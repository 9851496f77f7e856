"""The streaming-read calibration kernel reads every byte it is given exactly
once: each workgroup's XOR word equals the host XOR of the granules the grid
stride assigns to it (thread t of workgroup b owns granules g with
g mod (grid * 256) == 256 b + t), for every ring depth and a ragged tail."""

import numpy as np
import pytest

from gpu_util import device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("depth", [1, 2, 4, 8])
@pytest.mark.parametrize("grid,n16", [(1, 1), (3, 5000), (8, 256 * 8 * 8 * 3 + 17), (40, 100003)])
def test_stream_read_covers_every_granule_once(grid, n16, depth, nt):
    import gguf_block_quantized_qmv_amd as q
    dev = device()
    rng = np.random.default_rng(grid * 7 + n16)
    host = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).reshape(-1).copy()).to(dev)
    sink = q.qmv_stream_read(buf, grid=grid, depth=depth, nontemporal=nt)
    got = sink.cpu().numpy().view(np.uint32)
    g = np.arange(n16)
    owner = (g % (grid * 256)) // 256
    words = np.bitwise_xor.reduce(host, axis=1)
    want = np.zeros(grid, dtype=np.uint32)
    np.bitwise_xor.at(want, owner, words)
    assert np.array_equal(got, want)
