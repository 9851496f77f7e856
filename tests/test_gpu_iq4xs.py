"""GPU parity of the IQ4_XS dequantization and GEMV against the fp64 oracle.

Gates: dequantized weights bit-exact (IQ4_XS weights are exact in fp32); GEMV
floored elementwise relative error <= 2e-3 (tau = 1e-3 of the row's largest
|output|); rows of an M = 2..4 call bit-identical to M = 1 on the same
activation row; run-to-run determinism; output guard bands untouched. Shapes
span several units per lane, an odd number of super-blocks per row (units past
the row), rows past the last workgroup's, both lane groupings (16 lanes per row
up to K = 8192, 32 beyond) and the largest K that the staged activations allow.
"""

import json
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import GEMV_TOL, device, guarded, guards_intact, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    import gguf_block_quantized_qmv_amd as mod
    return mod


@pytest.fixture(scope="module")
def dev():
    return device()


def _golden_matrix():
    with open(os.path.join(os.path.dirname(__file__), "golden", "iq4_xs_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    raw = np.frombuffer(b"".join(bytes.fromhex(b["hex"]) for b in blocks), dtype=np.uint8)
    return raw, len(blocks)


@pytest.mark.parametrize("n,k,seed", [(64, 2048, 1), (37, 5120, 2), (3, 17408, 3), (5, 768, 4)])
def test_dequant_iq4_xs_f32_bit_exact(q, dev, n, k, seed):
    raw = synth.iq4_xs_weights(seed, n, k)
    got = host(q.qmv_dequant_iq4_xs_f32(to_dev(raw, dev), n, k))
    ref = oracle.dequant_iq4_xs(raw, n, k).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_iq4_xs_handbuilt_blocks_bit_exact(q, dev):
    raw, nb = _golden_matrix()
    got = host(q.qmv_dequant_iq4_xs_f32(to_dev(raw, dev), nb, 256))
    ref = oracle.dequant_iq4_xs(raw, nb, 256).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _gemv(q, dev, raw, x, n, k):
    m = x.shape[0]
    y, buf = guarded((m, n), torch.float32, dev)
    q.qmv_iq4_xs(to_dev(raw, dev), to_dev(x, dev), n, k, y=y)
    torch.cuda.synchronize()
    assert guards_intact(buf)
    return host(y)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k", [(64, 256), (100, 768), (37, 5120), (260, 2048), (24, 8448), (19, 17408)])
def test_iq4_xs_gemv_parity(q, dev, n, k, m):
    raw = synth.iq4_xs_weights(n + k + m, n, k)
    x = synth.bf16_normal(k + m, (m, k))
    y = _gemv(q, dev, raw, x, n, k)
    err = oracle.floored_rel_err(y, oracle.qmv_iq4_xs(raw, x, n, k))
    assert err <= GEMV_TOL, err


def test_iq4_xs_gemv_handbuilt_blocks(q, dev):
    # rows of the hand-built blocks (grid walk, signed and zero scales, subnormal d)
    raw, nb = _golden_matrix()
    x = synth.bf16_normal(90, (2, 256))
    y = _gemv(q, dev, raw, x, nb, 256)
    err = oracle.floored_rel_err(y, oracle.qmv_iq4_xs(raw, x, nb, 256))
    assert err <= GEMV_TOL, err


@pytest.mark.parametrize("n,k", [(48, 5120), (40, 17408), (16, 18944)])
def test_iq4_xs_rows_bit_identical_for_every_m(q, dev, n, k):
    raw = synth.iq4_xs_weights(91, n, k)
    x = synth.bf16_normal(92, (4, k))
    y4 = _gemv(q, dev, raw, x, n, k)
    for m in (1, 2, 3):
        ym = _gemv(q, dev, raw, x[:m], n, k)
        assert np.array_equal(ym.view(np.uint32), y4[:m].view(np.uint32)), m
    for r in range(4):
        y1 = _gemv(q, dev, raw, x[r:r + 1], n, k)
        assert np.array_equal(y1[0].view(np.uint32), y4[r].view(np.uint32)), r


def test_iq4_xs_deterministic(q, dev):
    n, k = 300, 5120
    raw = to_dev(synth.iq4_xs_weights(93, n, k), dev)
    x = to_dev(synth.bf16_normal(94, (2, k)), dev)
    a = host(q.qmv_iq4_xs(raw, x, n, k))
    b = host(q.qmv_iq4_xs(raw, x, n, k))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("n,k,m", [(17408, 5120, 1), (5120, 17408, 1), (17408, 5120, 4), (5120, 17408, 4)])
def test_iq4_xs_full_size_sampled_rows(q, dev, n, k, m):
    # the dense 27B-like FFN shapes in IQ4_XS; 128 sampled rows checked against the oracle
    w = synth.torch_iq4_xs_weights(95, n, k, dev)
    x = synth.bf16_normal(96 + m, (m, k))
    y = host(q.qmv_iq4_xs(w, to_dev(x, dev), n, k))
    assert np.isfinite(y).all()
    rows = np.sort(np.random.default_rng(n + m).choice(n, 128, replace=False))
    row_bytes = (k // 256) * 136
    wh = host(w.view(-1, row_bytes)[torch.as_tensor(rows, device=dev)])
    ref = oracle.qmv_iq4_xs(wh.reshape(-1), x, len(rows), k)
    assert oracle.floored_rel_err(y[:, rows], ref) <= GEMV_TOL
