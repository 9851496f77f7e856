"""GPU parity of the Q4_0 dequantization and GEMV against the fp64 oracle.

Gates: dequantized weights bit-exact (every Q4_0 weight is exact in fp32); GEMV
floored elementwise relative error <= 2e-3; rows of an M = 2..4 call
bit-identical to M = 1 on the same activation row; run-to-run determinism;
output guard bands untouched. The GEMV steps over groups of eight 18-byte
blocks (144 bytes, 256 weights), so its shapes are those of the Q4_K tests:
one-group rows, group counts that leave the last step partial, rows past the
last workgroup's, both lane groupings, the runtime-length loop and the dense
FFN shapes at full size (sampled rows). The dequantization takes any K that is
a multiple of 32, including odd block counts (blocks at 2 bytes into a dword).
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


def _golden():
    with open(os.path.join(os.path.dirname(__file__), "golden", "q4_0_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    return np.frombuffer(b"".join(bytes.fromhex(b["hex"]) for b in blocks), dtype=np.uint8), len(blocks)


@pytest.mark.parametrize("n,k,seed", [(64, 2048, 1), (37, 5120, 2), (3, 17408, 3), (5, 96, 4), (1, 32, 5),
                                      (7, 160, 6)])
def test_dequant_q4_0_f32_bit_exact(q, dev, n, k, seed):
    raw = synth.q4_0_weights(seed, n, k)
    got = host(q.qmv_dequant_q4_0_f32(to_dev(raw, dev), n, k))
    ref = oracle.dequant_q4_0_f32(raw, n, k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_q4_0_handbuilt_blocks(q, dev):
    raw, nb = _golden()
    got = host(q.qmv_dequant_q4_0_f32(to_dev(raw, dev), nb, 32))
    assert np.array_equal(got.view(np.uint32), oracle.dequant_q4_0_f32(raw, nb, 32).view(np.uint32))


def _gemv(q, dev, raw, x, n, k):
    m = x.shape[0]
    y, buf = guarded((m, n), torch.float32, dev)
    q.qmv_q4_0(to_dev(raw, dev), to_dev(x, dev), n, k, y=y)
    torch.cuda.synchronize()
    assert guards_intact(buf)
    return host(y)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k", [(1, 256), (64, 256), (100, 1280), (37, 5120), (260, 2048), (24, 9216), (9, 8448),
                                 (19, 17408)])
def test_q4_0_gemv_parity(q, dev, n, k, m):
    raw = synth.q4_0_weights(n + k + m, n, k)
    x = synth.bf16_normal(k + m, (m, k))
    y = _gemv(q, dev, raw, x, n, k)
    err = oracle.floored_rel_err(y, oracle.qmv_q4_0(raw, x, n, k))
    assert err <= GEMV_TOL, err


@pytest.mark.parametrize("m", [1, 2, 3])
def test_q4_0_gemv_runtime_length_rows(q, dev, m):
    # 73 groups of eight blocks: past the unrolled step counts and not a whole
    # number of steps (m = 4 would exceed the LDS stage at this K)
    n, k = 8, 18688
    raw = synth.q4_0_weights(97 + m, n, k)
    x = synth.bf16_normal(98 + m, (m, k))
    y = _gemv(q, dev, raw, x, n, k)
    assert oracle.floored_rel_err(y, oracle.qmv_q4_0(raw, x, n, k)) <= GEMV_TOL


def test_q4_0_gemv_handbuilt_blocks(q, dev):
    # the six hand-built blocks, padded with two zero-scale blocks to one group of eight
    raw, nb = _golden()
    pad = np.zeros(18 * (8 - nb), dtype=np.uint8)
    raw8 = np.concatenate([raw, pad])
    x = synth.bf16_normal(90, (2, 256))
    y = _gemv(q, dev, raw8, x, 1, 256)
    assert oracle.floored_rel_err(y, oracle.qmv_q4_0(raw8, x, 1, 256)) <= GEMV_TOL


@pytest.mark.parametrize("n,k", [(48, 5120), (40, 17408)])
def test_q4_0_rows_bit_identical_for_every_m(q, dev, n, k):
    raw = synth.q4_0_weights(91, n, k)
    x = synth.bf16_normal(92, (4, k))
    y4 = _gemv(q, dev, raw, x, n, k)
    for m in (1, 2, 3):
        ym = _gemv(q, dev, raw, x[:m], n, k)
        assert np.array_equal(ym.view(np.uint32), y4[:m].view(np.uint32)), m
    for r in range(4):
        y1 = _gemv(q, dev, raw, x[r:r + 1], n, k)
        assert np.array_equal(y1[0].view(np.uint32), y4[r].view(np.uint32)), r


def test_q4_0_deterministic(q, dev):
    n, k = 300, 5120
    raw = to_dev(synth.q4_0_weights(93, n, k), dev)
    x = to_dev(synth.bf16_normal(94, (2, k)), dev)
    a = host(q.qmv_q4_0(raw, x, n, k))
    b = host(q.qmv_q4_0(raw, x, n, k))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("n,k,m", [(17408, 5120, 1), (5120, 17408, 1), (17408, 5120, 4), (5120, 17408, 4)])
def test_q4_0_full_size_sampled_rows(q, dev, n, k, m):
    w = synth.torch_q4_0_weights(95, n, k, dev)
    x = synth.bf16_normal(96 + m, (m, k))
    y = host(q.qmv_q4_0(w, to_dev(x, dev), n, k))
    assert np.isfinite(y).all()
    rows = np.sort(np.random.default_rng(n + m).choice(n, 128, replace=False))
    row_bytes = (k // 32) * 18
    wh = host(w.view(-1, row_bytes)[torch.as_tensor(rows, device=dev)])
    ref = oracle.qmv_q4_0(wh.reshape(-1), x, len(rows), k)
    assert oracle.floored_rel_err(y[:, rows], ref) <= GEMV_TOL
