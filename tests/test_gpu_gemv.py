"""GPU parity of dequantization and the Q8_0 / Q4_K GEMV kernels against the fp64 oracle.

Gates: dequantized weights bit-exact (fp32 = RN_fp32 of the exact weight, bf16 =
RN_bf16 of that); GEMV floored elementwise relative error <= 2e-3 (tau = 1e-3 of
the row's largest |output|); rows of an M = 2..4 call bit-identical to M = 1 on
the same activation row (the memra pages' rule that verify must reproduce plain
decode byte for byte); run-to-run bitwise determinism; output guard bands
untouched. Shapes span several super-block steps and ragged tails.
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


def _golden(name):
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)["blocks"]


def _golden_q4k_matrix():
    blocks = _golden("q4_k_handbuilt.json")
    raw = np.frombuffer(b"".join(bytes.fromhex(b["hex"]) for b in blocks), dtype=np.uint8)
    return raw, len(blocks)


# ---------------------------------------------------------------- dequantization

@pytest.mark.parametrize("n,k,seed", [(64, 2048, 1), (37, 5120, 2), (3, 17408, 3)])
def test_dequant_q4_k_f32_bit_exact(q, dev, n, k, seed):
    raw = synth.q4_k_weights(seed, n, k)
    got = host(q.qmv_dequant_q4_k_f32(to_dev(raw, dev), n, k))
    ref = oracle.dequant_q4_k_f32(raw, n, k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_q4_k_handbuilt_blocks_bit_exact(q, dev):
    raw, nb = _golden_q4k_matrix()
    got = host(q.qmv_dequant_q4_k_f32(to_dev(raw, dev), nb, 256))
    for i, blk in enumerate(_golden("q4_k_handbuilt.json")):
        expect = np.array([float.fromhex(v) for v in blk["expect"]], dtype=np.float64).astype(np.float32)
        assert np.array_equal(got[i], expect), blk["name"]      # values; zero's sign is not part of the rational
        assert np.array_equal(got[i].view(np.uint32), oracle.dequant_q4_k_f32(bytes.fromhex(blk["hex"]), 1, 256)[0].view(np.uint32))


@pytest.mark.parametrize("n,k,seed", [(64, 2048, 4), (37, 5120, 5)])
def test_dequant_q4_k_bf16_bit_exact(q, dev, n, k, seed):
    raw = synth.q4_k_weights(seed, n, k)
    got = host(q.qmv_dequant_q4_k_bf16(to_dev(raw, dev), n, k)).view(np.uint16)
    assert np.array_equal(got, oracle.dequant_q4_k_bf16_bits(raw, n, k))


@pytest.mark.parametrize("n,k,seed", [(1024, 1024, 6), (33, 96, 7), (5, 32, 8)])
def test_dequant_q8_0_f32_bit_exact(q, dev, n, k, seed):
    raw = synth.q8_0_weights(seed, n, k)
    got = host(q.qmv_dequant_q8_0_f32(to_dev(raw, dev), n, k))
    assert np.array_equal(got.view(np.uint32), oracle.dequant_q8_0_f32(raw, n, k).view(np.uint32))


def test_dequant_q8_0_handbuilt_blocks(q, dev):
    blocks = _golden("q8_0_handbuilt.json")
    raw = np.frombuffer(b"".join(bytes.fromhex(b["hex"]) for b in blocks), dtype=np.uint8)
    got = host(q.qmv_dequant_q8_0_f32(to_dev(raw, dev), len(blocks), 32))
    for i, blk in enumerate(blocks):
        expect = np.array([float.fromhex(v) for v in blk["expect"]]).astype(np.float32)
        # exact rational expectations carry no sign of zero (d < 0, q = 0 gives -0.0 in IEEE)
        assert np.array_equal(got[i], expect), blk["name"]


# ---------------------------------------------------------------- Q8_0 GEMV

@pytest.mark.parametrize("n,k,m", [(1024, 1024, 1), (1024, 1024, 4), (37, 96, 2), (5, 2080, 3), (1, 32, 1)])
def test_q8_0_gemv_parity(q, dev, n, k, m):
    raw = synth.q8_0_weights(100 + m, n, k)
    x = synth.f32_normal(200 + m, (m, k))
    y, buf = guarded((m, n), torch.float32, dev)
    q.qmv_q8_0(to_dev(raw, dev), to_dev(x, dev), n, k, y=y)
    torch.cuda.synchronize()
    ref = oracle.qmv_q8_0(raw, x, n, k)
    err = oracle.floored_rel_err(host(y), ref)
    assert err <= GEMV_TOL, err
    assert guards_intact(buf)


def test_q8_0_rows_bit_identical_across_m(q, dev):
    n, k = 1024, 1024
    w = to_dev(synth.q8_0_weights(110, n, k), dev)
    x = to_dev(synth.f32_normal(111, (4, k)), dev)
    full = host(q.qmv_q8_0(w, x, n, k))
    for r in range(4):
        one = host(q.qmv_q8_0(w, x[r:r + 1].contiguous(), n, k))
        assert np.array_equal(one[0].view(np.uint32), full[r].view(np.uint32)), r


# ---------------------------------------------------------------- Q4_K GEMV

SHAPES = [(64, 5120), (48, 17408), (37, 1280), (19, 768), (1, 256), (130, 2048)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_q4_k_gemv_parity(q, dev, n, k, m):
    raw = synth.q4_k_weights(300 + n, n, k)
    x = synth.bf16_normal(400 + m, (m, k))
    y, buf = guarded((m, n), torch.float32, dev)
    q.qmv_q4_k(to_dev(raw, dev), to_dev(x, dev), n, k, y=y)
    torch.cuda.synchronize()
    ref = oracle.qmv_q4_k(raw, x, n, k)
    err = oracle.floored_rel_err(host(y), ref)
    assert err <= GEMV_TOL, err
    assert guards_intact(buf)


# Row lengths that reach every unrolled step count of both lane widths (16 lanes:
# 1..8 steps of 4 blocks, 32 lanes: 5..9 steps of 8 blocks, with and without a
# partial last step) and the runtime-loop kernel beyond 18432 (whole and partial
# last step); M = 1..4 as far as the activations fit in LDS.
K_SWEEP = [2560, 3840, 6144, 7168, 8192, 8448, 10240, 12288, 14336, 16384, 18432, 19712, 20480, 36864]


def _lds_fits(m, k):
    return m * ((k // 128) * 272 + (k // 32) * 4) <= 163840


@pytest.mark.parametrize("k", K_SWEEP)
def test_q4_k_step_counts_parity_and_bit_identity(q, dev, k):
    n = 23
    raw = synth.q4_k_weights(800 + k // 256, n, k)
    ms = [m for m in (1, 2, 3, 4) if _lds_fits(m, k)]
    x = synth.bf16_normal(900 + k // 256, (max(ms), k))
    wd = to_dev(raw, dev)
    ref = oracle.qmv_q4_k(raw, x, n, k)
    single = None
    for m in ms:
        y, buf = guarded((m, n), torch.float32, dev)
        q.qmv_q4_k(wd, to_dev(x[:m], dev), n, k, y=y)
        torch.cuda.synchronize()
        got = host(y)
        assert guards_intact(buf)
        err = oracle.floored_rel_err(got, ref[:m])
        assert err <= GEMV_TOL, (m, err)
        if m == 1:
            single = got[0]
        else:
            assert np.array_equal(got[0].view(np.uint32), single.view(np.uint32)), m


@pytest.mark.parametrize("n,k", [(5120, 2048), (2560, 8448)])
def test_q4_k_balanced_workgroups_parity(q, dev, n, k):
    # row counts that divide evenly over the CUs take the balanced launch (20 rows of
    # 16 lanes, 10 rows of 32 lanes per workgroup); rows must match the default launch
    raw = synth.q4_k_weights(950, n, k)
    x = synth.bf16_normal(951, (2, k))
    wd = to_dev(raw, dev)
    y1 = host(q.qmv_q4_k(wd, to_dev(x[:1], dev), n, k))
    assert oracle.floored_rel_err(y1, oracle.qmv_q4_k(raw, x[:1], n, k)) <= GEMV_TOL
    y2 = host(q.qmv_q4_k(wd, to_dev(x, dev), n, k))   # M = 2 uses 256-thread workgroups
    assert np.array_equal(y1[0].view(np.uint32), y2[0].view(np.uint32))


def test_q4_k_gemv_handbuilt_blocks(q, dev):
    # zero and subnormal scales, top-bit carries: one row per hand-built block
    raw, nb = _golden_q4k_matrix()
    x = synth.bf16_normal(500, (2, 256))
    y = host(q.qmv_q4_k(to_dev(raw, dev), to_dev(x, dev), nb, 256))
    ref = oracle.qmv_q4_k(raw, x, nb, 256)
    assert oracle.floored_rel_err(y, ref) <= GEMV_TOL


@pytest.mark.parametrize("n,k", [(17408, 5120), (5120, 17408), (37, 1280)])
def test_q4_k_rows_bit_identical_across_m(q, dev, n, k):
    w = synth.torch_q4_k_weights(7, n, k, dev)
    x = to_dev(synth.bf16_normal(600, (4, k)), dev)
    singles = [host(q.qmv_q4_k(w, x[r:r + 1].contiguous(), n, k))[0] for r in range(4)]
    for m in (2, 3, 4):
        multi = host(q.qmv_q4_k(w, x[:m].contiguous(), n, k))
        for r in range(m):
            assert np.array_equal(multi[r].view(np.uint32), singles[r].view(np.uint32)), (m, r)


def test_q4_k_deterministic_and_stream_independent(q, dev):
    n, k = 17408, 5120
    w = synth.torch_q4_k_weights(8, n, k, dev)
    x = to_dev(synth.bf16_normal(601, (1, k)), dev)
    a = host(q.qmv_q4_k(w, x, n, k))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = q.qmv_q4_k(w, x, n, k, stream=s)
    s.synchronize()
    assert np.array_equal(a.view(np.uint32), host(b).view(np.uint32))


@pytest.mark.parametrize("n,k", [(17408, 5120), (5120, 17408)])
@pytest.mark.parametrize("m", [1, 4])
def test_q4_k_full_size_sampled_rows(q, dev, n, k, m):
    # the decode shapes of the dense 27B-like FFN; 192 sampled rows checked against the oracle
    w = synth.torch_q4_k_weights(9 + m, n, k, dev)
    x = synth.bf16_normal(700 + m, (m, k))
    y = host(q.qmv_q4_k(w, to_dev(x, dev), n, k))
    rows = np.sort(np.random.default_rng(n + m).choice(n, 192, replace=False))
    row_bytes = (k // 256) * 144
    wh = host(w.view(-1, row_bytes)[torch.as_tensor(rows, device=dev)])
    ref = oracle.qmv_q4_k(wh.reshape(-1), x, len(rows), k)
    assert oracle.floored_rel_err(y[:, rows], ref) <= GEMV_TOL
    assert np.isfinite(y).all()
