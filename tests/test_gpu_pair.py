"""GPU parity of qmv_q4_k_pair: two Q4_K matrices on one activation in one launch.

The pair launch runs the Q4_K GEMV over 2n rows, the first n from matrix 0 and the
rest from matrix 1. Every output row takes the same instruction sequence as in a
one-matrix call, so both outputs must be bit-identical to two qmv_q4_k calls (the
memra pages' rule that a verify pass reproduces plain decode byte for byte), and
within the GEMV tolerance of the fp64 oracle. Shapes cover both lane widths, the
runtime-loop kernel, ragged n where one workgroup holds rows of both matrices, and
the 17408 x 5120 gate/up projections of the dense Q4_K_M decode pass.
"""

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


def _lds_fits(m, k):
    return m * ((k // 128) * 272 + (k // 32) * 4) <= 163840


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


# n values that leave a workgroup holding the tail of matrix 0 and the head of
# matrix 1 (16-lane rows: 16 or 20 rows per workgroup; 32-lane rows: 8 or 10)
SHAPES = [(17408, 5120), (37, 1280), (1, 256), (130, 2048), (2560, 8448), (23, 12288), (45, 20480), (3, 36864)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_pair_bit_identical_to_two_calls(q, dev, n, k):
    w0 = synth.torch_q4_k_weights(1000 + n % 97, n, k, dev)
    w1 = synth.torch_q4_k_weights(2000 + k // 256, n, k, dev)
    x = to_dev(synth.bf16_normal(3000 + n % 89, (4, k)), dev)
    for m in (m for m in (1, 2, 3, 4) if _lds_fits(m, k)):
        xm = x[:m].contiguous()
        y0, b0 = guarded((m, n), torch.float32, dev)
        y1, b1 = guarded((m, n), torch.float32, dev)
        q.qmv_q4_k_pair(w0, w1, xm, n, k, y0=y0, y1=y1)
        torch.cuda.synchronize()
        assert guards_intact(b0) and guards_intact(b1), m
        assert np.array_equal(_bits(host(y0)), _bits(host(q.qmv_q4_k(w0, xm, n, k)))), (m, "matrix 0")
        assert np.array_equal(_bits(host(y1)), _bits(host(q.qmv_q4_k(w1, xm, n, k)))), (m, "matrix 1")


@pytest.mark.parametrize("n,k,m", [(37, 1280, 3), (130, 2048, 1), (23, 12288, 2), (5, 20480, 3)])
def test_pair_matches_oracle(q, dev, n, k, m):
    r0, r1 = synth.q4_k_weights(4000 + n, n, k), synth.q4_k_weights(5000 + n, n, k)
    x = synth.bf16_normal(6000 + m, (m, k))
    y0, y1 = q.qmv_q4_k_pair(to_dev(r0, dev), to_dev(r1, dev), to_dev(x, dev), n, k)
    torch.cuda.synchronize()
    for got, raw in ((y0, r0), (y1, r1)):
        err = oracle.floored_rel_err(host(got), oracle.qmv_q4_k(raw, x, n, k))
        assert err <= GEMV_TOL, err


def test_pair_same_matrix_twice(q, dev):
    # both halves may read one buffer: the outputs are then equal bit for bit
    n, k = 130, 5120
    w = synth.torch_q4_k_weights(7000, n, k, dev)
    x = to_dev(synth.bf16_normal(7001, (2, k)), dev)
    y0, y1 = q.qmv_q4_k_pair(w, w, x, n, k)
    assert np.array_equal(_bits(host(y0)), _bits(host(y1)))


def test_pair_rejects_overlapping_outputs(q, dev):
    n, k = 16, 256
    w = synth.torch_q4_k_weights(7100, n, k, dev)
    x = to_dev(synth.bf16_normal(7101, (1, k)), dev)
    buf = torch.zeros(2 * n, dtype=torch.float32, device=dev)
    with pytest.raises(q.QmvError) as e:
        q.qmv_q4_k_pair(w, w, x, n, k, y0=buf[:n].view(1, n), y1=buf[n // 2:n // 2 + n].view(1, n))
    assert e.value.code == -7   # QMV_ERR_ALIAS, raised before any launch


@pytest.mark.parametrize("m", [1, 4])
def test_pair_full_size_sampled_rows(q, dev, m):
    # the gate/up projections of the dense Q4_K_M decode pass in the launch the benchmark times:
    # about 192 sampled rows of each output checked against the oracle, among them row n - 1 of
    # matrix 0 and row 0 of matrix 1, the two sides of the boundary in the 2n-row grid
    n, k = 17408, 5120
    w0 = synth.torch_q4_k_weights(8100 + m, n, k, dev)
    w1 = synth.torch_q4_k_weights(8200 + m, n, k, dev)
    x = synth.bf16_normal(8300 + m, (m, k))
    y0, y1 = q.qmv_q4_k_pair(w0, w1, to_dev(x, dev), n, k)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8400 + m)
    row_bytes = (k // 256) * 144
    for got, w, edge in ((y0, w0, [n - 1]), (y1, w1, [0])):
        rows = np.unique(np.concatenate([rng.choice(n, 190, replace=False), edge, [n // 2]]))
        wh = host(w.view(-1, row_bytes)[torch.as_tensor(rows, device=dev)])
        ref = oracle.qmv_q4_k(wh.reshape(-1), x, len(rows), k)
        yh = host(got)
        assert np.isfinite(yh).all()
        assert oracle.floored_rel_err(yh[:, rows], ref) <= GEMV_TOL


def test_pair_and_down_graph_replays_match_eager(q, dev):
    # one layer of the dense decode pass (the pair launch for gate and up, then the down launch)
    # captured once and replayed three times, with eager calls on other inputs in between: every
    # replay reproduces the eager outputs bit for bit
    n, k = 17408, 5120
    wg = synth.torch_q4_k_weights(8500, n, k, dev)
    wu = synth.torch_q4_k_weights(8501, n, k, dev)
    wd = synth.torch_q4_k_weights(8502, k, n, dev)
    x = to_dev(synth.bf16_normal(8503, (1, k)), dev)
    h = to_dev(synth.bf16_normal(8504, (1, n)), dev)
    other = to_dev(synth.bf16_normal(8505, (1, k)), dev)
    g_ref, u_ref = (host(t) for t in q.qmv_q4_k_pair(wg, wu, x, n, k))
    d_ref = host(q.qmv_q4_k(wd, h, k, n))
    yg = torch.empty((1, n), dtype=torch.float32, device=dev)
    yu = torch.empty((1, n), dtype=torch.float32, device=dev)
    yd = torch.empty((1, k), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.qmv_q4_k_pair(wg, wu, x, n, k, y0=yg, y1=yu)
        q.qmv_q4_k(wd, h, k, n, y=yd)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qmv_q4_k_pair(wg, wu, x, n, k, y0=yg, y1=yu)
        q.qmv_q4_k(wd, h, k, n, y=yd)
    for i in range(3):
        for t in (yg, yu, yd):
            t.fill_(float("nan"))
        q.qmv_q4_k_pair(wu, wg, other, n, k)   # eager work on other inputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(host(yg)), _bits(g_ref)), (i, "gate")
        assert np.array_equal(_bits(host(yu)), _bits(u_ref)), (i, "up")
        assert np.array_equal(_bits(host(yd)), _bits(d_ref)), (i, "down")
