"""GPU parity of the routed-expert MoE entry point against the fp64 oracle.

Gates: top-k expert ids and the (expert, token) gather list bit-exact; routing
weights within fp32 rounding of the oracle's; outputs within the floored 2e-3
relative gate; a token's output bit-identical whether it runs alone (T=1) or in
a batch of 3 (the memra README's one-numeric-class rule); run-to-run bitwise
determinism; output and workspace guards untouched.
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


def _run(q, dev, bank, logits, x, hidden, ffn, ne, tk):
    gate, up, down = bank
    t = x.shape[0]
    y, ybuf = guarded((t, hidden), torch.float32, dev)
    need = q.qmv_q4_k_moe_workspace(t, hidden, ffn, ne, tk)
    ws_buf = torch.full((need + 512,), 0xA5, dtype=torch.uint8, device=dev)
    ws = ws_buf[256:256 + need]
    y, ids, wts, pairs = q.qmv_q4_k_moe(to_dev(gate, dev), to_dev(up, dev), to_dev(down, dev), to_dev(logits, dev),
                                        to_dev(x, dev), hidden, ffn, ne, tk, y=y, ws=ws)
    torch.cuda.synchronize()
    assert guards_intact(ybuf)
    assert bool((ws_buf[:256] == 0xA5).all() and (ws_buf[256 + need:] == 0xA5).all())
    return host(y), host(ids), host(wts), host(pairs)


def _check(q, dev, seed, t, hidden, ffn, ne, tk, logits=None):
    bank = synth.moe_bank(seed, ne, hidden, ffn)
    if logits is None:
        logits = synth.moe_logits(seed, t, ne)
    x = synth.bf16_normal(seed + 1, (t, hidden))
    y, ids, wts, pairs = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    yr, idr, wr = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.array_equal(pairs, oracle.gather_pairs(idr))
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y, yr)
    assert err <= GEMV_TOL, err
    return y, ids, bank, logits, x


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_moe_small_bank_parity(q, dev, t):
    _check(q, dev, 10 + t, t, hidden=512, ffn=256, ne=16, tk=4)


@pytest.mark.parametrize("t", [1, 3])
def test_moe_35b_a3b_layer_parity(q, dev, t):
    # hidden 2048, 128 experts with 768x2048 gate/up and 2048x768 down, top-8
    _check(q, dev, 20 + t, t, hidden=2048, ffn=768, ne=128, tk=8)


def test_moe_token_bit_identical_alone_and_batched(q, dev):
    hidden, ffn, ne, tk = 2048, 768, 128, 8
    bank = synth.moe_bank(30, ne, hidden, ffn)
    logits = synth.moe_logits(30, 3, ne)
    logits[1] = logits[0]                           # tokens 0 and 1 share all experts
    logits[2, :64] = logits[0, :64]                 # token 2 shares some
    x = synth.bf16_normal(31, (3, hidden))
    y3, ids3, *_ = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    for t in range(3):
        y1, ids1, *_ = _run(q, dev, bank, logits[t:t + 1], x[t:t + 1], hidden, ffn, ne, tk)
        assert np.array_equal(ids1[0], ids3[t])
        assert np.array_equal(y1[0].view(np.uint32), y3[t].view(np.uint32)), t


@pytest.mark.parametrize("hidden", [256, 1280, 4608])
def test_moe_token_bit_identical_alone_and_batched_ragged_rows(q, dev, hidden):
    # rows of 1, 5 and 18 blocks: one token runs 32 lanes per row (8 blocks per step: 1, 1 and 3
    # steps, the last ragged), several tokens 16 lanes (4 blocks per step: 1, 2 and 5 steps); both
    # must give a token the same bits, and the batched call must pass the oracle gate
    ffn, ne, tk = 256, 16, 4
    bank = synth.moe_bank(60 + hidden // 256, ne, hidden, ffn)
    logits = synth.moe_logits(61, 4, ne)
    logits[3] = logits[1]                           # tokens 1 and 3 share all experts
    x = synth.bf16_normal(62, (4, hidden))
    y4, ids4, *_ = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    yr, idr, _ = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids4, idr)
    assert oracle.floored_rel_err(y4, yr) <= GEMV_TOL
    for t in range(4):
        y1, ids1, *_ = _run(q, dev, bank, logits[t:t + 1], x[t:t + 1], hidden, ffn, ne, tk)
        assert np.array_equal(ids1[0], ids4[t])
        assert np.array_equal(y1[0].view(np.uint32), y4[t].view(np.uint32)), t


def test_moe_deterministic(q, dev):
    hidden, ffn, ne, tk = 2048, 768, 128, 8
    bank = synth.moe_bank(32, ne, hidden, ffn)
    logits = synth.moe_logits(32, 4, ne)
    x = synth.bf16_normal(33, (4, hidden))
    a = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    b = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])


def test_moe_tied_logits_pick_lower_ids(q, dev):
    ne, tk = 32, 4
    logits = np.full((2, ne), -1.0, dtype=np.float32)
    logits[0, [30, 4, 9, 1, 17]] = 2.0             # five tied maxima -> 1, 4, 9, 17
    logits[1, :] = 0.5                              # all tied -> 0, 1, 2, 3
    _, ids, *_ = _check(q, dev, 40, 2, hidden=256, ffn=256, ne=ne, tk=tk, logits=logits)
    assert ids.tolist() == [[1, 4, 9, 17], [0, 1, 2, 3]]


@pytest.mark.parametrize("ne,tk,t", [(8, 8, 2), (256, 8, 4), (65, 3, 3), (2, 1, 1)])
def test_moe_expert_counts(q, dev, ne, tk, t):
    _check(q, dev, 50 + ne, t, hidden=256, ffn=512, ne=ne, tk=tk)
