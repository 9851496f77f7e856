"""GPU parity of the routed-expert MoE prefill (grouped matrix-core products) against the fp64 oracle.

Gates: top-k expert ids bit-exact; routing weights within fp32 rounding of the
oracle's; outputs within the floored 2e-3 relative gate; a token's output does
not depend on the other tokens of the call (a prefix of the prompt run alone
gives bit-identical rows); run-to-run bitwise determinism; output and workspace
guards untouched. The cases span one partial chunk of 16 pairs, experts with
several chunks, k = 1, k = n_experts (every token takes every expert), and a
35B-A3B-like layer (hidden 2048, 128 experts, top-8), and that layer at 512
tokens with sampled tokens checked. The pair counts reach one, two and four
weight tiles per wave, and the 32-pair gate/up form; hidden 2560 at 2048 pairs
takes the 16-pair form at four tiles per wave (32 rows of x exceed the LDS
stage there).
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


def _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk):
    t = x.shape[0]
    y, ybuf = guarded((t, hidden), torch.float32, dev)
    need = q.qmv_q4_k_moe_prefill_workspace(t, hidden, ffn, ne, tk)
    assert need > 0
    ws_buf = torch.full((need + 512,), 0xA5, dtype=torch.uint8, device=dev)
    ws = ws_buf[256:256 + need]
    y, ids, wts = q.qmv_q4_k_moe_prefill(*bank_d, to_dev(logits, dev), to_dev(x, dev), hidden, ffn, ne, tk, y=y,
                                         ws=ws)
    torch.cuda.synchronize()
    assert guards_intact(ybuf)
    assert bool((ws_buf[:256] == 0xA5).all() and (ws_buf[256 + need:] == 0xA5).all())
    return host(y), host(ids), host(wts)


CASES = [(3, 512, 256, 16, 4, 1), (9, 512, 256, 16, 4, 2), (37, 256, 512, 8, 2, 3), (200, 512, 256, 32, 8, 5),
         (11, 256, 256, 8, 1, 6), (5, 256, 256, 4, 4, 7), (6, 2048, 768, 128, 8, 4), (256, 512, 256, 32, 8, 8),
         (256, 2560, 256, 8, 8, 9)]


@pytest.mark.parametrize("t,hidden,ffn,ne,tk,seed", CASES)
def test_moe_prefill_parity(q, dev, t, hidden, ffn, ne, tk, seed):
    bank = synth.moe_bank(seed, ne, hidden, ffn)
    bank_d = tuple(to_dev(b, dev) for b in bank)
    logits = synth.moe_logits(seed, t, ne)
    x = synth.bf16_normal(seed + 1, (t, hidden))
    y, ids, wts = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    yr, idr, wr = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y, yr)
    assert err <= GEMV_TOL, err


def test_moe_prefill_full_layer_sampled_tokens(q, dev):
    # the timed workload: 512 tokens through the 35B-A3B layer; the oracle takes five sampled tokens
    t, hidden, ffn, ne, tk = 512, 2048, 768, 128, 8
    bank = synth.moe_bank(21, ne, hidden, ffn)
    bank_d = tuple(to_dev(b, dev) for b in bank)
    logits = synth.moe_logits(21, t, ne)
    x = synth.bf16_normal(22, (t, hidden))
    y, ids, wts = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    assert np.isfinite(y).all()
    pick = np.array([0, 137, 255, 300, 511])
    yr, idr, wr = oracle.moe_q4_k(*bank, logits[pick], x[pick], hidden, ffn, ne, tk)
    assert np.array_equal(ids[pick], idr)
    assert np.allclose(wts[pick], wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y[pick], yr)
    assert err <= GEMV_TOL, err


def test_moe_prefill_rows_do_not_depend_on_the_other_tokens(q, dev):
    t, hidden, ffn, ne, tk = 40, 512, 256, 16, 4
    bank_d = tuple(to_dev(b, dev) for b in synth.moe_bank(13, ne, hidden, ffn))
    logits = synth.moe_logits(13, t, ne)
    x = synth.bf16_normal(14, (t, hidden))
    y_all, _, _ = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    for n in (1, 17):
        y_pre, _, _ = _run(q, dev, bank_d, logits[:n], x[:n], hidden, ffn, ne, tk)
        assert np.array_equal(y_pre.view(np.uint32), y_all[:n].view(np.uint32)), n


def test_moe_prefill_deterministic(q, dev):
    t, hidden, ffn, ne, tk = 64, 512, 256, 32, 8
    bank_d = tuple(to_dev(b, dev) for b in synth.moe_bank(11, ne, hidden, ffn))
    logits = synth.moe_logits(11, t, ne)
    x = synth.bf16_normal(12, (t, hidden))
    a = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    b = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])


@pytest.mark.parametrize("t,tk", [(300, 4), (600, 4)])
def test_moe_prefill_all_tokens_on_the_same_experts(q, dev, t, tk):
    # tied logits: every token picks experts 0 .. k-1 (ties to the lower id), so each of them holds
    # t pairs in many chunks; 1200 pairs run the 16-pair gate/up, 2400 the 32-pair one
    hidden, ffn, ne = 512, 256, 16
    bank = synth.moe_bank(31, ne, hidden, ffn)
    bank_d = tuple(to_dev(b, dev) for b in bank)
    logits = np.zeros((t, ne), dtype=np.float32)
    x = synth.bf16_normal(32, (t, hidden))
    y, ids, wts = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, np.tile(np.arange(tk, dtype=ids.dtype), (t, 1)))
    yr, idr, wr = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y, yr)
    assert err <= GEMV_TOL, err


def test_moe_prefill_many_tokens(q, dev):
    # 4096 tokens, top-2 of 8 experts: about 1024 pairs per expert, 32 chunks of 32 each
    t, hidden, ffn, ne, tk = 4096, 256, 256, 8, 2
    bank = synth.moe_bank(33, ne, hidden, ffn)
    bank_d = tuple(to_dev(b, dev) for b in bank)
    logits = synth.moe_logits(33, t, ne)
    x = synth.bf16_normal(34, (t, hidden))
    y, ids, wts = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    yr, idr, wr = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y, yr)
    assert err <= GEMV_TOL, err
