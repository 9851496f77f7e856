"""GPU parity of the IQ4_XS routed-expert MoE entry point against the fp64 oracle.

Gates (as for the Q4_K form): top-k expert ids and the (expert, token) gather
list bit-exact; routing weights within fp32 rounding of the oracle's; outputs
within the floored 2e-3 relative gate; a token's output bit-identical alone
(T=1) and in a batch of 3; run-to-run bitwise determinism; output and
workspace guards untouched. Shapes cover the 35B-A3B layer (hidden 2048, 128
experts of F=768, top-8), a row shorter than one 16-lane pass (hidden 256),
several super-blocks per W_down row, and expert counts below, at and above k.
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
    need = q.qmv_iq4_xs_moe_workspace(t, hidden, ffn, ne, tk)
    ws_buf = torch.full((need + 512,), 0xA5, dtype=torch.uint8, device=dev)
    ws = ws_buf[256:256 + need]
    y, ids, wts, pairs = q.qmv_iq4_xs_moe(to_dev(gate, dev), to_dev(up, dev), to_dev(down, dev),
                                          to_dev(logits, dev), to_dev(x, dev), hidden, ffn, ne, tk, y=y, ws=ws)
    torch.cuda.synchronize()
    assert guards_intact(ybuf)
    assert bool((ws_buf[:256] == 0xA5).all() and (ws_buf[256 + need:] == 0xA5).all())
    return host(y), host(ids), host(wts), host(pairs)


def _check(q, dev, seed, t, hidden, ffn, ne, tk, logits=None):
    bank = synth.moe_bank_iq4_xs(seed, ne, hidden, ffn)
    if logits is None:
        logits = synth.moe_logits(seed, t, ne)
    x = synth.bf16_normal(seed + 1, (t, hidden))
    y, ids, wts, pairs = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    yr, idr, wr = oracle.moe_iq4_xs(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.array_equal(pairs, oracle.gather_pairs(idr))
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    err = oracle.floored_rel_err(y, yr)
    assert err <= GEMV_TOL, err
    return y, ids


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_iq4_xs_moe_small_bank_parity(q, dev, t):
    _check(q, dev, 110 + t, t, hidden=512, ffn=256, ne=16, tk=4)


@pytest.mark.parametrize("t", [1, 3, 4])
def test_iq4_xs_moe_35b_a3b_layer_parity(q, dev, t):
    _check(q, dev, 120 + t, t, hidden=2048, ffn=768, ne=128, tk=8)


@pytest.mark.parametrize("hidden,ffn,ne,tk,t", [(256, 512, 8, 8, 2), (768, 1024, 65, 3, 3), (256, 256, 2, 1, 1),
                                                (1280, 256, 256, 8, 4)])
def test_iq4_xs_moe_shapes_and_expert_counts(q, dev, hidden, ffn, ne, tk, t):
    _check(q, dev, 130 + ne, t, hidden=hidden, ffn=ffn, ne=ne, tk=tk)


def test_iq4_xs_moe_token_bit_identical_alone_and_batched(q, dev):
    hidden, ffn, ne, tk = 2048, 768, 128, 8
    bank = synth.moe_bank_iq4_xs(140, ne, hidden, ffn)
    logits = synth.moe_logits(140, 3, ne)
    logits[1] = logits[0]                           # tokens 0 and 1 share all experts
    logits[2, :64] = logits[0, :64]                 # token 2 shares some
    x = synth.bf16_normal(141, (3, hidden))
    y3, ids3, *_ = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    for t in range(3):
        y1, ids1, *_ = _run(q, dev, bank, logits[t:t + 1], x[t:t + 1], hidden, ffn, ne, tk)
        assert np.array_equal(ids1[0], ids3[t])
        assert np.array_equal(y1[0].view(np.uint32), y3[t].view(np.uint32)), t


@pytest.mark.parametrize("hidden", [256, 1280, 4608])
def test_iq4_xs_moe_token_bit_identical_alone_and_batched_ragged_rows(q, dev, hidden):
    # rows of 1, 5 and 18 super-blocks, so that the one-token lane width (32 lanes per row) and
    # the several-token one (16) both end on a partial pass; a token's bits must not depend on the
    # token count, and the batched call must pass the oracle gate
    ffn, ne, tk = 256, 16, 4
    bank = synth.moe_bank_iq4_xs(160 + hidden // 256, ne, hidden, ffn)
    logits = synth.moe_logits(161, 4, ne)
    logits[3] = logits[1]                           # tokens 1 and 3 share all experts
    x = synth.bf16_normal(162, (4, hidden))
    y4, ids4, *_ = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    yr, idr, _ = oracle.moe_iq4_xs(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids4, idr)
    assert oracle.floored_rel_err(y4, yr) <= GEMV_TOL
    for t in range(4):
        y1, ids1, *_ = _run(q, dev, bank, logits[t:t + 1], x[t:t + 1], hidden, ffn, ne, tk)
        assert np.array_equal(ids1[0], ids4[t])
        assert np.array_equal(y1[0].view(np.uint32), y4[t].view(np.uint32)), t


def test_iq4_xs_moe_deterministic(q, dev):
    hidden, ffn, ne, tk = 2048, 768, 128, 8
    bank = synth.moe_bank_iq4_xs(142, ne, hidden, ffn)
    logits = synth.moe_logits(142, 4, ne)
    x = synth.bf16_normal(143, (4, hidden))
    a = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    b = _run(q, dev, bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])


def test_iq4_xs_moe_matches_its_experts_run_as_gemvs(q, dev):
    # top-1 with a clear winner: y is W_down h of one expert, h from the gate/up GEMVs
    hidden, ffn, ne = 2048, 768, 8
    gate, up, down = synth.moe_bank_iq4_xs(144, ne, hidden, ffn)
    logits = np.full((1, ne), -2.0, dtype=np.float32)
    logits[0, 5] = 3.0
    x = synth.bf16_normal(145, (1, hidden))
    y, ids, *_ = _run(q, dev, (gate, up, down), logits, x, hidden, ffn, ne, 1)
    assert ids.tolist() == [[5]]
    size = ffn * (hidden // 256) * 136
    g = oracle.qmv_iq4_xs(gate[5 * size:6 * size], x, ffn, hidden)[0]
    u = oracle.qmv_iq4_xs(up[5 * size:6 * size], x, ffn, hidden)[0]
    h = g / (1 + np.exp(-g)) * u
    ref = oracle.dequant_iq4_xs(down[5 * size:6 * size], hidden, ffn) @ h
    assert oracle.floored_rel_err(y, ref[None]) <= GEMV_TOL
