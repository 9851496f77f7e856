"""GPU parity of the routed-expert MoE prefill entry point against the fp64 oracle.

The entry point runs a prompt's tokens as consecutive groups of up to four
through the routed-expert kernels. Gates: top-k expert ids bit-exact; routing
weights within fp32 rounding of the oracle's; outputs within the floored 2e-3
relative gate; every token's output bit-identical to the routed-expert entry
point on that token alone (one numerical program per request); run-to-run
bitwise determinism; output and workspace guards untouched. Token counts span
one partial group, several groups with a partial last one, and a 35B-A3B-like
layer (hidden 2048, 128 experts, top-8).
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
    ws_buf = torch.full((need + 512,), 0xA5, dtype=torch.uint8, device=dev)
    ws = ws_buf[256:256 + need]
    y, ids, wts = q.qmv_q4_k_moe_prefill(*bank_d, to_dev(logits, dev), to_dev(x, dev), hidden, ffn, ne, tk, y=y,
                                         ws=ws)
    torch.cuda.synchronize()
    assert guards_intact(ybuf)
    assert bool((ws_buf[:256] == 0xA5).all() and (ws_buf[256 + need:] == 0xA5).all())
    return host(y), host(ids), host(wts)


@pytest.mark.parametrize("t,hidden,ffn,ne,tk,seed", [(3, 512, 256, 16, 4, 1), (9, 512, 256, 16, 4, 2),
                                                     (37, 256, 512, 8, 2, 3), (6, 2048, 768, 128, 8, 4)])
def test_moe_prefill_parity_and_alone_bit_identity(q, dev, t, hidden, ffn, ne, tk, seed):
    bank = synth.moe_bank(seed, ne, hidden, ffn)
    bank_d = tuple(to_dev(b, dev) for b in bank)
    logits = synth.moe_logits(seed, t, ne)
    x = synth.bf16_normal(seed + 1, (t, hidden))
    y, ids, wts = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    yr, idr, wr = oracle.moe_q4_k(*bank, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(ids, idr)
    assert np.allclose(wts, wr, rtol=2e-6, atol=0)
    assert oracle.floored_rel_err(y, yr) <= GEMV_TOL
    for r in range(t):
        y1, _, _, _ = q.qmv_q4_k_moe(*bank_d, to_dev(logits[r:r + 1], dev), to_dev(x[r:r + 1], dev), hidden, ffn, ne,
                                     tk, routing=False)
        assert np.array_equal(host(y1)[0].view(np.uint32), y[r].view(np.uint32)), r


def test_moe_prefill_deterministic(q, dev):
    t, hidden, ffn, ne, tk = 64, 512, 256, 32, 8
    bank_d = tuple(to_dev(b, dev) for b in synth.moe_bank(11, ne, hidden, ffn))
    logits = synth.moe_logits(11, t, ne)
    x = synth.bf16_normal(12, (t, hidden))
    a = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    b = _run(q, dev, bank_d, logits, x, hidden, ffn, ne, tk)
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1], b[1])
