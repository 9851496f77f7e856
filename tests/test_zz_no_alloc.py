"""The allocation-free routed-expert entry point (qmv_q4_k_moe_noalloc), called
through the C ABI, against qmv_q4_k_moe with a caller workspace.

Both run the same kernels, so the outputs, routing ids, weights and gather list
must agree bit for bit; two calls in a row, the second with a smaller input (3
tokens on the 35B-A3B layer, then 1 token on a smaller bank), check that the
fixed scratch array carries nothing from one call into the next. The first call
is also held to the oracle's gates, so agreement is not agreement on garbage.
"""

import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import GEMV_TOL, device, guarded, guards_intact, host, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _both(q, dev, seed, t, hidden, ffn, ne, tk):
    gate, up, down = synth.moe_bank(seed, ne, hidden, ffn)
    logits = synth.moe_logits(seed, t, ne)
    x = synth.bf16_normal(seed + 1, (t, hidden))
    g, u, d, lg, xd = (to_dev(a, dev) for a in (gate, up, down, logits, x))
    bank = g.numel()
    outs = []
    for noalloc in (True, False):
        y, ybuf = guarded((t, hidden), torch.float32, dev)
        ids = torch.full((t, tk), -1, dtype=torch.int32, device=dev)
        wts = torch.full((t, tk), float("nan"), dtype=torch.float32, device=dev)
        pairs = torch.full((t * tk, 2), -1, dtype=torch.int32, device=dev)
        if noalloc:
            rc = q.lib.qmv_q4_k_moe_noalloc(_ptr(g), _ptr(u), _ptr(d), bank, _ptr(lg), _ptr(xd), _ptr(y), _ptr(ids),
                                            _ptr(wts), _ptr(pairs), t, hidden, ffn, ne, tk, None)
        else:
            need = q.lib.qmv_q4_k_moe_workspace(t, hidden, ffn, ne, tk)
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            rc = q.lib.qmv_q4_k_moe(_ptr(g), _ptr(u), _ptr(d), bank, _ptr(lg), _ptr(xd), _ptr(y), _ptr(ids),
                                    _ptr(wts), _ptr(pairs), _ptr(ws), need, t, hidden, ffn, ne, tk, None)
        assert rc == 0, (noalloc, rc)
        torch.cuda.synchronize()
        assert guards_intact(ybuf)
        outs.append(tuple(host(v) for v in (y, ids, wts, pairs)))
    (y0, i0, w0, p0), (y1, i1, w1, p1) = outs
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(i0, i1) and np.array_equal(p0, p1)
    assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
    return y0, i0, (gate, up, down), logits, x


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    import gguf_block_quantized_qmv_amd as q
    dev = device()
    # call 1: the 35B-A3B layer at 3 tokens (77,824 bytes of scratch), also against the oracle
    y, ids, bank, logits, x = _both(q, dev, 91, 3, 2048, 768, 128, 8)
    yr, idr, _ = oracle.moe_q4_k(*bank, logits, x, 2048, 768, 128, 8)
    assert np.array_equal(ids, idr)
    assert oracle.floored_rel_err(y, yr) <= GEMV_TOL
    # call 2: one token on a smaller bank (4096 + 4 * 256 * 4 bytes of scratch)
    _both(q, dev, 92, 1, 512, 256, 16, 4)


def test_noalloc_rejects_what_the_workspace_entry_point_rejects():
    import gguf_block_quantized_qmv_amd as q
    dev = device()
    g = torch.zeros(16 * 256 * 2 * 144, dtype=torch.uint8, device=dev)
    lg = torch.zeros((1, 16), dtype=torch.float32, device=dev)
    xd = torch.zeros((1, 512), dtype=torch.int16, device=dev)
    y = torch.zeros((1, 512), dtype=torch.float32, device=dev)
    args = (_ptr(g), _ptr(g), _ptr(g), g.numel(), _ptr(lg), _ptr(xd), _ptr(y), None, None, None)
    assert q.lib.qmv_q4_k_moe_noalloc(*args, 5, 512, 256, 16, 4, None) == -5          # T above 4
    assert q.lib.qmv_q4_k_moe_noalloc(*args[:3], g.numel() - 1, *args[4:], 1, 512, 256, 16, 4, None) == -3


def _noalloc(q, dev, args, y, stream):
    g, u, d, bank, lg, xd, t, hidden, ffn, ne, tk = args
    return q.lib.qmv_q4_k_moe_noalloc(_ptr(g), _ptr(u), _ptr(d), bank, _ptr(lg), _ptr(xd), _ptr(y), None, None, None,
                                      t, hidden, ffn, ne, tk, stream)


def _layer(dev, seed, hidden, ffn, ne, tk):
    gate, up, down = synth.moe_bank(seed, ne, hidden, ffn)
    lg = to_dev(synth.moe_logits(seed, 1, ne), dev)
    xd = to_dev(synth.bf16_normal(seed + 1, (1, hidden)), dev)
    g, u, d = (to_dev(a, dev) for a in (gate, up, down))
    return (g, u, d, g.numel(), lg, xd, 1, hidden, ffn, ne, tk)


def test_noalloc_one_token_back_to_back_and_graph_replays():
    """One token at a time, the decode case: five calls in a row on different
    tokens and banks each agree bit for bit with the workspace entry point,
    and so do three replays of a captured call with other calls through the
    same array in between (each replay must rewrite everything it reads)."""
    import gguf_block_quantized_qmv_amd as q
    dev = device()
    shapes = [(2048, 768, 128, 8), (512, 256, 16, 4), (2048, 768, 128, 8), (1024, 512, 64, 6), (2048, 768, 128, 8)]
    for i, shp in enumerate(shapes):
        _both(q, dev, 200 + i, 1, *shp)

    main = _layer(dev, 300, 2048, 768, 128, 8)
    other = _layer(dev, 301, 2048, 768, 128, 8)
    y_ref, _, _, _ = q.qmv_q4_k_moe(*main[:3], main[4], main[5], 2048, 768, 128, 8, routing=False)
    y_other = torch.empty((1, 2048), dtype=torch.float32, device=dev)
    y_graph = torch.full((1, 2048), float("nan"), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert _noalloc(q, dev, main, y_graph, ctypes.c_void_p(s.cuda_stream)) == 0   # warm-up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        assert _noalloc(q, dev, main, y_graph, ctypes.c_void_p(s.cuda_stream)) == 0
    for _ in range(3):
        y_graph.fill_(float("nan"))
        assert _noalloc(q, dev, other, y_other, None) == 0   # another token through the same array
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int32), y_ref.view(torch.int32))
