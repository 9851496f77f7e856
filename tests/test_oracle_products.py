"""Pins for the oracle's products: GEMV, routed-expert MoE and prefill.

CPU only. The GEMV is checked against exact rational arithmetic on tiny shapes
and against closed forms; the MoE against an independent weighted sum of dense
per-expert products, hand-set routings and Python's own sort; the prefill
against identity rows and the bf16 rounding bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------- GEMV

def _exact_dot_rows(w64, x64):
    """Exact rational W @ x^T for small shapes (every value is a binary64 dyadic)."""
    wf = [[Fraction(float(v)) for v in row] for row in w64]
    out = []
    for xr in np.atleast_2d(x64):
        xf = [Fraction(float(v)) for v in xr]
        out.append([sum((a * b for a, b in zip(row, xf)), Fraction(0)) for row in wf])
    return out


@pytest.mark.parametrize("n_rows,k,m", [(3, 256, 1), (2, 512, 4), (5, 256, 3)])
def test_q4_k_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.q4_k_weights(31 + m, n_rows, k)
    x = synth.bf16_normal(41 + m, (m, k))
    y = oracle.qmv_q4_k(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_q4_k(raw, n_rows, k), oracle.bf16_bits_to_f64(x))
    assert y.shape == (m, n_rows)
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("n_rows,k,m", [(3, 64, 1), (4, 96, 2)])
def test_q8_0_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.q8_0_weights(51, n_rows, k)
    x = synth.f32_normal(52, (m, k))
    y = oracle.qmv_q8_0(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_q8_0(raw, n_rows, k), x.astype(np.float64))
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("n_rows,k,m", [(3, 256, 1), (2, 512, 4)])
def test_iq4_xs_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.iq4_xs_weights(71 + m, n_rows, k)
    x = synth.bf16_normal(72 + m, (m, k))
    y = oracle.qmv_iq4_xs(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_iq4_xs(raw, n_rows, k), oracle.bf16_bits_to_f64(x))
    assert y.shape == (m, n_rows)
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("n_rows,k,m", [(3, 256, 1), (2, 512, 4)])
def test_q5_k_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.q5_k_weights(81 + m, n_rows, k)
    x = synth.bf16_normal(82 + m, (m, k))
    y = oracle.qmv_q5_k(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_q5_k(raw, n_rows, k), oracle.bf16_bits_to_f64(x))
    assert y.shape == (m, n_rows)
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("n_rows,k,m", [(3, 256, 1), (2, 512, 4)])
def test_q6_k_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.q6_k_weights(91 + m, n_rows, k)
    x = synth.bf16_normal(92 + m, (m, k))
    y = oracle.qmv_q6_k(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_q6_k(raw, n_rows, k), oracle.bf16_bits_to_f64(x))
    assert y.shape == (m, n_rows)
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


@pytest.mark.parametrize("n_rows,k,m", [(3, 64, 1), (2, 256, 4), (4, 96, 3)])
def test_q4_0_gemv_matches_exact_rational(n_rows, k, m):
    raw = synth.q4_0_weights(61 + m, n_rows, k)
    x = synth.bf16_normal(62 + m, (m, k))
    y = oracle.qmv_q4_0(raw, x, n_rows, k)
    exact = _exact_dot_rows(oracle.dequant_q4_0(raw, n_rows, k), oracle.bf16_bits_to_f64(x))
    assert y.shape == (m, n_rows)
    for r in range(m):
        for n in range(n_rows):
            e = exact[r][n]
            assert abs(Fraction(float(y[r, n])) - e) <= abs(e) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 30)


def test_q4_0_gemv_half_block_closed_form(golden_dir):
    # x = 1 on the low-nibble half (weights 0..15) or the high-nibble half
    # (16..31): y = d * (sum of that half's nibbles - 128), from the stated fields
    with open(os.path.join(golden_dir, "q4_0_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        raw = bytes.fromhex(blk["hex"])
        d = oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        for half in (0, 1):
            x = np.zeros((1, 32), dtype=np.uint16)
            x[0, 16 * half:16 * half + 16] = 0x3F80
            y = oracle.qmv_q4_0(raw, x, 1, 32)[0, 0]
            assert y == d * (sum(blk["q"][16 * half:16 * half + 16]) - 128), (blk["name"], half)


def test_q6_k_gemv_constant_over_sixteen_weights_closed_form(golden_dir):
    # x = 1 on weights 16i .. 16i + 15 only: y = d sc_i sum(q), from the stated fields
    with open(os.path.join(golden_dir, "q6_k_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        raw = bytes.fromhex(blk["hex"])
        d = oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        for i in range(16):
            x = np.zeros((1, 256), dtype=np.uint16)
            x[0, 16 * i:16 * i + 16] = 0x3F80
            y = oracle.qmv_q6_k(raw, x, 1, 256)[0, 0]
            assert y == d * blk["sc"][i] * sum(blk["q"][16 * i:16 * i + 16]), (blk["name"], i)


def test_q5_k_gemv_constant_over_one_subblock_closed_form(golden_dir):
    # x = 1 on sub-block j only: y = d sc_j sum(q over j) - 32 dmin m_j, from the stated fields
    with open(os.path.join(golden_dir, "q5_k_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        raw = bytes.fromhex(blk["hex"])
        d = oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        dmin = oracle.fp16_bits_to_f64(np.array([blk["dmin_bits"]]))[0]
        for j in range(8):
            x = np.zeros((1, 256), dtype=np.uint16)
            x[0, 32 * j:32 * j + 32] = 0x3F80
            y = oracle.qmv_q5_k(raw, x, 1, 256)[0, 0]
            qsum = sum(blk["q"][32 * j:32 * j + 32])
            assert y == d * blk["sc"][j] * qsum - 32 * dmin * blk["m"][j], (blk["name"], j)


def test_gemv_unit_vector_selects_a_column():
    n_rows, k = 7, 512
    raw = synth.q4_k_weights(61, n_rows, k)
    w = oracle.dequant_q4_k(raw, n_rows, k)
    for col in (0, 1, 31, 32, 255, 256, 300, 511):
        x = np.zeros((1, k), dtype=np.uint16)
        x[0, col] = 0x3F80                                   # bf16 1.0
        assert np.array_equal(oracle.qmv_q4_k(raw, x, n_rows, k)[0], w[:, col])


def test_gemv_constant_over_one_subblock_closed_form(golden_dir):
    with open(os.path.join(golden_dir, "q4_k_handbuilt.json")) as f:
        blocks = json.load(f)["blocks"]
    for blk in blocks:
        raw = bytes.fromhex(blk["hex"])
        d = oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        dmin = oracle.fp16_bits_to_f64(np.array([blk["dmin_bits"]]))[0]
        for j in range(8):
            x = np.zeros((1, 256), dtype=np.uint16)
            x[0, 32 * j:32 * j + 32] = 0x3F80
            y = oracle.qmv_q4_k(raw, x, 1, 256)[0, 0]
            qsum = sum(blk["q"][32 * j:32 * j + 32])
            assert y == d * blk["sc"][j] * qsum - 32 * dmin * blk["m"][j], (blk["name"], j)


def test_gemv_rows_are_independent():
    # y row r depends only on x row r: a multi-row product equals the stacked 1-row ones
    raw = synth.q4_k_weights(62, 9, 768)
    x = synth.bf16_normal(63, (4, 768))
    y = oracle.qmv_q4_k(raw, x, 9, 768)
    for r in range(4):
        assert np.array_equal(y[r], oracle.qmv_q4_k(raw, x[r:r + 1], 9, 768)[0])


def test_floored_rel_err_definition():
    ref = np.array([[100.0, 1.0, 0.0, -0.01]])
    # tau = 0.1: errors 0.2 on 100 -> 2e-3; 0.001 on 1 -> 1e-3; 1e-4 on 0 -> 1e-3; 0 on -0.01
    y = ref + np.array([[0.2, 0.001, 1e-4, 0.0]])
    assert abs(oracle.floored_rel_err(y, ref) - 2e-3) < 1e-15


# ---------------------------------------------------------------- routing + MoE

def test_route_equal_logits_give_equal_weights_and_lowest_ids():
    logits = np.zeros((1, 128), dtype=np.float32)
    ids, w = oracle.route_top_k(logits, 8)
    assert list(ids[0]) == list(range(8))
    assert np.all(w == 0.125)


def test_route_ties_resolve_to_lower_id():
    logits = np.full((1, 128), -1.0, dtype=np.float32)
    logits[0, [100, 5, 77, 3, 120, 64, 9, 50, 51, 2]] = 2.0     # ten tied maxima
    ids, w = oracle.route_top_k(logits, 8)
    assert list(ids[0]) == [2, 3, 5, 9, 50, 51, 64, 77]
    assert np.all(w == 0.125)


def test_route_matches_python_sort_and_closed_form_softmax():
    logits = synth.moe_logits(71, 16, 128)
    ids, w = oracle.route_top_k(logits, 8)
    for t in range(16):
        lt = [float(v) for v in logits[t]]
        expect = sorted(range(128), key=lambda e: (-lt[e], e))[:8]
        assert list(ids[t]) == expect
        # softmax over all 128, then renormalised over the 8 selected
        p = np.exp(np.array(lt) - max(lt))
        p /= p.sum()
        ren = p[expect] / p[expect].sum()
        assert np.allclose(w[t], ren, rtol=1e-13, atol=0)
        assert abs(w[t].sum() - 1.0) < 1e-15
        assert np.all(np.diff(w[t]) <= 0)


def test_route_hand_set_logits():
    logits = (np.arange(128, dtype=np.float32) / 8).reshape(1, 128)
    ids, w = oracle.route_top_k(logits, 8)
    assert list(ids[0]) == list(range(127, 119, -1))
    e = np.exp(-np.arange(8) / 8)
    assert np.allclose(w[0], e / e.sum(), rtol=1e-14, atol=0)


def test_gather_pairs_sorted_by_expert_then_token():
    ids = np.array([[5, 1, 9], [1, 7, 5], [9, 2, 1]])
    assert oracle.gather_pairs(ids).tolist() == [[1, 0], [1, 1], [1, 2], [2, 2], [5, 0], [5, 1], [7, 1], [9, 0], [9, 2]]


def test_silu_closed_forms():
    from scipy.special import expit
    g = np.linspace(-30, 30, 601)
    assert np.allclose(oracle.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([1.0]))[0] == pytest.approx(1 / (1 + np.exp(-1.0)), rel=1e-15)


def _small_moe(seed, t_count, hidden=256, ffn=256, n_exp=16, top_k=4):
    gate, up, down = synth.moe_bank(seed, n_exp, hidden, ffn)
    logits = synth.moe_logits(seed, t_count, n_exp)
    x = synth.bf16_normal(seed + 1, (t_count, hidden))
    return gate, up, down, logits, x, hidden, ffn, n_exp, top_k


def test_moe_equals_weighted_sum_of_dense_expert_products():
    gate, up, down, logits, x, hidden, ffn, n_exp, top_k = _small_moe(81, 3)
    y, ids, w = oracle.moe_q4_k(gate, up, down, logits, x, hidden, ffn, n_exp, top_k)
    from scipy.special import expit
    xs = oracle.bf16_bits_to_f64(x)
    for t in range(3):
        acc = np.zeros(hidden)
        for j in range(top_k):
            e = int(ids[t, j])
            wg = oracle.dequant_q4_k(oracle.expert_matrix(gate, e, ffn, hidden), ffn, hidden)
            wu = oracle.dequant_q4_k(oracle.expert_matrix(up, e, ffn, hidden), ffn, hidden)
            wd = oracle.dequant_q4_k(oracle.expert_matrix(down, e, hidden, ffn), hidden, ffn)
            g = np.array([np.dot(wg[i], xs[t]) for i in range(ffn)])
            u = np.array([np.dot(wu[i], xs[t]) for i in range(ffn)])
            h = g * expit(g) * u
            acc += w[t, j] * np.array([np.dot(wd[i], h) for i in range(hidden)])
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())


def test_moe_expert_bank_layout_is_expert_major():
    gate, up, down, *_ = _small_moe(82, 1)
    size = 256 * (256 // 256) * 144
    assert np.array_equal(oracle.expert_matrix(gate, 3, 256, 256), gate[3 * size:4 * size])
    assert oracle.expert_matrix(down, 15, 256, 256).size == size


def test_moe_token_output_independent_of_batch():
    gate, up, down, logits, x, hidden, ffn, n_exp, top_k = _small_moe(83, 3)
    y3, ids3, _ = oracle.moe_q4_k(gate, up, down, logits, x, hidden, ffn, n_exp, top_k)
    for t in range(3):
        y1, ids1, _ = oracle.moe_q4_k(gate, up, down, logits[t:t + 1], x[t:t + 1], hidden, ffn, n_exp, top_k)
        assert np.array_equal(ids1[0], ids3[t])
        assert np.allclose(y1[0], y3[t], rtol=1e-13, atol=0)


def test_moe_iq4_xs_equals_weighted_sum_of_dense_expert_products():
    # IQ4_XS experts: every product written out dot by dot from the exact weights
    hidden, ffn, n_exp, top_k = 256, 256, 8, 3
    gate, up, down = synth.moe_bank_iq4_xs(84, n_exp, hidden, ffn)
    logits = synth.moe_logits(84, 2, n_exp)
    x = synth.bf16_normal(85, (2, hidden))
    y, ids, w = oracle.moe_iq4_xs(gate, up, down, logits, x, hidden, ffn, n_exp, top_k)
    from scipy.special import expit
    xs = oracle.bf16_bits_to_f64(x)
    for t in range(2):
        acc = np.zeros(hidden)
        for j in range(top_k):
            e = int(ids[t, j])
            size = ffn * (hidden // 256) * 136
            wg = oracle.dequant_iq4_xs(gate[e * size:(e + 1) * size], ffn, hidden)
            wu = oracle.dequant_iq4_xs(up[e * size:(e + 1) * size], ffn, hidden)
            wd = oracle.dequant_iq4_xs(down[e * size:(e + 1) * size], hidden, ffn)
            g = np.array([np.dot(wg[i], xs[t]) for i in range(ffn)])
            u = np.array([np.dot(wu[i], xs[t]) for i in range(ffn)])
            h = g * expit(g) * u
            acc += w[t, j] * np.array([np.dot(wd[i], h) for i in range(hidden)])
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())


def test_moe_iq4_xs_single_expert_is_the_dense_ffn():
    # top_k = 1: the routing weight is exactly 1 and y is one expert's FFN
    hidden, ffn, n_exp = 256, 512, 4
    gate, up, down = synth.moe_bank_iq4_xs(86, n_exp, hidden, ffn)
    logits = np.full((1, n_exp), -3.0, dtype=np.float32)
    logits[0, 2] = 1.0
    x = synth.bf16_normal(87, (1, hidden))
    y, ids, w = oracle.moe_iq4_xs(gate, up, down, logits, x, hidden, ffn, n_exp, 1)
    assert ids.tolist() == [[2]] and w.tolist() == [[1.0]]
    size = ffn * (hidden // 256) * 136
    xs = oracle.bf16_bits_to_f64(x)[0]
    g = oracle.qmv_iq4_xs(gate[2 * size:3 * size], x, ffn, hidden)[0]
    u = oracle.qmv_iq4_xs(up[2 * size:3 * size], x, ffn, hidden)[0]
    h = g / (1 + np.exp(-g)) * u
    wd = oracle.dequant_iq4_xs(down[2 * size:3 * size], hidden, ffn)
    assert np.allclose(y[0], wd @ h, rtol=1e-13, atol=0)
    assert np.isfinite(xs).all()


def test_moe_iq4_xs_bank_layout_is_expert_major():
    gate, up, down = synth.moe_bank_iq4_xs(88, 4, 256, 512)
    size = 512 * 1 * 136
    assert gate.size == 4 * size and down.size == 4 * 256 * 2 * 136
    assert np.array_equal(oracle.expert_matrix(gate, 3, 512, 256, 136), gate[3 * size:4 * size])
    assert oracle.expert_matrix(down, 1, 256, 512, 136).size == 256 * 2 * 136


# ---------------------------------------------------------------- prefill

def test_prefill_identity_rows_reproduce_weights():
    n_rows, k = 6, 512
    raw = synth.q4_k_weights(91, n_rows, k)
    cols = [0, 17, 255, 256, 400, 511]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for r, c in enumerate(cols):
        x[r, c] = 0x3F80
    y, yb = oracle.prefill_q4_k(raw, x, n_rows, k)
    w = oracle.dequant_q4_k(raw, n_rows, k)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_q4_k_bf16_bits(raw, n_rows, k))
    for r, c in enumerate(cols):
        assert np.array_equal(y[r], w[:, c])
        assert np.array_equal(yb[r], wb[:, c])


def test_prefill_rows_equal_gemv():
    raw = synth.q4_k_weights(92, 33, 768)
    x = synth.bf16_normal(93, (5, 768))
    y, _ = oracle.prefill_q4_k(raw, x, 33, 768)
    assert np.array_equal(y, oracle.qmv_q4_k(raw, x, 33, 768))


def test_bf16_weight_tile_error_bound():
    # RN_bf16(RN_fp32(w)) is within one bf16 half-ulp plus one fp32 half-ulp of w
    raw = synth.q4_k_weights(94, 64, 1024)
    w = oracle.dequant_q4_k(raw, 64, 1024)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_q4_k_bf16_bits(raw, 64, 1024))
    bound = np.abs(w) * (2.0 ** -8 + 2.0 ** -24) * (1 + 2.0 ** -7)
    assert np.all(np.abs(wb - w) <= bound)


def test_prefill_bf16_weight_error_is_the_predicted_size():
    # With bf16 weight tiles the product differs from the exact one by ~1.6e-3
    # (normwise); the test bounds it so a wrong rounding path would show.
    raw = synth.q4_k_weights(95, 128, 2048)
    x = synth.bf16_normal(96, (32, 2048))
    y, yb = oracle.prefill_q4_k(raw, x, 128, 2048)
    e = oracle.frobenius_rel_err(yb, y)
    assert 1.0e-3 < e < 2.0e-3
