"""The pins must catch plausible mistakes planted in the oracle (CPU only).

Each case rewrites one line of the oracle's source text (a dropped term, a wrong
sign, a wrong index or byte, a transposed operand, a swapped nibble), loads the
result as a separate module, and runs a battery of pins against it. Every
mutant must fail at least one pin; the unmodified oracle must pass all of them.
"""

import inspect
import json
import os
import types

import numpy as np
import pytest

import oracle.gguf_oracle as gg
import synth

SRC = inspect.getsource(gg)

MUTATIONS = {
    "nibbles_swapped": [("= byte & 0x0F", "= byte >> 5"), ("= byte >> 4", "= byte & 0x0F"), ("= byte >> 5", "= byte >> 4")],
    "chunk_order": [("byte = Q[..., 32 * c: 32 * c + 32]", "byte = Q[..., 32 * (3 - c): 32 * (3 - c) + 32]")],
    "sc_from_min_byte": [("sc[..., j] = S[..., j] & 0x3F", "sc[..., j] = S[..., j + 4] & 0x3F")],
    "sc_top_bits_wrong_byte": [("((S[..., j - 4] >> 6) << 4)", "((S[..., j] >> 6) << 4)")],
    "m_top_bits_wrong_byte": [("m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j] >> 6) << 4)",
                               "m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j - 4] >> 6) << 4)")],
    "q5_high_bit_of_other_half": [("((H >> (2 * c)) & 1) << 4", "((H >> (2 * c + 1)) & 1) << 4")],
    "q5_high_bit_weight_eight": [("q[:, :, 64 * c + 32: 64 * c + 64] += ((H >> (2 * c + 1)) & 1) << 4",
                                  "q[:, :, 64 * c + 32: 64 * c + 64] += ((H >> (2 * c + 1)) & 1) << 3")],
    "q6_high_bits_of_next_quarter": [("high = (H[:, :, 32 * h: 32 * h + 32] >> (2 * c)) & 3",
                                      "high = (H[:, :, 32 * h: 32 * h + 32] >> (2 * (c ^ 1))) & 3")],
    "q6_quant_not_centred": [("low + 16 * high - 32", "low + 16 * high - 31")],
    "q6_scale_per_32": [("scale = (d[:, :, None] * sc).repeat(16, axis=2)",
                         "scale = (d[:, :, None] * sc[:, :, ::2]).repeat(32, axis=2)")],
    "m_low_bits_from_low_nibble": [("m[..., j] = (S[..., j + 4] >> 4)", "m[..., j] = (S[..., j + 4] & 0x0F)")],
    "fp16_big_endian": [("(blocks[:, :, 0] | (blocks[:, :, 1] << 8))", "(blocks[:, :, 1] | (blocks[:, :, 0] << 8))")],
    "min_sign_flipped": [("return (scale * q - offset)", "return (scale * q + offset)")],
    "dmin_as_scale": [("scale = (d[:, :, None] * sc)", "scale = (dmin[:, :, None] * sc)")],
    "min_term_dropped": [("return (scale * q - offset)", "return (scale * q)")],
    "subblock_index_shift": [("scale = (d[:, :, None] * sc).repeat(32, axis=2)",
                              "scale = np.roll(d[:, :, None] * sc, 1, axis=2).repeat(32, axis=2)")],
    "q4_0_nibble_halves_swapped": [("q = np.concatenate([qs & 0x0F, qs >> 4], axis=2)",
                                    "q = np.concatenate([qs >> 4, qs & 0x0F], axis=2)")],
    "q4_0_offset_dropped": [("(d[:, :, None] * (q - 8))", "(d[:, :, None] * q)")],
    "q4_0_offset_off_by_one": [("(d[:, :, None] * (q - 8))", "(d[:, :, None] * (q - 7))")],
    "q4_0_interleaved_nibbles": [("q = np.concatenate([qs & 0x0F, qs >> 4], axis=2)",
                                  "q = np.stack([qs & 0x0F, qs >> 4], axis=3).reshape(qs.shape[0], qs.shape[1], 32)")],
    "q8_0_unsigned_quants": [("q = blocks[:, :, 2:].view(np.int8).astype(np.int64)",
                              "q = blocks[:, :, 2:].astype(np.int64)")],
    "gemv_transposed": [("return x2 @ np.asarray(w, dtype=np.float64).T", "return (np.asarray(w, dtype=np.float64) @ x2.T)")],
    "route_ties_to_higher_id": [("order = np.lexsort((expert, -lg[t]))", "order = np.lexsort((-expert, -lg[t]))")],
    "route_on_smallest": [("order = np.lexsort((expert, -lg[t]))", "order = np.lexsort((expert, lg[t]))")],
    "route_not_renormalised": [("wts[t] = e / e.sum()", "wts[t] = e")],
    "silu_wrong_sign": [("return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))")],
    "moe_weight_dropped": [("y[t] += wts[t, j] * (wd @ h)", "y[t] += (wd @ h)")],
    "moe_up_dropped": [("h = silu(wg @ x[t]) * (wu @ x[t])", "h = silu(wg @ x[t])")],
    "bf16_tile_truncates": [("wb = bf16_bits_to_f64(round_f32_to_bf16_bits(round_to_f32(w)))",
                             "wb = bf16_bits_to_f64((round_to_f32(w).view(np.uint32) >> 16).astype(np.uint16))")],
}


def _load(source: str) -> types.ModuleType:
    mod = types.ModuleType("oracle_mutant")
    exec(compile(source, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _golden(name):
    here = os.path.join(os.path.dirname(__file__), "golden", name)
    with open(here) as f:
        return json.load(f)["blocks"]


def _pins(o) -> list:
    """Run a battery of pins against oracle-like module o; return the names that fail."""
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # a mutant that crashes fails the pin too
            failed.append(name)

    def golden_q4():
        for blk in _golden("q4_k_handbuilt.json"):
            w = o.dequant_q4_k(bytes.fromhex(blk["hex"]), 1, 256)[0]
            if not np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]):
                return False
        return True

    def golden_q5():
        for blk in _golden("q5_k_handbuilt.json"):
            w = o.dequant_q5_k(bytes.fromhex(blk["hex"]), 1, 256)[0]
            if not np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]):
                return False
        return True

    def golden_q6():
        for blk in _golden("q6_k_handbuilt.json"):
            w = o.dequant_q6_k(bytes.fromhex(blk["hex"]), 1, 256)[0]
            if not np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]):
                return False
        return True

    def golden_q40():
        for blk in _golden("q4_0_handbuilt.json"):
            w = o.dequant_q4_0(bytes.fromhex(blk["hex"]), 1, 32)[0]
            if not np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]):
                return False
        return True

    def golden_q8():
        for blk in _golden("q8_0_handbuilt.json"):
            w = o.dequant_q8_0(bytes.fromhex(blk["hex"]), 1, 32)[0]
            if not np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]):
                return False
        return True

    def gemv_unit_vectors():
        raw = synth.q4_k_weights(5, 3, 512)
        w = gg.dequant_q4_k(raw, 3, 512)        # reference weights from the unmodified oracle's pins
        x = np.zeros((2, 512), dtype=np.uint16)
        x[0, 7] = 0x3F80
        x[1, 300] = 0x3F80
        y = o.qmv_q4_k(raw, x, 3, 512)
        return y.shape == (2, 3) and np.array_equal(y[0], w[:, 7]) and np.array_equal(y[1], w[:, 300])

    def route_hand_set():
        lg = np.full((1, 32), -1.0, dtype=np.float32)
        lg[0, [30, 4, 9, 1]] = 2.0
        lg[0, 20] = 1.0
        ids, wts = o.route_top_k(lg, 5)
        e = np.exp(np.array([0, 0, 0, 0, -1.0]))
        return list(ids[0]) == [1, 4, 9, 30, 20] and np.allclose(wts[0], e / e.sum(), rtol=1e-14, atol=0)

    def silu_closed_form():
        return abs(o.silu(np.array([2.0]))[0] - 2.0 / (1 + np.exp(-2.0))) < 1e-15

    def moe_dense_sum():
        gate, up, down = synth.moe_bank(7, 8, 256, 256)
        lg = synth.moe_logits(7, 1, 8)
        x = synth.bf16_normal(8, (1, 256))
        y, ids, wts = o.moe_q4_k(gate, up, down, lg, x, 256, 256, 8, 2)
        xs = gg.bf16_bits_to_f64(x)[0]
        acc = np.zeros(256)
        order = sorted(range(8), key=lambda e: (-float(lg[0, e]), e))[:2]
        p = np.exp(lg[0, order].astype(np.float64) - lg[0, order[0]])
        p /= p.sum()
        for e, r in zip(order, p):
            wg = gg.dequant_q4_k(gg.expert_matrix(gate, e, 256, 256), 256, 256)
            wu = gg.dequant_q4_k(gg.expert_matrix(up, e, 256, 256), 256, 256)
            wd = gg.dequant_q4_k(gg.expert_matrix(down, e, 256, 256), 256, 256)
            g = wg @ xs
            acc += r * (wd @ (g / (1 + np.exp(-g)) * (wu @ xs)))
        return np.allclose(y[0], acc, rtol=1e-12, atol=1e-12 * np.abs(acc).max())

    def bf16_tile_ties():
        # exact weights 1 + 2^-8 + 2^-9 (round up) and 1 + 2^-8 (tie -> even -> 1)
        w = np.array([[1 + 2.0 ** -8 + 2.0 ** -9, 1 + 2.0 ** -8]])
        got = o.bf16_bits_to_f64(o.round_f32_to_bf16_bits(o.round_to_f32(w)))
        raw = synth.q4_k_weights(9, 8, 256)
        x = np.zeros((64, 256), dtype=np.uint16)
        x[np.arange(64), np.arange(64)] = 0x3F80          # unit rows e_0 .. e_63
        _, yb = o.prefill_q4_k(raw, x, 8, 256)
        wb_ref = gg.bf16_bits_to_f64(gg.round_f32_to_bf16_bits(gg.round_to_f32(gg.dequant_q4_k(raw, 8, 256))))
        return list(got[0]) == [1 + 2.0 ** -7, 1.0] and np.array_equal(yb, wb_ref[:, :64].T)

    check("golden_q4", golden_q4)
    check("golden_q5", golden_q5)
    check("golden_q6", golden_q6)
    check("golden_q8", golden_q8)
    check("golden_q40", golden_q40)
    check("gemv_unit_vectors", gemv_unit_vectors)
    check("route_hand_set", route_hand_set)
    check("silu_closed_form", silu_closed_form)
    check("moe_dense_sum", moe_dense_sum)
    check("bf16_tile", bf16_tile_ties)
    return failed


def test_unmodified_oracle_passes_the_battery():
    assert _pins(_load(SRC)) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    src = SRC
    for old, new in MUTATIONS[name]:
        assert old in src, f"mutation anchor missing: {old!r}"
        src = src.replace(old, new)
    assert src != SRC
    assert _pins(_load(src)), f"no pin caught the planted mistake {name}"
