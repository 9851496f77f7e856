"""Pins for the oracle's block decoding (Q8_0, Q4_0, Q4_K, Q5_K, Q6_K, IQ4_XS) and scalar formats.

Everything here runs on the CPU. Each check ties the oracle to something other
than itself: hand-built blocks whose values are known by construction
(tests/golden), locality invariants of the byte layout, the pack/unpack
bijection, requantisation round trips and closed-form special values.
"""

import json
import os
import sys

import numpy as np
import pytest

import oracle
import synth

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
from make_handbuilt_blocks import (  # noqa: E402
    IQ4_XS_GRID, pack_iq4_indices, pack_iq4_xs_scales, pack_nibbles, pack_q4_0_quants, pack_q5_high_bits,
    pack_q6_planes, pack_scales_mins)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)["blocks"]


# ---------------------------------------------------------------- scalars

@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x7BFF, 65504.0), (0x0001, 2.0 ** -24),
    (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14), (0x3555, (1 + 0x155 / 1024) * 2.0 ** -2),
    (0x0000, 0.0),
])
def test_fp16_decode_closed_forms(bits, value):
    assert oracle.fp16_bits_to_f64(np.array([bits]))[0] == value


def test_fp16_negative_zero_keeps_sign():
    v = oracle.fp16_bits_to_f64(np.array([0x8000]))[0]
    assert v == 0.0 and np.signbit(v)


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4300, 128.0), (0x0001, 2.0 ** -133), (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127),
])
def test_bf16_decode_closed_forms(bits, value):
    assert oracle.bf16_bits_to_f64(np.array([bits]))[0] == value


def test_bf16_round_nearest_even():
    # ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 -> even (1.0);
    #       1 + 3*2^-8 sits halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -8)], dtype=np.float32)
    got = oracle.bf16_bits_to_f64(oracle.round_f32_to_bf16_bits(vals))
    assert list(got) == [1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0]


def test_synth_bf16_generator_rounds_like_the_library():
    bits = synth.bf16_normal(5, (4096,))
    g = synth.rng(5, 16, 0)
    x = g.standard_normal(size=(4096,), dtype=np.float32)
    assert np.array_equal(bits, oracle.round_f32_to_bf16_bits(x))


# ---------------------------------------------------------------- Q8_0

def test_q8_0_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "q8_0_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, q = oracle.q8_0_fields(raw, 1, 32)
        assert list(q[0, 0]) == blk["q"], blk["name"]
        w = oracle.dequant_q8_0(raw, 1, 32)[0]
        expect = np.array([float.fromhex(v) for v in blk["expect"]])
        assert np.array_equal(w, expect), blk["name"]


def test_q8_0_multi_block_row_major():
    # Row n, block t must come from bytes (n*K/32 + t)*34: build 3 rows x 2 blocks
    # whose scale encodes (n, t) and whose quants encode the in-block index.
    n_rows, k = 3, 64
    raw = bytearray()
    for n in range(n_rows):
        for t in range(2):
            d_bits = 0x3C00 + (n * 2 + t) * 0x400          # 1, 2, 4, 8, 16, 32
            raw += bytes([d_bits & 0xFF, d_bits >> 8]) + bytes(range(32))
    w = oracle.dequant_q8_0(bytes(raw), n_rows, k)
    for n in range(n_rows):
        for t in range(2):
            assert np.array_equal(w[n, 32 * t:32 * t + 32], (2.0 ** (n * 2 + t)) * np.arange(32))


def test_q8_0_requant_round_trip():
    raw = synth.q8_0_weights(11, 64, 256)
    d, q = oracle.q8_0_fields(raw, 64, 256)
    w = oracle.dequant_q8_0(raw, 64, 256).reshape(64, 8, 32)
    nz = d != 0
    q_back = np.rint(w / np.where(nz, d, 1.0)[:, :, None])
    assert np.array_equal(q_back[nz], q[nz])


def test_q8_0_full_quantiser_round_trip_on_blocks_with_extreme_quant():
    # A full quantiser d' = RN_fp16(max|w| / 127), q' = round(w / d') reproduces the
    # block exactly when the block contains +-127 (then max|w| = 127 d).
    raw = bytearray(synth.q8_0_weights(12, 16, 128))
    blocks = np.frombuffer(raw, dtype=np.uint8).reshape(-1, 34).copy()
    blocks[:, 2 + 7] = np.uint8(127)
    blocks[::2, 2 + 19] = np.uint8(0x81)  # -127
    raw = blocks.reshape(-1)
    d, q = oracle.q8_0_fields(raw, 16, 128)
    w = oracle.dequant_q8_0(raw, 16, 128).reshape(16, 4, 32)
    d_new = (np.abs(w).max(axis=2) / 127.0).astype(np.float16).astype(np.float64)
    assert np.array_equal(d_new, d)
    ok = d_new != 0
    q_new = np.rint(w / np.where(ok, d_new, 1.0)[:, :, None])
    assert np.array_equal(q_new[ok], q[ok])


def test_q8_0_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_q8_0(bytes(33), 1, 32)
    with pytest.raises(ValueError):
        oracle.dequant_q8_0(bytes(34), 1, 31)


# ---------------------------------------------------------------- Q4_K

def test_q4_k_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "q4_k_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, dmin, sc, m, q = oracle.q4_k_fields(raw, 1, 256)
        assert list(sc[0, 0]) == blk["sc"], blk["name"]
        assert list(m[0, 0]) == blk["m"], blk["name"]
        assert list(q[0, 0]) == blk["q"], blk["name"]
        assert d[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        assert dmin[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["dmin_bits"]]))[0]
        w = oracle.dequant_q4_k(raw, 1, 256)[0]
        expect = np.array([float.fromhex(v) for v in blk["expect"]])
        assert np.array_equal(w, expect), blk["name"]


def test_q4_k_handbuilt_top_bits_by_value(golden_dir):
    # Values read straight off the hand derivation: d=0.5, dmin=0.25, all q=1.
    blk = {b["name"]: b for b in _load(golden_dir, "q4_k_handbuilt.json")}["top_bit_carries"]
    w = oracle.dequant_q4_k(bytes.fromhex(blk["hex"]), 1, 256)[0]
    assert list(w[::32]) == [31.5, 29.25, 14.75, 22.0, 8.25, 12.25, -3.5, 22.25]


def test_q4_k_quant_byte_locality():
    raw = bytearray(synth.q4_k_weights(21, 1, 256))
    base = oracle.dequant_q4_k(bytes(raw), 1, 256)[0]
    _, _, sc, _, _ = oracle.q4_k_fields(bytes(raw), 1, 256)
    for p in range(128):
        c, l = divmod(p, 32)
        for mask, weight in ((0x0F, 64 * c + l), (0xF0, 64 * c + 32 + l)):
            mod = bytearray(raw)
            mod[16 + p] ^= mask
            w = oracle.dequant_q4_k(bytes(mod), 1, 256)[0]
            changed = np.nonzero(w != base)[0]
            if sc[0, 0, weight // 32] != 0:
                assert list(changed) == [weight], (p, mask)
            else:
                assert changed.size == 0


# (byte index in S, bit) -> (field, sub-block, value of that bit in the field)
def _scale_bit_owner(i, bit):
    if i < 4:
        return ("sc", i, 1 << bit) if bit < 6 else ("sc", i + 4, 1 << (bit - 2))
    if i < 8:
        return ("m", i - 4, 1 << bit) if bit < 6 else ("m", i, 1 << (bit - 2))
    return ("sc", i - 4, 1 << bit) if bit < 4 else ("m", i - 4, 1 << (bit - 4))


def test_q4_k_scale_byte_locality():
    raw = bytearray(synth.q4_k_weights(22, 1, 256))
    _, _, sc0, m0, _ = oracle.q4_k_fields(bytes(raw), 1, 256)
    for i in range(12):
        for bit in range(8):
            mod = bytearray(raw)
            mod[4 + i] ^= 1 << bit
            _, _, sc1, m1, _ = oracle.q4_k_fields(bytes(mod), 1, 256)
            field, j, val = _scale_bit_owner(i, bit)
            dsc = (sc1 - sc0)[0, 0]
            dm = (m1 - m0)[0, 0]
            hit, other = (dsc, dm) if field == "sc" else (dm, dsc)
            assert np.count_nonzero(other) == 0, (i, bit)
            assert list(np.nonzero(hit)[0]) == [j], (i, bit)
            assert abs(hit[j]) == val, (i, bit)


def test_q4_k_pack_unpack_bijection():
    # every value of every 6-bit field, in every position, survives pack -> decode
    rng = np.random.default_rng(3)
    for j in range(8):
        for v in range(64):
            for field in ("sc", "m"):
                sc = list(rng.integers(0, 64, 8))
                m = list(rng.integers(0, 64, 8))
                (sc if field == "sc" else m)[j] = v
                q = list(rng.integers(0, 16, 256))
                raw = bytes([0, 0x3C, 0, 0x3C]) + pack_scales_mins(sc, m) + pack_nibbles(q)
                _, _, dsc, dm, dq = oracle.q4_k_fields(raw, 1, 256)
                assert list(dsc[0, 0]) == sc and list(dm[0, 0]) == m and list(dq[0, 0]) == q
    # and random bytes survive decode -> pack
    raw = synth.q4_k_weights(23, 8, 512)
    _, _, sc, m, q = oracle.q4_k_fields(raw, 8, 512)
    blocks = raw.reshape(-1, 144)
    for b in range(blocks.shape[0]):
        n, t = divmod(b, 2)
        assert pack_scales_mins(list(sc[n, t]), list(m[n, t])) == bytes(blocks[b, 4:16])
        assert pack_nibbles(list(q[n, t])) == bytes(blocks[b, 16:])


def test_q4_k_requant_round_trip():
    raw = synth.q4_k_weights(24, 32, 512)
    d, dmin, sc, m, q = oracle.q4_k_fields(raw, 32, 512)
    w = oracle.dequant_q4_k(raw, 32, 512).reshape(32, 2, 8, 32)
    scale = d[:, :, None] * sc
    off = dmin[:, :, None] * m
    ok = scale != 0
    q_back = np.rint((w + off[..., None]) / np.where(ok, scale, 1.0)[..., None])
    q4 = q.reshape(32, 2, 8, 32)
    assert np.array_equal(q_back[ok], q4[ok])


def test_q4_k_weights_are_exact_dyadics():
    # every weight is an integer multiple of 2^-24 below 2^50: fp64 holds it exactly
    raw = synth.q4_k_weights(25, 16, 1024)
    w = oracle.dequant_q4_k(raw, 16, 1024)
    scaled = w * 2.0 ** 24
    assert np.array_equal(scaled, np.rint(scaled))
    assert np.max(np.abs(scaled)) < 2.0 ** 50


def test_q4_k_generator_distributions():
    raw = synth.q4_k_weights(26, 256, 2048)
    d, dmin, sc, m, q = oracle.q4_k_fields(raw, 256, 2048)
    assert sc.min() == 0 and sc.max() == 63 and m.min() == 0 and m.max() == 63
    assert q.min() == 0 and q.max() == 15
    assert abs(sc.mean() - 31.5) < 0.5 and abs(m.mean() - 31.5) < 0.5 and abs(q.mean() - 7.5) < 0.05
    # d ~ |N(0,1)| * 0.002: mean 0.002*sqrt(2/pi)
    assert abs(d.mean() / (0.002 * np.sqrt(2 / np.pi)) - 1) < 0.02
    assert abs(dmin.mean() / (0.002 * np.sqrt(2 / np.pi)) - 1) < 0.02


def test_q4_k_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_q4_k(bytes(143), 1, 256)
    with pytest.raises(ValueError):
        oracle.dequant_q4_k(bytes(144), 1, 128)


def test_fp32_target_rounds_once():
    # weights that fp32 cannot hold are rounded to nearest: d*sc*q has <= 21 bits,
    # dmin*m <= 17, their difference can need more than 24 bits.
    raw = synth.q4_k_weights(27, 64, 1024)
    w = oracle.dequant_q4_k(raw, 64, 1024)
    w32 = oracle.dequant_q4_k_f32(raw, 64, 1024)
    assert w32.dtype == np.float32
    err = np.abs(w32.astype(np.float64) - w)
    ulp = np.spacing(np.abs(w32)).astype(np.float64)
    assert np.all(err <= 0.5 * ulp)
    assert np.count_nonzero(err) > 0        # some weights really need the rounding


# ---------------------------------------------------------------- Q5_K

def test_q5_k_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "q5_k_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, dmin, sc, m, q = oracle.q5_k_fields(raw, 1, 256)
        assert list(sc[0, 0]) == blk["sc"], blk["name"]
        assert list(m[0, 0]) == blk["m"], blk["name"]
        assert list(q[0, 0]) == blk["q"], blk["name"]
        assert d[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        assert dmin[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["dmin_bits"]]))[0]
        w = oracle.dequant_q5_k(raw, 1, 256)[0]
        expect = np.array([float.fromhex(v) for v in blk["expect"]])
        assert np.array_equal(w, expect), blk["name"]


def test_q5_k_handbuilt_values_by_hand(golden_dir):
    blocks = {b["name"]: b for b in _load(golden_dir, "q5_k_handbuilt.json")}
    # d = 1, dmin = 0, sc_j = j + 1, every q = 16: w = 16 (j + 1)
    w = oracle.dequant_q5_k(bytes.fromhex(blocks["high_plane_all"]["hex"]), 1, 256)[0]
    assert list(w[::32]) == [16.0, 32.0, 48.0, 64.0, 80.0, 96.0, 112.0, 128.0]
    # d = 1, dmin = 1, sc = 1, m_j = j + 1; chunk 2 (weights 128..191) carries the high bit
    w = oracle.dequant_q5_k(bytes.fromhex(blocks["chunk2_plane"]["hex"]), 1, 256)[0]
    assert list(w[[0, 5, 127, 128, 133, 191, 192, 255]]) == [-1.0, 4.0, 11.0, 11.0, 16.0, 25.0, -7.0, 7.0]
    # d = -0: the scale term vanishes and w = -dmin * m_j exactly
    w = oracle.dequant_q5_k(bytes.fromhex(blocks["negative_zero_d"]["hex"]), 1, 256)[0]
    assert list(w[::32]) == [0.0, -7.0, -63.0, -32.0, -63.0, -17.0, -50.0, -5.0]


def _q5_to_q4_bytes(raw5):
    """The Q4_K block with Q5_K's header and nibbles (the high-bit plane dropped)."""
    b = np.asarray(raw5, dtype=np.uint8).reshape(-1, 176)
    return np.concatenate([b[:, :16], b[:, 48:]], axis=1).reshape(-1)


def test_q5_k_without_high_bits_is_q4_k():
    raw = synth.q5_k_weights(71, 8, 512).reshape(-1, 176).copy()
    raw[:, 16:48] = 0
    w5 = oracle.dequant_q5_k(raw.reshape(-1), 8, 512)
    w4 = oracle.dequant_q4_k(_q5_to_q4_bytes(raw), 8, 512)
    assert np.array_equal(w5, w4)


def test_q5_k_all_high_bits_add_sixteen_scales():
    raw = synth.q5_k_weights(72, 8, 512).reshape(-1, 176).copy()
    lo = raw.copy()
    lo[:, 16:48] = 0
    hi = raw.copy()
    hi[:, 16:48] = 0xFF
    d, _, sc, _, _ = oracle.q5_k_fields(lo.reshape(-1), 8, 512)
    step = (16 * d[:, :, None] * sc).repeat(32, axis=2).reshape(8, 512)
    diff = oracle.dequant_q5_k(hi.reshape(-1), 8, 512) - oracle.dequant_q5_k(lo.reshape(-1), 8, 512)
    assert np.array_equal(diff, step)


def test_q5_k_high_bit_locality():
    raw = bytearray(synth.q5_k_weights(73, 1, 256))
    base = oracle.dequant_q5_k(bytes(raw), 1, 256)[0]
    d, _, sc, _, q = oracle.q5_k_fields(bytes(raw), 1, 256)
    for l in range(32):
        for bit in range(8):
            weight = 64 * (bit // 2) + 32 * (bit % 2) + l
            mod = bytearray(raw)
            mod[16 + l] ^= 1 << bit
            w = oracle.dequant_q5_k(bytes(mod), 1, 256)[0]
            changed = np.nonzero(w != base)[0]
            step = 16 * d[0, 0] * sc[0, 0, weight // 32]
            if step != 0:
                assert list(changed) == [weight], (l, bit)
                sign = -1 if q[0, 0, weight] >= 16 else 1
                assert w[weight] - base[weight] == sign * step
            else:
                assert changed.size == 0


def test_q5_k_nibble_byte_locality():
    raw = bytearray(synth.q5_k_weights(74, 1, 256))
    base = oracle.dequant_q5_k(bytes(raw), 1, 256)[0]
    _, _, sc, _, _ = oracle.q5_k_fields(bytes(raw), 1, 256)
    for p in range(128):
        c, l = divmod(p, 32)
        for mask, weight in ((0x0F, 64 * c + l), (0xF0, 64 * c + 32 + l)):
            mod = bytearray(raw)
            mod[48 + p] ^= mask
            changed = np.nonzero(oracle.dequant_q5_k(bytes(mod), 1, 256)[0] != base)[0]
            assert list(changed) == ([weight] if sc[0, 0, weight // 32] != 0 else []), (p, mask)


def test_q5_k_pack_unpack_bijection():
    # every 5-bit quant value in every position survives pack -> decode, and random bytes decode -> pack
    rng = np.random.default_rng(5)
    for v in range(32):
        q = list(rng.integers(0, 32, 256))
        for i in range(v, 256, 32):
            q[i] = v
        raw = bytes([0, 0x3C, 0, 0x3C]) + pack_scales_mins([1] * 8, [0] * 8) + pack_q5_high_bits(q) + \
            pack_nibbles([t & 15 for t in q])
        assert list(oracle.q5_k_fields(raw, 1, 256)[4][0, 0]) == q
    raw = synth.q5_k_weights(75, 4, 512)
    _, _, sc, m, q = oracle.q5_k_fields(raw, 4, 512)
    blocks = raw.reshape(-1, 176)
    for b in range(blocks.shape[0]):
        n, t = divmod(b, 2)
        assert pack_scales_mins(list(sc[n, t]), list(m[n, t])) == bytes(blocks[b, 4:16])
        assert pack_q5_high_bits(list(q[n, t])) == bytes(blocks[b, 16:48])
        assert pack_nibbles([v & 15 for v in q[n, t]]) == bytes(blocks[b, 48:])


def test_q5_k_requant_round_trip():
    raw = synth.q5_k_weights(76, 16, 512)
    d, dmin, sc, m, q = oracle.q5_k_fields(raw, 16, 512)
    w = oracle.dequant_q5_k(raw, 16, 512).reshape(16, 2, 8, 32)
    scale = d[:, :, None] * sc
    off = dmin[:, :, None] * m
    ok = scale != 0
    q_back = np.rint((w + off[..., None]) / np.where(ok, scale, 1.0)[..., None])
    assert np.array_equal(q_back[ok], q.reshape(16, 2, 8, 32)[ok])


def test_q5_k_weights_exact_and_fp32_target_rounds_once():
    raw = synth.q5_k_weights(77, 32, 1024)
    w = oracle.dequant_q5_k(raw, 32, 1024)
    scaled = w * 2.0 ** 24
    assert np.array_equal(scaled, np.rint(scaled)) and np.max(np.abs(scaled)) < 2.0 ** 50
    w32 = oracle.dequant_q5_k_f32(raw, 32, 1024)
    err = np.abs(w32.astype(np.float64) - w)
    assert np.all(err <= 0.5 * np.spacing(np.abs(w32)).astype(np.float64))


def test_q5_k_generator_distributions():
    raw = synth.q5_k_weights(78, 128, 2048)
    d, dmin, sc, m, q = oracle.q5_k_fields(raw, 128, 2048)
    assert q.min() == 0 and q.max() == 31 and abs(q.mean() - 15.5) < 0.1
    assert sc.min() == 0 and sc.max() == 63 and abs(m.mean() - 31.5) < 0.5
    assert abs(d.mean() / (0.001 * np.sqrt(2 / np.pi)) - 1) < 0.03
    assert abs(dmin.mean() / (0.002 * np.sqrt(2 / np.pi)) - 1) < 0.03


def test_q5_k_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_q5_k(bytes(175), 1, 256)
    with pytest.raises(ValueError):
        oracle.dequant_q5_k(bytes(176), 1, 128)


# ---------------------------------------------------------------- Q6_K

def test_q6_k_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "q6_k_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, sc, q = oracle.q6_k_fields(raw, 1, 256)
        assert list(sc[0, 0]) == blk["sc"], blk["name"]
        assert list(q[0, 0]) == blk["q"], blk["name"]
        assert d[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        w = oracle.dequant_q6_k(raw, 1, 256)[0]
        expect = np.array([float.fromhex(v) for v in blk["expect"]])
        assert np.array_equal(w, expect), blk["name"]


def test_q6_k_handbuilt_values_by_hand(golden_dir):
    blocks = {b["name"]: b for b in _load(golden_dir, "q6_k_handbuilt.json")}
    # d = 1, every q = -32, sc = 1: every weight is -32
    assert set(oracle.dequant_q6_k(bytes.fromhex(blocks["all_min"]["hex"]), 1, 256)[0]) == {-32.0}
    # d = 0.5, q = 31, scales alternate 127, -128: 0.5 * 127 * 31 and 0.5 * -128 * 31
    w = oracle.dequant_q6_k(bytes.fromhex(blocks["all_max"]["hex"]), 1, 256)[0]
    assert list(w[[0, 15, 16, 31, 255]]) == [1968.5, 1968.5, -1984.0, -1984.0, -1984.0]
    # d = 1, quarter c of each half holds q = 16c - 31; scales 1, -1, 2, -2, ...
    w = oracle.dequant_q6_k(bytes.fromhex(blocks["quarter_code"]["hex"]), 1, 256)[0]
    assert list(w[[0, 16, 32, 48, 64, 96, 128, 255]]) == [-31.0, 31.0, -30.0, 30.0, 3.0, 68.0, -155.0, -136.0]
    # d = -0.25, q = -1: w = 0.25 * sc
    w = oracle.dequant_q6_k(bytes.fromhex(blocks["negative_d"]["hex"]), 1, 256)[0]
    assert list(w[::16]) == [25.0, -25.0, 12.5, -12.5, 6.25, -6.25, 3.0, -3.0, 1.5, -1.5, 0.75, -0.75,
                             0.25, -0.25, 0.0, 0.0]


def test_q6_k_low_plane_byte_locality():
    raw = bytearray(synth.q6_k_weights(81, 1, 256))
    base = oracle.dequant_q6_k(bytes(raw), 1, 256)[0]
    _, sc, _ = oracle.q6_k_fields(bytes(raw), 1, 256)
    for p in range(128):
        h, r = divmod(p, 64)
        c0, l = divmod(r, 32)
        for mask, c in ((0x0F, c0), (0xF0, c0 + 2)):
            weight = 128 * h + 32 * c + l
            mod = bytearray(raw)
            mod[p] ^= mask
            changed = np.nonzero(oracle.dequant_q6_k(bytes(mod), 1, 256)[0] != base)[0]
            assert list(changed) == ([weight] if sc[0, 0, weight // 16] != 0 else []), (p, mask)


def test_q6_k_high_plane_bit_locality():
    raw = bytearray(synth.q6_k_weights(82, 1, 256))
    base = oracle.dequant_q6_k(bytes(raw), 1, 256)[0]
    d, sc, q = oracle.q6_k_fields(bytes(raw), 1, 256)
    for p in range(64):
        h, l = divmod(p, 32)
        for bit in range(8):
            c = bit // 2
            weight = 128 * h + 32 * c + l
            mod = bytearray(raw)
            mod[128 + p] ^= 1 << bit
            w = oracle.dequant_q6_k(bytes(mod), 1, 256)[0]
            changed = np.nonzero(w != base)[0]
            step = d[0, 0] * sc[0, 0, weight // 16] * (16 << (bit % 2))
            if step != 0:
                assert list(changed) == [weight], (p, bit)
                assert abs(w[weight] - base[weight]) == abs(step)
            else:
                assert changed.size == 0


def test_q6_k_scale_byte_owns_sixteen_weights():
    raw = bytearray(synth.q6_k_weights(83, 1, 256))
    base = oracle.dequant_q6_k(bytes(raw), 1, 256)[0]
    d, sc, q = oracle.q6_k_fields(bytes(raw), 1, 256)
    for i in range(16):
        mod = bytearray(raw)
        mod[192 + i] = (sc[0, 0, i] + 1) & 0xFF if sc[0, 0, i] != 127 else 0x80
        w = oracle.dequant_q6_k(bytes(mod), 1, 256)[0]
        changed = set(np.nonzero(w != base)[0])
        expected = {16 * i + t for t in range(16) if q[0, 0, 16 * i + t] != 0}
        assert changed == expected, i


def test_q6_k_pack_unpack_bijection():
    rng = np.random.default_rng(7)
    for v in range(-32, 32):
        q = list(rng.integers(-32, 32, 256))
        for i in range((v + 32) % 16, 256, 16):
            q[i] = v
        raw = pack_q6_planes(q) + bytes([1] * 16) + bytes([0, 0x3C])
        assert list(oracle.q6_k_fields(raw, 1, 256)[2][0, 0]) == q
    raw = synth.q6_k_weights(84, 4, 512)
    _, sc, q = oracle.q6_k_fields(raw, 4, 512)
    blocks = raw.reshape(-1, 210)
    for b in range(blocks.shape[0]):
        n, t = divmod(b, 2)
        assert pack_q6_planes([int(v) for v in q[n, t]]) == bytes(blocks[b, :192])
        assert bytes([int(v) & 0xFF for v in sc[n, t]]) == bytes(blocks[b, 192:208])


def test_q6_k_requant_round_trip():
    raw = synth.q6_k_weights(85, 16, 512)
    d, sc, q = oracle.q6_k_fields(raw, 16, 512)
    w = oracle.dequant_q6_k(raw, 16, 512).reshape(16, 2, 16, 16)
    scale = d[:, :, None] * sc
    ok = scale != 0
    q_back = np.rint(w / np.where(ok, scale, 1.0)[..., None])
    assert np.array_equal(q_back[ok], q.reshape(16, 2, 16, 16)[ok])


def test_q6_k_weights_exact_and_fp32_target_rounds_once():
    raw = synth.q6_k_weights(86, 32, 1024)
    w = oracle.dequant_q6_k(raw, 32, 1024)
    scaled = w * 2.0 ** 24
    assert np.array_equal(scaled, np.rint(scaled)) and np.max(np.abs(scaled)) < 2.0 ** 50
    w32 = oracle.dequant_q6_k_f32(raw, 32, 1024)
    err = np.abs(w32.astype(np.float64) - w)
    assert np.all(err <= 0.5 * np.spacing(np.abs(w32)).astype(np.float64))


def test_q6_k_generator_distributions():
    raw = synth.q6_k_weights(87, 128, 2048)
    d, sc, q = oracle.q6_k_fields(raw, 128, 2048)
    assert q.min() == -32 and q.max() == 31 and abs(q.mean() + 0.5) < 0.1
    assert sc.min() == -128 and sc.max() == 127 and abs(sc.mean() + 0.5) < 1.0
    assert abs(d.mean() / (0.0002 * np.sqrt(2 / np.pi)) - 1) < 0.03


def test_q6_k_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_q6_k(bytes(209), 1, 256)
    with pytest.raises(ValueError):
        oracle.dequant_q6_k(bytes(210), 1, 128)


# ---------------------------------------------------------------- IQ4_XS

def test_iq4_xs_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "iq4_xs_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, ls, q = oracle.iq4_xs_fields(raw, 1, 256)
        assert list(ls[0, 0]) == blk["ls"], blk["name"]
        assert list(q[0, 0]) == blk["q"], blk["name"]
        assert d[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        w = oracle.dequant_iq4_xs(raw, 1, 256)[0]
        expect = np.array([float.fromhex(v) for v in blk["expect"]])
        assert np.array_equal(w, expect), blk["name"]


def test_iq4_xs_handbuilt_values_by_hand(golden_dir):
    blocks = {b["name"]: b for b in _load(golden_dir, "iq4_xs_handbuilt.json")}
    # d = 1, every scale 33 (weight scale 1): the weights walk the grid
    w = oracle.dequant_iq4_xs(bytes.fromhex(blocks["grid_walk"]["hex"]), 1, 256)[0]
    assert list(w[:16]) == [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]
    # d = 0.5, weight scales 0, 1, -1, -32, 31, -16, 16, 15; at i = 32j the index (7i + 3) % 16
    # is 3 (grid value -65) for every j, so the first weights are 0.5 * s * -65
    w = oracle.dequant_iq4_xs(bytes.fromhex(blocks["signed_scales"]["hex"]), 1, 256)[0]
    assert list(w[::32]) == [0.0, -32.5, 32.5, 1040.0, -1007.5, 520.0, -520.0, -487.5]
    # a scale of 32 zeroes the whole block, whatever the indices
    assert not oracle.dequant_iq4_xs(bytes.fromhex(blocks["zero_point_scale"]["hex"]), 1, 256).any()


def test_iq4_xs_grid_shape():
    g = np.asarray(oracle.IQ4_GRID)
    assert g.shape == (16,) and np.all(np.diff(g) > 0)     # 16 distinct, increasing
    assert g.min() == -127 and g.max() == 113              # the int8-range endpoints of the format
    assert list(g) == IQ4_XS_GRID                           # the golden script's own transcription


def test_iq4_xs_index_byte_locality():
    raw = bytearray(synth.iq4_xs_weights(61, 1, 256))
    base = oracle.dequant_iq4_xs(bytes(raw), 1, 256)[0]
    _, ls, _ = oracle.iq4_xs_fields(bytes(raw), 1, 256)
    for p in range(128):
        j, i = divmod(p, 16)
        for mask, weight in ((0x0F, 32 * j + i), (0xF0, 32 * j + 16 + i)):
            mod = bytearray(raw)
            mod[8 + p] ^= mask
            w = oracle.dequant_iq4_xs(bytes(mod), 1, 256)[0]
            changed = np.nonzero(w != base)[0]
            if ls[0, 0, weight // 32] != 32 and base.any():
                assert list(changed) == [weight], (p, mask)
            else:
                assert changed.size == 0


def test_iq4_xs_scale_bit_locality():
    # bit b of byte 2..7 belongs to exactly one sub-block scale: H bit 2j + t is bit 4 + t of
    # ls_j; L[j // 2] bit 4 (j % 2) + t is bit t of ls_j
    raw = bytearray(synth.iq4_xs_weights(62, 1, 256))
    _, ls0, _ = oracle.iq4_xs_fields(bytes(raw), 1, 256)
    for byte in range(6):
        for bit in range(8):
            mod = bytearray(raw)
            mod[2 + byte] ^= 1 << bit
            _, ls1, _ = oracle.iq4_xs_fields(bytes(mod), 1, 256)
            diff = (ls1 - ls0)[0, 0]
            if byte < 2:
                hb = 8 * byte + bit
                j, val = hb // 2, 1 << (4 + hb % 2)
            else:
                j, val = 2 * (byte - 2) + bit // 4, 1 << (bit % 4)
            assert list(np.nonzero(diff)[0]) == [j], (byte, bit)
            assert abs(diff[j]) == val, (byte, bit)


def test_iq4_xs_pack_unpack_bijection():
    rng = np.random.default_rng(5)
    for j in range(8):
        for v in range(64):
            ls = list(rng.integers(0, 64, 8))
            ls[j] = v
            q = list(rng.integers(0, 16, 256))
            raw = bytes([0, 0x3C]) + pack_iq4_xs_scales(ls) + pack_iq4_indices(q)
            _, dls, dq = oracle.iq4_xs_fields(raw, 1, 256)
            assert list(dls[0, 0]) == ls and list(dq[0, 0]) == q
    raw = synth.iq4_xs_weights(63, 4, 768)
    _, ls, q = oracle.iq4_xs_fields(raw, 4, 768)
    blocks = raw.reshape(-1, 136)
    for b in range(blocks.shape[0]):
        n, t = divmod(b, 3)
        assert pack_iq4_xs_scales(list(ls[n, t])) == bytes(blocks[b, 2:8])
        assert pack_iq4_indices(list(q[n, t])) == bytes(blocks[b, 8:])


def test_iq4_xs_requant_round_trip():
    # nearest-grid requantisation of the exact weights recovers every index (grid values are distinct)
    raw = synth.iq4_xs_weights(64, 16, 512)
    d, ls, q = oracle.iq4_xs_fields(raw, 16, 512)
    w = oracle.dequant_iq4_xs(raw, 16, 512).reshape(16, 2, 8, 32)
    scale = d[:, :, None] * (ls - 32)
    ok = scale != 0
    t = w / np.where(ok, scale, 1.0)[..., None]
    q_back = np.argmin(np.abs(t[..., None] - np.asarray(oracle.IQ4_GRID)[None, None, None, None, :]), axis=-1)
    assert np.array_equal(q_back[ok], q.reshape(16, 2, 8, 32)[ok])


def test_iq4_xs_weights_are_exact_in_fp32():
    raw = synth.iq4_xs_weights(65, 16, 1024)
    w = oracle.dequant_iq4_xs(raw, 16, 1024)
    assert np.array_equal(w, w.astype(np.float32).astype(np.float64))
    scaled = w * 2.0 ** 24
    assert np.array_equal(scaled, np.rint(scaled))


def test_iq4_xs_generator_distributions():
    raw = synth.iq4_xs_weights(66, 256, 2048)
    d, ls, q = oracle.iq4_xs_fields(raw, 256, 2048)
    assert ls.min() == 0 and ls.max() == 63 and q.min() == 0 and q.max() == 15
    assert abs(ls.mean() - 31.5) < 0.5 and abs(q.mean() - 7.5) < 0.05
    assert abs(d.mean() / (0.0005 * np.sqrt(2 / np.pi)) - 1) < 0.02


def test_iq4_xs_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_iq4_xs(bytes(135), 1, 256)
    with pytest.raises(ValueError):
        oracle.dequant_iq4_xs(bytes(136), 1, 128)


# ---------------------------------------------------------------- Q4_0

def test_q4_0_handbuilt_blocks(golden_dir):
    for blk in _load(golden_dir, "q4_0_handbuilt.json"):
        raw = bytes.fromhex(blk["hex"])
        d, q = oracle.q4_0_fields(raw, 1, 32)
        assert list(q[0, 0]) == blk["q"], blk["name"]
        assert d[0, 0] == oracle.fp16_bits_to_f64(np.array([blk["d_bits"]]))[0]
        w = oracle.dequant_q4_0(raw, 1, 32)[0]
        assert np.array_equal(w, [float.fromhex(v) for v in blk["expect"]]), blk["name"]


def test_q4_0_handbuilt_values_by_hand(golden_dir):
    blocks = {b["name"]: bytes.fromhex(b["hex"]) for b in _load(golden_dir, "q4_0_handbuilt.json")}
    w = lambda name: list(oracle.dequant_q4_0(blocks[name], 1, 32)[0])  # noqa: E731
    # d = 1, byte j = 0x11 * j: weights j and 16 + j both j - 8
    assert w("unit_scale_ramp") == [float(j - 8) for j in range(16)] * 2
    # d = 0.5, bytes 0xF0: the first 16 weights -4, the last 16 weights 3.5
    assert w("halves_differ") == [-4.0] * 16 + [3.5] * 16
    # d = 1, byte j = (j << 4) | (15 - j): weight j is 7 - j, weight 16 + j is j - 8
    assert w("position_code") == [float(7 - j) for j in range(16)] + [float(j - 8) for j in range(16)]
    # d = 2^-24, all nibbles 8 except weight 31's: zeros, then -8 * 2^-24
    assert w("subnormal_scale") == [0.0] * 31 + [-8 * 2.0 ** -24]
    # d = -2, nibbles 3: every weight 10
    assert w("negative_scale") == [10.0] * 32
    assert w("zero_scale") == [0.0] * 32


def test_q4_0_nibble_locality():
    raw = bytearray(synth.q4_0_weights(85, 1, 32))
    base = oracle.dequant_q4_0(bytes(raw), 1, 32)[0]
    d, _ = oracle.q4_0_fields(bytes(raw), 1, 32)
    for j in range(16):
        for mask, weight in ((0x0F, j), (0xF0, 16 + j)):
            mod = bytearray(raw)
            mod[2 + j] ^= mask
            w = oracle.dequant_q4_0(bytes(mod), 1, 32)[0]
            changed = np.nonzero(w != base)[0]
            assert list(changed) == ([weight] if d[0, 0] != 0 else []), (j, mask)
            step = abs(w[weight] - base[weight])
            assert step == abs(d[0, 0]) * abs(((raw[2 + j] ^ mask) & mask) - (raw[2 + j] & mask)) / (16 if mask == 0xF0 else 1)


def test_q4_0_scale_bytes_own_the_block():
    raw = bytearray(synth.q4_0_weights(86, 2, 64))
    base = oracle.dequant_q4_0(bytes(raw), 2, 64)
    _, q = oracle.q4_0_fields(bytes(raw), 2, 64)
    for blk in range(4):
        for byte in (0, 1):
            mod = bytearray(raw)
            mod[18 * blk + byte] ^= 0x04
            changed = set(map(tuple, np.argwhere(oracle.dequant_q4_0(bytes(mod), 2, 64) != base)))
            n, t = divmod(blk, 2)
            assert changed == {(n, 32 * t + j) for j in range(32) if q[n, t, j] != 8}, (blk, byte)


def test_q4_0_pack_unpack_bijection():
    for v in range(16):
        for pos in range(32):
            q = [(pos + 3 * i) % 16 for i in range(32)]
            q[pos] = v
            raw = bytes([0x00, 0x3C]) + pack_q4_0_quants(q)
            assert list(oracle.q4_0_fields(raw, 1, 32)[1][0, 0]) == q
    raw = synth.q4_0_weights(87, 3, 96)
    _, q = oracle.q4_0_fields(raw, 3, 96)
    blocks = raw.reshape(-1, 18)
    for b in range(blocks.shape[0]):
        n, t = divmod(b, 3)
        assert pack_q4_0_quants([int(v) for v in q[n, t]]) == bytes(blocks[b, 2:])


def test_q4_0_requant_round_trip():
    raw = synth.q4_0_weights(88, 4, 256)
    w = oracle.dequant_q4_0(raw, 4, 256).reshape(4, 8, 32)
    d, q = oracle.q4_0_fields(raw, 4, 256)
    nz = d != 0
    q_back = np.rint(w / np.where(nz, d, 1.0)[:, :, None]) + 8
    assert np.array_equal(q_back[nz], q[nz])
    assert np.all(w[~nz] == 0)


def test_q4_0_weights_exact_in_fp32_and_generator_distribution():
    raw = synth.q4_0_weights(89, 64, 1024)
    w = oracle.dequant_q4_0(raw, 64, 1024)
    assert np.array_equal(oracle.dequant_q4_0_f32(raw, 64, 1024).astype(np.float64), w)
    d, q = oracle.q4_0_fields(raw, 64, 1024)
    counts = np.bincount(q.reshape(-1), minlength=16)
    assert counts.min() > 0.9 * q.size / 16 and counts.max() < 1.1 * q.size / 16
    assert (d < 0).mean() > 0.4 and (d > 0).mean() > 0.4


def test_q4_0_rejects_wrong_sizes():
    with pytest.raises(ValueError):
        oracle.dequant_q4_0(bytes(17), 1, 32)
    with pytest.raises(ValueError):
        oracle.dequant_q4_0(bytes(18), 1, 16)

