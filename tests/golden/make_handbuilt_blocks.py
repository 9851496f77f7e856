"""Writes tests/golden/{q8_0,q4_0,q4_k,q5_k,q6_k,iq4_xs}_handbuilt.json: hand-built blocks with known values.

Run from the repository root:  python tests/golden/make_handbuilt_blocks.py

Each block is stated by its fields (fp16 scale bit patterns, 6-bit scales and
mins, quants). Its bytes are assembled from those fields by this script's own
bit-level encoder of the public GGUF layouts (Q8_0: fp16 d then 32 int8;
Q4_K: fp16 d, fp16 dmin, 12 packed scale/min bytes, 128 nibble bytes). For the
Q4_K blocks the 12 scale bytes were also derived by hand and are written below
as literals; the script stops if its encoder disagrees with them.

The expected weights are computed here from the stated fields with exact
rational arithmetic (w = d*q for Q8_0, w = d*(q - 8) for Q4_0, w = d*sc_j*q - dmin*m_j for Q4_K,
w = d*(ls_j - 32)*grid[q] for IQ4_XS, the Q4_K form with 5-bit q for Q5_K,
w = d*sc_i*q for Q6_K);
they are closed forms by construction
and do not come from the oracle or the GPU. The memra pages name these formats
(memra README, model support table: Q8_0, Q4_K_M and IQ4_XS GGUF models) but
print no block bytes, so no value here is theirs. The IQ4_XS grid below is this
script's own transcription of the public format's 16 values.
"""

from __future__ import annotations

import json
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def fp16_value(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (finite only)."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    if exp == 0x1F:
        raise ValueError("non-finite fp16 in a golden block")
    if exp == 0:
        return sign * Fraction(man, 1 << 24)
    return sign * Fraction(1024 + man, 1 << 10) * (Fraction(2) ** (exp - 15))


def frac_to_hex(v: Fraction) -> str:
    f = float(v)
    assert Fraction(f) == v, "golden value not exact in binary64"
    return f.hex()


# ---------------------------------------------------------------- Q8_0

def q8_0_block(d_bits: int, q: list[int]) -> bytes:
    assert len(q) == 32 and all(-128 <= v <= 127 for v in q)
    return bytes([d_bits & 0xFF, d_bits >> 8]) + bytes([v & 0xFF for v in q])


Q8_0_BLOCKS = [
    ("unit_scale_ramp", 0x3C00, [j - 16 for j in range(32)]),
    ("subnormal_scale", 0x0001, [127, -127, 1, -1] + [0] * 27 + [5]),
    ("negative_scale", 0xC000, [(-1) ** j * j for j in range(32)]),
    ("max_finite_scale", 0x7BFF, [127] + [3] * 30 + [-127]),
    ("zero_scale", 0x0000, [(7 * j) % 255 - 127 for j in range(32)]),
]


# ---------------------------------------------------------------- Q4_K

def pack_scales_mins(sc: list[int], m: list[int]) -> bytes:
    """Bit-level encoder of the 12 scale/min bytes (this script's own statement).

    j < 4 : sc_j -> bits 0..5 of S[j],   m_j -> bits 0..5 of S[j+4]
    j >= 4: sc_j bits 0..3 -> bits 0..3 of S[j+4], bits 4..5 -> bits 6..7 of S[j-4]
            m_j  bits 0..3 -> bits 4..7 of S[j+4], bits 4..5 -> bits 6..7 of S[j]
    """
    S = [0] * 12
    for j in range(8):
        assert 0 <= sc[j] < 64 and 0 <= m[j] < 64
    for j in range(4):
        S[j] |= sc[j]
        S[j + 4] |= m[j]
    for j in range(4, 8):
        S[j + 4] |= (sc[j] & 0xF) | ((m[j] & 0xF) << 4)
        S[j - 4] |= (sc[j] >> 4) << 6
        S[j] |= (m[j] >> 4) << 6
    return bytes(S)


def pack_nibbles(q: list[int]) -> bytes:
    """Quant bytes: Q[32c + l] = q[64c + l] | q[64c + 32 + l] << 4."""
    assert len(q) == 256 and all(0 <= v < 16 for v in q)
    out = bytearray(128)
    for c in range(4):
        for l in range(32):
            out[32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    return bytes(out)


# (name, d_bits, dmin_bits, sc[8], m[8], q[256], hand-derived scale bytes as hex)
Q4_K_BLOCKS = [
    ("distinct_scales", 0x3C00, 0x0000, [1, 2, 3, 4, 5, 6, 7, 8], [0] * 8,
     [i % 16 for i in range(256)], "010203040000000005060708"),
    ("distinct_mins", 0x3C00, 0x3C00, [1] * 8, [1, 2, 3, 4, 5, 6, 7, 8],
     [(i >> 4) & 15 for i in range(256)], "010101010102030451617181"),
    ("top_bit_carries", 0x3800, 0x3400, [63, 62, 61, 60, 48, 33, 18, 47], [0, 7, 63, 32, 63, 17, 50, 5],
     [1] * 256, "ffbe7dbcc047ff20f011225f"),
    ("subnormal_scales", 0x0001, 0x0003, [63] * 8, [63] * 8,
     [15] * 256, "ffffffffffffffffffffffff"),
    ("zero_d", 0x0000, 0x3C00, [63, 62, 61, 60, 48, 33, 18, 47], [0, 7, 63, 32, 63, 17, 50, 5],
     [(5 * i + 3) % 16 for i in range(256)], "ffbe7dbcc047ff20f011225f"),
    ("position_code", 0x3C00, 0x0000, [1] * 8, [0] * 8,
     [(i * 7 + (i >> 5)) % 16 for i in range(256)], "010101010000000001010101"),
]


# ---------------------------------------------------------------- Q5_K

def pack_q5_high_bits(q: list[int]) -> bytes:
    """The 32 high-bit bytes: bit 2c of H[l] is bit 4 of q[64c + l], bit 2c + 1
    is bit 4 of q[64c + 32 + l]."""
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    out = bytearray(32)
    for c in range(4):
        for l in range(32):
            out[l] |= (q[64 * c + l] >> 4) << (2 * c)
            out[l] |= (q[64 * c + 32 + l] >> 4) << (2 * c + 1)
    return bytes(out)


# (name, d_bits, dmin_bits, sc[8], m[8], q[256], hand-derived scale bytes, hand-derived high-bit bytes)
Q5_K_BLOCKS = [
    ("high_plane_all", 0x3C00, 0x0000, [1, 2, 3, 4, 5, 6, 7, 8], [0] * 8,
     [16] * 256, "010203040000000005060708", "ff" * 32),
    ("high_halves", 0x3800, 0x3400, [63, 62, 61, 60, 48, 33, 18, 47], [0, 7, 63, 32, 63, 17, 50, 5],
     [(i % 16) + (16 if i % 64 >= 32 else 0) for i in range(256)], "ffbe7dbcc047ff20f011225f", "aa" * 32),
    ("chunk2_plane", 0x3C00, 0x3C00, [1] * 8, [1, 2, 3, 4, 5, 6, 7, 8],
     [(i % 16) + (16 if 128 <= i < 192 else 0) for i in range(256)], "010101010102030451617181", "30" * 32),
    ("odd_positions", 0x0001, 0x0003, [63] * 8, [63] * 8,
     [31 if i % 2 else 15 for i in range(256)], "ff" * 12, "00ff" * 16),
    ("zero_plane", 0x3C00, 0x0000, [1] * 8, [0] * 8,
     [(i * 7 + (i >> 5)) % 16 for i in range(256)], "010101010000000001010101", "00" * 32),
    ("negative_zero_d", 0x8000, 0x3C00, [63, 62, 61, 60, 48, 33, 18, 47], [0, 7, 63, 32, 63, 17, 50, 5],
     [16 + (5 * i + 3) % 16 for i in range(256)], "ffbe7dbcc047ff20f011225f", "ff" * 32),
]


# ---------------------------------------------------------------- Q4_0

def pack_q4_0_quants(q: list[int]) -> bytes:
    """The 16 quant bytes of a Q4_0 block: weight j (j < 16) in the low nibble of
    byte j, weight 16 + j in its high nibble; q are the stored nibbles in [0, 15]."""
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    return bytes([q[j] | (q[16 + j] << 4) for j in range(16)])


# (name, d_bits, q[32] stored nibbles, hand-derived quant bytes)
Q4_0_BLOCKS = [
    ("unit_scale_ramp", 0x3C00, [j % 16 for j in range(32)], "00112233445566778899aabbccddeeff"),
    ("halves_differ", 0x3800, [0] * 16 + [15] * 16, "f0" * 16),
    ("position_code", 0x3C00, [15 - j for j in range(16)] + list(range(16)), "0f1e2d3c4b5a69788796a5b4c3d2e1f0"),
    ("subnormal_scale", 0x0001, [8] * 31 + [0], "88" * 15 + "08"),
    ("negative_scale", 0xC000, [3] * 32, "33" * 16),
    ("zero_scale", 0x0000, [5, 9] * 16, "5599" * 8),
]


# ---------------------------------------------------------------- Q6_K

def pack_q6_planes(q: list[int]) -> bytes:
    """The 128 low-bit and 64 high-bit bytes of signed 6-bit quants q in [-32, 31]:
    weight 128h + 32c + l (u = q + 32) puts u & 15 in L[64h + 32(c % 2) + l] (low
    nibble for c < 2, high nibble otherwise) and u >> 4 in bits 2c, 2c + 1 of H[32h + l]."""
    assert len(q) == 256 and all(-32 <= v < 32 for v in q)
    low = bytearray(128)
    high = bytearray(64)
    for h in range(2):
        for c in range(4):
            for l in range(32):
                u = q[128 * h + 32 * c + l] + 32
                low[64 * h + 32 * (c % 2) + l] |= (u & 15) << (0 if c < 2 else 4)
                high[32 * h + l] |= (u >> 4) << (2 * c)
    return bytes(low) + bytes(high)


# (name, d_bits, sc[16] int8, q[256], hand-derived low-plane bytes, hand-derived high-plane bytes)
Q6_K_BLOCKS = [
    ("all_min", 0x3C00, [1] * 16, [-32] * 256, "00" * 128, "00" * 64),
    ("all_max", 0x3800, [127, -128] * 8, [31] * 256, "ff" * 128, "ff" * 64),
    ("all_zero_quants", 0x3C00, [5] * 16, [0] * 256, "00" * 128, "aa" * 64),
    ("quarter_code", 0x3C00, [1, -1, 2, -2, 3, -3, 4, -4, 5, -5, 6, -6, 7, -7, 8, -8],
     [16 * ((i % 128) // 32) + 1 - 32 for i in range(256)], "11" * 128, "e4" * 64),
    ("position_code", 0x0001, [1, 2, 4, 8, 16, 32, 64, 127, -1, -2, -4, -8, -16, -32, -64, -128],
     [(i % 32) % 16 - 32 for i in range(256)], "00112233445566778899aabbccddeeff" * 8, "00" * 64),
    ("negative_d", 0xB400, [100, -100, 50, -50, 25, -25, 12, -12, 6, -6, 3, -3, 1, -1, 0, 0],
     [-1] * 256, "ff" * 128, "55" * 64),
]


# ---------------------------------------------------------------- IQ4_XS

IQ4_XS_GRID = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]


def pack_iq4_xs_scales(ls: list[int]) -> bytes:
    """The 6 scale bytes (this script's own statement of the layout).

    bytes 0..1: little-endian 16-bit H, bits 2j..2j+1 = bits 4..5 of ls_j
    bytes 2..5: L[0..3], L[j // 2] holds bits 0..3 of ls_j (low nibble for even j)
    """
    assert len(ls) == 8 and all(0 <= v < 64 for v in ls)
    h = 0
    low = [0] * 4
    for j, v in enumerate(ls):
        h |= (v >> 4) << (2 * j)
        low[j // 2] |= (v & 0xF) << (4 * (j % 2))
    return bytes([h & 0xFF, h >> 8]) + bytes(low)


def pack_iq4_indices(q: list[int]) -> bytes:
    """Index bytes: byte 16j + i = q[32j + i] | q[32j + 16 + i] << 4."""
    assert len(q) == 256 and all(0 <= v < 16 for v in q)
    out = bytearray(128)
    for j in range(8):
        for i in range(16):
            out[16 * j + i] = q[32 * j + i] | (q[32 * j + 16 + i] << 4)
    return bytes(out)


# (name, d_bits, ls[8], q[256], hand-derived scale bytes as hex)
IQ4_XS_BLOCKS = [
    ("grid_walk", 0x3C00, [33] * 8, [i % 16 for i in range(256)], "aaaa11111111"),
    ("signed_scales", 0x3800, [32, 33, 31, 0, 63, 16, 48, 47], [(7 * i + 3) % 16 for i in range(256)],
     "1ab7100f0ff0"),
    ("zero_point_scale", 0x3C00, [32] * 8, [(11 * i + 5) % 16 for i in range(256)], "aaaa00000000"),
    ("subnormal_d", 0x0001, [63, 0, 63, 0, 63, 0, 63, 0], [15 - i % 16 for i in range(256)], "33330f0f0f0f"),
    ("position_code", 0x3C00, [34] * 8, [(5 * i + (i >> 4)) % 16 for i in range(256)], "aaaa22222222"),
    ("negative_d", 0xBC00, [40, 24, 35, 29, 32, 60, 5, 50], [(3 * i) % 16 for i in range(256)], "66ce88d3c025"),
]


def main() -> None:
    q8 = []
    for name, d_bits, q in Q8_0_BLOCKS:
        raw = q8_0_block(d_bits, q)
        d = fp16_value(d_bits)
        q8.append({
            "name": name,
            "d_bits": d_bits,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(d * v) for v in q],
        })

    q40 = []
    for name, d_bits, q, q_hex in Q4_0_BLOCKS:
        qb = pack_q4_0_quants(q)
        if qb.hex() != q_hex:
            raise SystemExit(f"{name}: encoder gives {qb.hex()}, hand derivation says {q_hex}")
        raw = bytes([d_bits & 0xFF, d_bits >> 8]) + qb
        assert len(raw) == 18
        d = fp16_value(d_bits)
        q40.append({
            "name": name,
            "d_bits": d_bits,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(d * (v - 8)) for v in q],
        })

    q4 = []
    for name, d_bits, dmin_bits, sc, m, q, s_hex in Q4_K_BLOCKS:
        s_bytes = pack_scales_mins(sc, m)
        if s_bytes.hex() != s_hex:
            raise SystemExit(f"{name}: encoder gives {s_bytes.hex()}, hand derivation says {s_hex}")
        raw = bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8]) + s_bytes + pack_nibbles(q)
        assert len(raw) == 144
        d, dmin = fp16_value(d_bits), fp16_value(dmin_bits)
        expect = [d * sc[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)]
        q4.append({
            "name": name,
            "d_bits": d_bits,
            "dmin_bits": dmin_bits,
            "sc": sc,
            "m": m,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(v) for v in expect],
        })

    q5 = []
    for name, d_bits, dmin_bits, sc, m, q, s_hex, h_hex in Q5_K_BLOCKS:
        s_bytes = pack_scales_mins(sc, m)
        if s_bytes.hex() != s_hex:
            raise SystemExit(f"{name}: encoder gives {s_bytes.hex()}, hand derivation says {s_hex}")
        h_bytes = pack_q5_high_bits(q)
        if h_bytes.hex() != h_hex:
            raise SystemExit(f"{name}: encoder gives high bits {h_bytes.hex()}, hand derivation says {h_hex}")
        raw = (bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8]) + s_bytes + h_bytes +
               pack_nibbles([v & 15 for v in q]))
        assert len(raw) == 176
        d, dmin = fp16_value(d_bits), fp16_value(dmin_bits)
        expect = [d * sc[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)]
        q5.append({
            "name": name,
            "d_bits": d_bits,
            "dmin_bits": dmin_bits,
            "sc": sc,
            "m": m,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(v) for v in expect],
        })

    q6 = []
    for name, d_bits, sc, q, l_hex, h_hex in Q6_K_BLOCKS:
        planes = pack_q6_planes(q)
        if planes[:128].hex() != l_hex or planes[128:].hex() != h_hex:
            raise SystemExit(f"{name}: encoder gives {planes.hex()}, hand derivation says {l_hex}{h_hex}")
        assert all(-128 <= v < 128 for v in sc)
        raw = planes + bytes([v & 0xFF for v in sc]) + bytes([d_bits & 0xFF, d_bits >> 8])
        assert len(raw) == 210
        d = fp16_value(d_bits)
        expect = [d * sc[i // 16] * q[i] for i in range(256)]
        q6.append({
            "name": name,
            "d_bits": d_bits,
            "sc": sc,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(v) for v in expect],
        })

    iq4 = []
    for name, d_bits, ls, q, s_hex in IQ4_XS_BLOCKS:
        s_bytes = pack_iq4_xs_scales(ls)
        if s_bytes.hex() != s_hex:
            raise SystemExit(f"{name}: encoder gives {s_bytes.hex()}, hand derivation says {s_hex}")
        raw = bytes([d_bits & 0xFF, d_bits >> 8]) + s_bytes + pack_iq4_indices(q)
        assert len(raw) == 136
        d = fp16_value(d_bits)
        expect = [d * (ls[i // 32] - 32) * IQ4_XS_GRID[q[i]] for i in range(256)]
        iq4.append({
            "name": name,
            "d_bits": d_bits,
            "ls": ls,
            "q": q,
            "hex": raw.hex(),
            "expect": [frac_to_hex(v) for v in expect],
        })

    note = ("Hand-built blocks with known values (closed forms by construction). "
            "Formats named on the memra README model support table (Q8_0, Q4_K_M GGUF); "
            "layouts are the public GGUF ones. Written by tests/golden/make_handbuilt_blocks.py.")
    with open(os.path.join(HERE, "q8_0_handbuilt.json"), "w") as f:
        json.dump({"citation": note, "blocks": q8}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "q4_0_handbuilt.json"), "w") as f:
        json.dump({"citation": note.replace("(Q8_0, Q4_K_M GGUF)", "(Q8_0, Q4_K_M GGUF; the Gemma-4 QAT rows: Q4_0)"),
                   "blocks": q40}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "q4_k_handbuilt.json"), "w") as f:
        json.dump({"citation": note, "blocks": q4}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "q5_k_handbuilt.json"), "w") as f:
        json.dump({"citation": note.replace("(Q8_0, Q4_K_M GGUF)", "(Q8_0, Q4_K_M GGUF, whose K-quant mix includes Q5_K)"),
                   "blocks": q5}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "q6_k_handbuilt.json"), "w") as f:
        json.dump({"citation": note.replace("(Q8_0, Q4_K_M GGUF)", "(Q8_0, Q4_K_M GGUF, whose K-quant mix includes Q6_K)"),
                   "blocks": q6}, f, indent=1)
        f.write("\n")
    with open(os.path.join(HERE, "iq4_xs_handbuilt.json"), "w") as f:
        json.dump({"citation": note.replace("(Q8_0, Q4_K_M GGUF)", "(Q8_0, Q4_K_M, IQ4_XS GGUF)"), "blocks": iq4},
                  f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
