"""CPU fp64 oracle for GGUF block-quantized matrix-vector products.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, links or calls
this module: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may. It shares no code with the HIP library (no helpers, no tables, no
constants); the only code both sides consume is the seeded input generator in
synth/.

What is computed, and where it comes from
-----------------------------------------
The memra pages (memra README: the model support table lists Q8_0 and Q4_K_M
GGUF models, dense and MoE; the speed table's 35B-A3B MoE decode row; the
memra-bench card, "Drafts": Q4_K_M draft blocks measured faster than Q8_0 and
K=2..3 speculative drafts) name the formats and the workloads but print no block
layout, no kernel and no formula. The operation they rest on has a plain
definition -- a dense matrix product whose weights are the dequantized block
values -- so this oracle is that definition written out in fp64:

* decode each weight exactly from the stored bytes (every Q8_0 and Q4_K weight
  is an integer multiple of 2^-24 below 2^50, so fp64 holds it exactly);
* multiply with numpy's fp64 matmul (a library primitive);
* MoE: top-k routing on the fp32 logits, softmax renormalised over the k
  selected experts, silu(gate) * up, down, weighted sum in rank order;
* prefill: the same product for many rows, plus the variant whose weights are
  first rounded to fp32 and then to bf16 (the prescribed bf16 tile).

The byte layouts are the public GGUF ones (Q8_0: fp16 d + 32 int8; Q4_0: fp16 d
+ 16 bytes of nibbles, low nibbles first in weight order; Q4_K: fp16
d, fp16 dmin, 12 bytes of packed 6-bit scales and mins, 128 bytes of nibbles;
Q5_K: Q4_K plus a 32-byte plane of fifth bits; Q6_K: a 4-bit and a 2-bit plane
of signed 6-bit quants, 16 int8 scales, fp16 d;
IQ4_XS: fp16 d, 6-bit sub-block scales in 6 bytes, 128 bytes of 4-bit indices
into a 16-entry integer grid), restated in this module's own words next to the
code that reads them.

Parity pins live in tests/test_oracle_*.py (hand-built blocks written as hex,
locality invariants, pack/unpack bijection, requantisation round trips, exact
rational brute force, closed forms, MoE = weighted dense sum).

Parity unpinned: that the Q4_K 6-bit scale/min packing and nibble order, the
Q5_K and Q6_K bit planes, and the IQ4_XS scale packing, index order and
16-entry grid, used here equal those
of real llama.cpp-written GGUF tensors. No GGUF file, gguf
package or llama.cpp is in reach, and the pages print no block bytes, so every
in-repository check would also pass with a self-consistent mis-layout.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# scalar formats
# ----------------------------------------------------------------------------


def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 (little-endian bit patterns, subnormals honoured) -> float64."""
    return np.asarray(bits, dtype=np.uint16).view("<f2").astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: a bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view("<f4").astype(np.float64)


def round_to_f32(values) -> np.ndarray:
    """Round float64 values to the nearest fp32 (ties to even), returned as fp32."""
    return np.asarray(values, dtype=np.float64).astype(np.float32)


def round_f32_to_bf16_bits(values_f32) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 (ties to even); returns uint16 bits.

    Uses torch's CPU bf16 conversion as the library primitive.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ----------------------------------------------------------------------------
# Q8_0: 34-byte blocks of 32 weights along K
# ----------------------------------------------------------------------------

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32


def _as_bytes(raw) -> np.ndarray:
    return np.frombuffer(raw, dtype=np.uint8) if isinstance(raw, (bytes, bytearray)) else np.asarray(raw, dtype=np.uint8).reshape(-1)


def q8_0_fields(raw, n_rows: int, k: int):
    """Split a row-major Q8_0 matrix into (d [N, K/32] float64, q [N, K/32, 32] int64).

    Block t of row n starts at byte (n*K/32 + t)*34; bytes 0..1 hold the
    little-endian fp16 scale d, bytes 2..33 the signed int8 quants q_0..q_31.
    """
    if k % Q8_0_BLOCK_WEIGHTS:
        raise ValueError("Q8_0 needs K to be a multiple of 32")
    nb = k // Q8_0_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * Q8_0_BLOCK_BYTES:
        raise ValueError("byte count does not match the Q8_0 shape")
    blocks = b.reshape(n_rows, nb, Q8_0_BLOCK_BYTES)
    d_bits = blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)
    d = fp16_bits_to_f64(d_bits)
    q = blocks[:, :, 2:].view(np.int8).astype(np.int64)
    return d, q


def dequant_q8_0(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact Q8_0 weights: w[n, 32t + j] = d[n, t] * q[n, t, j]  (float64 [N, K])."""
    d, q = q8_0_fields(raw, n_rows, k)
    return (d[:, :, None] * q).reshape(n_rows, k)


# ----------------------------------------------------------------------------
# Q4_0: 18-byte blocks of 32 weights along K
# ----------------------------------------------------------------------------
#
# The format of the Gemma-4 QAT rows of the memra README's model support table.
# Public GGUF layout, restated: a little-endian fp16 scale d, then 16 bytes;
# byte j holds weight j in its low nibble and weight 16 + j in its high nibble.
# Each weight is d times its nibble minus 8 (a signed 4-bit value in [-8, 7]).

Q4_0_BLOCK_BYTES = 18
Q4_0_BLOCK_WEIGHTS = 32


def q4_0_fields(raw, n_rows: int, k: int):
    """Split a row-major Q4_0 matrix into (d [N, K/32] float64, q [N, K/32, 32] int64).

    Block t of row n starts at byte (n*K/32 + t)*18; q holds the stored nibbles
    in [0, 15] in weight order (the 16 low nibbles, then the 16 high nibbles).
    """
    if k % Q4_0_BLOCK_WEIGHTS:
        raise ValueError("Q4_0 needs K to be a multiple of 32")
    nb = k // Q4_0_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * Q4_0_BLOCK_BYTES:
        raise ValueError("byte count does not match the Q4_0 shape")
    blocks = b.reshape(n_rows, nb, Q4_0_BLOCK_BYTES)
    d = fp16_bits_to_f64(blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8))
    qs = blocks[:, :, 2:].astype(np.int64)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=2)
    return d, q


def dequant_q4_0(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact Q4_0 weights: w[n, 32t + j] = d[n, t] * (q[n, t, j] - 8)  (float64 [N, K])."""
    d, q = q4_0_fields(raw, n_rows, k)
    return (d[:, :, None] * (q - 8)).reshape(n_rows, k)


def dequant_q4_0_f32(raw, n_rows: int, k: int) -> np.ndarray:
    """Q4_0 weights in fp32 (exact: d has 11 significant bits, q - 8 at most 4)."""
    return round_to_f32(dequant_q4_0(raw, n_rows, k))


# ----------------------------------------------------------------------------
# Q4_K: 144-byte super-blocks of 256 weights along K
# ----------------------------------------------------------------------------

Q4_K_BLOCK_BYTES = 144
Q4_K_BLOCK_WEIGHTS = 256


def q4_k_fields(raw, n_rows: int, k: int):
    """Decode a row-major Q4_K matrix into its fields.

    Returns (d, dmin, sc, m, q):
      d, dmin : float64 [N, nb]      the two fp16 super-block scales
      sc, m   : int64   [N, nb, 8]   6-bit scale and min of sub-block j = 0..7
      q       : int64   [N, nb, 256] the 4-bit quant of each weight, in weight order

    Byte layout of one super-block (block b of row n starts at (n*K/256 + b)*144):
      0..1    fp16 d (little-endian)        2..3   fp16 dmin
      4..15   S[0..11]: packed scales/mins  16..143 Q[0..127]: packed nibbles
    Scales and mins: for sub-blocks j < 4, sc_j is the low 6 bits of S[j] and
    m_j the low 6 bits of S[j+4]. For j >= 4 the low 4 bits come from S[j+4]
    (its low nibble for sc_j, its high nibble for m_j) and the top 2 bits come
    from the otherwise unused top 2 bits of S[j-4] (for sc_j) and S[j] (for m_j).
    Quants: the 256 weights form four 64-weight chunks c; byte Q[32c + l] holds
    weight 64c + l in its low nibble and weight 64c + 32 + l in its high nibble.
    """
    if k % Q4_K_BLOCK_WEIGHTS:
        raise ValueError("Q4_K needs K to be a multiple of 256")
    nb = k // Q4_K_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * Q4_K_BLOCK_BYTES:
        raise ValueError("byte count does not match the Q4_K shape")
    blocks = b.reshape(n_rows, nb, Q4_K_BLOCK_BYTES).astype(np.int64)

    d = fp16_bits_to_f64((blocks[:, :, 0] | (blocks[:, :, 1] << 8)).astype(np.uint16))
    dmin = fp16_bits_to_f64((blocks[:, :, 2] | (blocks[:, :, 3] << 8)).astype(np.uint16))

    sc, m = _k_scales_mins(blocks[:, :, 4:16])
    q = _k_nibbles(blocks[:, :, 16:])
    return d, dmin, sc, m, q


def _k_scales_mins(S):
    """The eight 6-bit scales and mins of a K-quant super-block from its 12 packed
    bytes S (int64 [..., 12]); see q4_k_fields for the bit positions."""
    sc = np.empty(S.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty(S.shape[:-1] + (8,), dtype=np.int64)
    for j in range(4):
        sc[..., j] = S[..., j] & 0x3F
        m[..., j] = S[..., j + 4] & 0x3F
    for j in range(4, 8):
        sc[..., j] = (S[..., j + 4] & 0x0F) | ((S[..., j - 4] >> 6) << 4)
        m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j] >> 6) << 4)
    return sc, m


def _k_nibbles(Q):
    """The 256 low 4-bit quants from 128 packed bytes Q (int64 [..., 128]): byte
    Q[32c + l] holds weight 64c + l (low nibble) and 64c + 32 + l (high nibble)."""
    q = np.empty(Q.shape[:-1] + (256,), dtype=np.int64)
    for c in range(4):
        byte = Q[..., 32 * c: 32 * c + 32]
        q[..., 64 * c: 64 * c + 32] = byte & 0x0F
        q[..., 64 * c + 32: 64 * c + 64] = byte >> 4
    return q


def dequant_q4_k(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact Q4_K weights: w = d * sc_j * q - dmin * m_j for weight i of sub-block j.

    float64 [N, K]; weight 256b + 32j + i of row n.
    """
    d, dmin, sc, m, q = q4_k_fields(raw, n_rows, k)
    nb = k // Q4_K_BLOCK_WEIGHTS
    scale = (d[:, :, None] * sc).repeat(32, axis=2)      # [N, nb, 256]
    offset = (dmin[:, :, None] * m).repeat(32, axis=2)
    return (scale * q - offset).reshape(n_rows, nb * 256)


def dequant_q4_k_f32(raw, n_rows: int, k: int) -> np.ndarray:
    """The fp32 dequantization target: each exact weight rounded once to fp32."""
    return round_to_f32(dequant_q4_k(raw, n_rows, k))


# ----------------------------------------------------------------------------
# Q5_K: 176-byte super-blocks of 256 weights along K
# ----------------------------------------------------------------------------
#
# The sibling K-quant of Q4_K (the memra README's model support table lists
# Q4_K_M GGUF files, which mix K-quants, and the memra-bench card flags a Q5_K
# expert mix). Public GGUF layout, restated: the Q4_K header, then a plane of
# 32 bytes holding the fifth bit of every quant, then the Q4_K nibbles.

Q5_K_BLOCK_BYTES = 176


def q5_k_fields(raw, n_rows: int, k: int):
    """Decode a row-major Q5_K matrix into its fields.

    Returns (d, dmin, sc, m, q) with the shapes of q4_k_fields; q is 5-bit.

    Byte layout of one super-block (block b of row n starts at (n*K/256 + b)*176):
      0..1    fp16 d         2..3    fp16 dmin
      4..15   S[0..11]: scales/mins packed exactly as in Q4_K
      16..47  H[0..31]: the high-bit plane
      48..175 Q[0..127]: low nibbles, in Q4_K's order
    Weight 64c + l (c = 0..3, l < 32) has low bits Q[32c + l] & 15 and high bit
    (H[l] >> 2c) & 1; weight 64c + 32 + l has low bits Q[32c + l] >> 4 and high
    bit (H[l] >> (2c + 1)) & 1. The quant is low + 16 * high, in [0, 31].
    """
    if k % Q4_K_BLOCK_WEIGHTS:
        raise ValueError("Q5_K needs K to be a multiple of 256")
    nb = k // Q4_K_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * Q5_K_BLOCK_BYTES:
        raise ValueError("byte count does not match the Q5_K shape")
    blocks = b.reshape(n_rows, nb, Q5_K_BLOCK_BYTES).astype(np.int64)
    d = fp16_bits_to_f64((blocks[:, :, 0] | (blocks[:, :, 1] << 8)).astype(np.uint16))
    dmin = fp16_bits_to_f64((blocks[:, :, 2] | (blocks[:, :, 3] << 8)).astype(np.uint16))
    sc, m = _k_scales_mins(blocks[:, :, 4:16])
    H = blocks[:, :, 16:48]
    q = _k_nibbles(blocks[:, :, 48:])
    for c in range(4):
        q[:, :, 64 * c: 64 * c + 32] += ((H >> (2 * c)) & 1) << 4
        q[:, :, 64 * c + 32: 64 * c + 64] += ((H >> (2 * c + 1)) & 1) << 4
    return d, dmin, sc, m, q


def dequant_q5_k(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact Q5_K weights: w = d * sc_j * q - dmin * m_j, as Q4_K with 5-bit q.

    float64 [N, K]; every weight is an integer multiple of 2^-24 below 2^50.
    """
    d, dmin, sc, m, q = q5_k_fields(raw, n_rows, k)
    nb = k // Q4_K_BLOCK_WEIGHTS
    scale = (d[:, :, None] * sc).repeat(32, axis=2)
    offset = (dmin[:, :, None] * m).repeat(32, axis=2)
    return (scale * q - offset).reshape(n_rows, nb * 256)


def dequant_q5_k_f32(raw, n_rows: int, k: int) -> np.ndarray:
    """The fp32 dequantization target: each exact Q5_K weight rounded once to fp32."""
    return round_to_f32(dequant_q5_k(raw, n_rows, k))


# ----------------------------------------------------------------------------
# Q6_K: 210-byte super-blocks of 256 weights along K
# ----------------------------------------------------------------------------
#
# The other sibling K-quant a Q4_K_M file mixes in (the memra README's model
# support table lists Q4_K_M GGUF files). Public GGUF layout, restated: signed
# 6-bit quants in a 4-bit plane and a 2-bit plane, one int8 scale per 16
# weights, one fp16 d; no min term.

Q6_K_BLOCK_BYTES = 210


def q6_k_fields(raw, n_rows: int, k: int):
    """Decode a row-major Q6_K matrix into its fields.

    Returns (d, sc, q):
      d  : float64 [N, nb]       the fp16 super-block scale
      sc : int64   [N, nb, 16]   the int8 scale of weights 16i .. 16i + 15
      q  : int64   [N, nb, 256]  the signed quant of each weight, in [-32, 31]

    Byte layout of one super-block (block b of row n starts at (n*K/256 + b)*210):
      0..127    L[0..127]: low 4 bits of the quants
      128..191  H[0..63]:  high 2 bits of the quants
      192..207  S[0..15]:  int8 scales
      208..209  fp16 d
    Weight 128h + 32c + l (half h = 0, 1; quarter c = 0..3; l < 32) takes its
    low bits from L[64h + 32(c % 2) + l] (the low nibble for c < 2, the high
    nibble for c >= 2), its high bits from bits 2c, 2c + 1 of H[32h + l], and
    its scale from S[8h + 2c + l // 16]; q = low + 16 * high - 32.
    """
    if k % Q4_K_BLOCK_WEIGHTS:
        raise ValueError("Q6_K needs K to be a multiple of 256")
    nb = k // Q4_K_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * Q6_K_BLOCK_BYTES:
        raise ValueError("byte count does not match the Q6_K shape")
    blocks = b.reshape(n_rows, nb, Q6_K_BLOCK_BYTES).astype(np.int64)
    L = blocks[:, :, 0:128]
    H = blocks[:, :, 128:192]
    sc = blocks[:, :, 192:208].astype(np.uint8).view(np.int8).astype(np.int64)
    d = fp16_bits_to_f64((blocks[:, :, 208] | (blocks[:, :, 209] << 8)).astype(np.uint16))
    q = np.empty((n_rows, nb, 256), dtype=np.int64)
    for h in range(2):
        for c in range(4):
            low_src = L[:, :, 64 * h + 32 * (c % 2): 64 * h + 32 * (c % 2) + 32]
            low = (low_src & 0x0F) if c < 2 else (low_src >> 4)
            high = (H[:, :, 32 * h: 32 * h + 32] >> (2 * c)) & 3
            q[:, :, 128 * h + 32 * c: 128 * h + 32 * c + 32] = low + 16 * high - 32
    return d, sc, q


def dequant_q6_k(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact Q6_K weights: w = d * sc_i * q for weight 16i + t of a super-block.

    float64 [N, K]; every weight is an integer multiple of 2^-24 below 2^40.
    """
    d, sc, q = q6_k_fields(raw, n_rows, k)
    nb = k // Q4_K_BLOCK_WEIGHTS
    scale = (d[:, :, None] * sc).repeat(16, axis=2)
    return (scale * q).reshape(n_rows, nb * 256)


def dequant_q6_k_f32(raw, n_rows: int, k: int) -> np.ndarray:
    """The fp32 dequantization target: each exact Q6_K weight rounded once to fp32
    (d*sc*q can need 25 significant bits)."""
    return round_to_f32(dequant_q6_k(raw, n_rows, k))


def dequant_q8_0_f32(raw, n_rows: int, k: int) -> np.ndarray:
    """Q8_0 weights in fp32 (exact: d has 11 significant bits, q at most 7)."""
    return round_to_f32(dequant_q8_0(raw, n_rows, k))


def dequant_q4_k_bf16_bits(raw, n_rows: int, k: int) -> np.ndarray:
    """The bf16 tile target: RN_bf16(RN_fp32(w)), as uint16 bit patterns."""
    return round_f32_to_bf16_bits(dequant_q4_k_f32(raw, n_rows, k))


# ----------------------------------------------------------------------------
# IQ4_XS: 136-byte super-blocks of 256 weights along K
# ----------------------------------------------------------------------------
#
# The memra README's model support table ships its 35B-A3B MoE in IQ4_XS and
# the memra-bench card's Drafts section carries a UD-IQ4_XS draft of it; the
# pages print no layout, so the one below is the public GGUF format, restated
# here: eight sub-blocks of 32 weights, each with a 6-bit scale ls_j, and
# 4-bit indices into a fixed 16-entry table of signed integers.

IQ4_XS_BLOCK_BYTES = 136
IQ4_XS_BLOCK_WEIGHTS = 256
# the non-linear 4-bit grid of the format (index 0..15 -> integer value)
IQ4_GRID = (-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113)


def iq4_xs_fields(raw, n_rows: int, k: int):
    """Decode a row-major IQ4_XS matrix into its fields.

    Returns (d, ls, q):
      d  : float64 [N, nb]       the fp16 super-block scale
      ls : int64   [N, nb, 8]    6-bit scale of sub-block j = 0..7 (the weight scale is ls - 32)
      q  : int64   [N, nb, 256]  the 4-bit grid index of each weight, in weight order

    Byte layout of one super-block (block b of row n starts at (n*K/256 + b)*136):
      0..1   fp16 d (little-endian)
      2..3   H: 16 bits, bits 2j..2j+1 are the top two bits of ls_j
      4..7   L[0..3]: the low 4 bits of ls_j in the low nibble of L[j/2] for even j,
             in its high nibble for odd j
      8..135 the indices: sub-block j owns bytes 8 + 16j .. 8 + 16j + 15; byte i of
             those holds weight 32j + i in its low nibble and weight 32j + 16 + i in
             its high nibble
    """
    if k % IQ4_XS_BLOCK_WEIGHTS:
        raise ValueError("IQ4_XS needs K to be a multiple of 256")
    nb = k // IQ4_XS_BLOCK_WEIGHTS
    b = _as_bytes(raw)
    if b.size != n_rows * nb * IQ4_XS_BLOCK_BYTES:
        raise ValueError("byte count does not match the IQ4_XS shape")
    blocks = b.reshape(n_rows, nb, IQ4_XS_BLOCK_BYTES).astype(np.int64)
    d = fp16_bits_to_f64((blocks[:, :, 0] | (blocks[:, :, 1] << 8)).astype(np.uint16))
    H = blocks[:, :, 2] | (blocks[:, :, 3] << 8)
    L = blocks[:, :, 4:8]
    ls = np.empty((n_rows, nb, 8), dtype=np.int64)
    for j in range(8):
        low = (L[:, :, j // 2] >> (4 * (j % 2))) & 0x0F
        ls[:, :, j] = low | (((H >> (2 * j)) & 0x3) << 4)
    Q = blocks[:, :, 8:]
    q = np.empty((n_rows, nb, 256), dtype=np.int64)
    for j in range(8):
        byte = Q[:, :, 16 * j: 16 * j + 16]
        q[:, :, 32 * j: 32 * j + 16] = byte & 0x0F
        q[:, :, 32 * j + 16: 32 * j + 32] = byte >> 4
    return d, ls, q


def dequant_iq4_xs(raw, n_rows: int, k: int) -> np.ndarray:
    """Exact IQ4_XS weights: w = d * (ls_j - 32) * grid[q] for weight i of sub-block j.

    float64 [N, K]. d has 11 significant bits, ls - 32 at most 6 and a grid value
    at most 7, so every weight is exact in fp64 (and in fp32).
    """
    d, ls, q = iq4_xs_fields(raw, n_rows, k)
    nb = k // IQ4_XS_BLOCK_WEIGHTS
    grid = np.asarray(IQ4_GRID, dtype=np.int64)
    scale = (d[:, :, None] * (ls - 32)).repeat(32, axis=2)   # [N, nb, 256]
    return (scale * grid[q]).reshape(n_rows, nb * 256)


def qmv_iq4_xs(raw, x_bf16_bits, n_rows: int, k: int) -> np.ndarray:
    """IQ4_XS matrix times bf16 activation rows -> float64 [M, N]."""
    return gemv(dequant_iq4_xs(raw, n_rows, k), bf16_bits_to_f64(x_bf16_bits))


# ----------------------------------------------------------------------------
# matrix-vector products (decode and speculative verify)
# ----------------------------------------------------------------------------


def gemv(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[r, n] = sum_k w[n, k] * x[r, k] in float64 (x: [M, K] or [K])."""
    x2 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x2 @ np.asarray(w, dtype=np.float64).T


def qmv_q8_0(raw, x_f32, n_rows: int, k: int) -> np.ndarray:
    """Q8_0 matrix times fp32 activation rows -> float64 [M, N]."""
    return gemv(dequant_q8_0(raw, n_rows, k), np.asarray(x_f32, dtype=np.float32).astype(np.float64))


def qmv_q4_0(raw, x_bf16_bits, n_rows: int, k: int) -> np.ndarray:
    """Q4_0 matrix times bf16 activation rows -> float64 [M, N]."""
    return gemv(dequant_q4_0(raw, n_rows, k), bf16_bits_to_f64(x_bf16_bits))


def qmv_q5_k(raw, x_bf16_bits, n_rows: int, k: int) -> np.ndarray:
    """Q5_K matrix times bf16 activation rows -> float64 [M, N]."""
    return gemv(dequant_q5_k(raw, n_rows, k), bf16_bits_to_f64(x_bf16_bits))


def qmv_q6_k(raw, x_bf16_bits, n_rows: int, k: int) -> np.ndarray:
    """Q6_K matrix times bf16 activation rows -> float64 [M, N]."""
    return gemv(dequant_q6_k(raw, n_rows, k), bf16_bits_to_f64(x_bf16_bits))


def qmv_q4_k(raw, x_bf16_bits, n_rows: int, k: int) -> np.ndarray:
    """Q4_K matrix times bf16 activation rows -> float64 [M, N]."""
    return gemv(dequant_q4_k(raw, n_rows, k), bf16_bits_to_f64(x_bf16_bits))


# ----------------------------------------------------------------------------
# routed-expert MoE
# ----------------------------------------------------------------------------


def route_top_k(logits, top_k: int):
    """Top-k expert selection with weights renormalised over the selected experts.

    Selection is on the fp32 logits themselves, largest first, ties to the lower
    expert id. The weights are the softmax restricted to the selected experts,
    which equals a softmax over all experts followed by renormalisation over the
    k selected. Returns (ids int32 [T, k], weights float64 [T, k]).
    """
    lg = np.atleast_2d(np.asarray(logits, dtype=np.float32)).astype(np.float64)
    t_count, n_exp = lg.shape
    if not 1 <= top_k <= n_exp:
        raise ValueError("top_k out of range")
    ids = np.empty((t_count, top_k), dtype=np.int32)
    wts = np.empty((t_count, top_k), dtype=np.float64)
    expert = np.arange(n_exp)
    for t in range(t_count):
        order = np.lexsort((expert, -lg[t]))   # primary: logit descending; secondary: id ascending
        sel = order[:top_k]
        e = np.exp(lg[t, sel] - lg[t, sel[0]])
        ids[t] = sel
        wts[t] = e / e.sum()
    return ids, wts


def gather_pairs(ids) -> np.ndarray:
    """All (expert, token) pairs of a routing, sorted by expert then token: int32 [P, 2]."""
    ids = np.atleast_2d(np.asarray(ids))
    pairs = [(int(e), t) for t in range(ids.shape[0]) for e in ids[t]]
    pairs.sort()
    return np.asarray(pairs, dtype=np.int32).reshape(-1, 2)


def silu(g):
    """silu(g) = g / (1 + e^-g)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def expert_matrix(bank_raw, expert: int, n_rows: int, k: int, block_bytes: int = Q4_K_BLOCK_BYTES) -> np.ndarray:
    """Bytes of one expert's matrix inside a bank (experts stored back to back).

    block_bytes: bytes per 256-weight super-block (144 for Q4_K, 136 for IQ4_XS).
    """
    b = _as_bytes(bank_raw)
    size = n_rows * (k // Q4_K_BLOCK_WEIGHTS) * block_bytes
    return b[expert * size:(expert + 1) * size]


def _moe(dequant, block_bytes: int, gate_raw, up_raw, down_raw, logits, x_bf16_bits, hidden: int, ffn: int,
         n_experts: int, top_k: int):
    x = bf16_bits_to_f64(np.atleast_2d(x_bf16_bits))
    t_count = x.shape[0]
    ids, wts = route_top_k(logits, top_k)
    if ids.shape[0] != t_count:
        raise ValueError("logits and activations disagree on the token count")
    y = np.zeros((t_count, hidden), dtype=np.float64)
    cache = {}
    for t in range(t_count):
        for j in range(top_k):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = (
                    dequant(expert_matrix(gate_raw, e, ffn, hidden, block_bytes), ffn, hidden),
                    dequant(expert_matrix(up_raw, e, ffn, hidden, block_bytes), ffn, hidden),
                    dequant(expert_matrix(down_raw, e, hidden, ffn, block_bytes), hidden, ffn),
                )
            wg, wu, wd = cache[e]
            h = silu(wg @ x[t]) * (wu @ x[t])
            y[t] += wts[t, j] * (wd @ h)
    return y, ids, wts


def moe_q4_k(gate_raw, up_raw, down_raw, logits, x_bf16_bits, hidden: int, ffn: int,
             n_experts: int, top_k: int):
    """Routed-expert FFN for each token t, Q4_K experts.

    y_t = sum_j r_j * W_down[e_j] @ (silu(W_gate[e_j] @ x_t) * (W_up[e_j] @ x_t)),
    with (e_j, r_j) from route_top_k and the sum taken in rank order j.
    Returns (y float64 [T, hidden], ids int32 [T, k], weights float64 [T, k]).
    """
    return _moe(dequant_q4_k, Q4_K_BLOCK_BYTES, gate_raw, up_raw, down_raw, logits, x_bf16_bits, hidden, ffn,
                n_experts, top_k)


def moe_iq4_xs(gate_raw, up_raw, down_raw, logits, x_bf16_bits, hidden: int, ffn: int,
               n_experts: int, top_k: int):
    """The same routed-expert FFN with IQ4_XS experts (the format the memra README's
    model support table lists for its 35B-A3B MoE); banks of 136-byte blocks."""
    return _moe(dequant_iq4_xs, IQ4_XS_BLOCK_BYTES, gate_raw, up_raw, down_raw, logits, x_bf16_bits, hidden, ffn,
                n_experts, top_k)


# ----------------------------------------------------------------------------
# prefill-sized product
# ----------------------------------------------------------------------------


def prefill_q4_k(raw, x_bf16_bits, n_rows: int, k: int):
    """Y = X @ W^T for many activation rows.

    Returns (Y_exact, Y_bf16w), both float64 [M, N]: the first with the exact
    weights, the second with the weights rounded to fp32 and then to bf16 (the
    bf16 tile a prefill GEMM multiplies).
    """
    x = bf16_bits_to_f64(x_bf16_bits)
    w = dequant_q4_k(raw, n_rows, k)
    wb = bf16_bits_to_f64(round_f32_to_bf16_bits(round_to_f32(w)))
    return x @ w.T, x @ wb.T


# ----------------------------------------------------------------------------
# comparison metrics used by the parity gates
# ----------------------------------------------------------------------------


def floored_rel_err(y, y_ref, floor_frac: float = 1e-3) -> float:
    """max_i |y_i - yref_i| / max(|yref_i|, tau), tau = floor_frac * max_i |yref_i| per row.

    Rows are the leading axis (one activation row each); a 1-D input is one row.
    """
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    r = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    tau = floor_frac * np.max(np.abs(r), axis=1, keepdims=True)
    den = np.maximum(np.abs(r), tau)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(y - r) / den)) if r.size else 0.0


def frobenius_rel_err(y, y_ref) -> float:
    """||y - yref||_F / ||yref||_F."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    nr = np.linalg.norm(r)
    return float(np.linalg.norm(y - r) / nr) if nr > 0 else float(np.linalg.norm(y - r))
