// Q4_K super-block decoding helpers for the gfx950 kernels.
//
// Super-block (144 bytes, 256 weights): fp16 d | fp16 dmin | S[0..11] packed
// 6-bit scales/mins | Q[0..127] nibbles. Sub-block j (32 weights) has scale sc_j
// and min m_j; weight = d*sc_j*q - dmin*m_j. For j < 4, sc_j = S[j] & 63 and
// m_j = S[j+4] & 63; for j >= 4 the low four bits sit in S[j+4] (low nibble
// for sc_j, high nibble for m_j) and the top two bits in bits 6..7 of S[j-4]
// (sc_j) and S[j] (m_j). Byte Q[32c + l] holds weight 64c + l (low nibble,
// sub-block 2c) and weight 64c + 32 + l (high nibble, sub-block 2c + 1).
#pragma once

#include "qmv_device.h"

namespace qmv {

constexpr int kQ4KBlockBytes = 144;
constexpr int kQ5KBlockBytes = 176;   // Q5_K: the Q4_K header, 32 bytes of fifth bits, the Q4_K nibbles
constexpr int kQ4KBlockWeights = 256;

// Byte-permute selectors and masks that extract, for 64-weight chunk c of a
// super-block, the four 6-bit fields [sc_2c, sc_2c+1, m_2c, m_2c+1] into the
// four bytes of one register with two v_perm_b32 and a few masks, with no
// branch on c (lanes of a wave hold different chunks).
struct ScaleSel {
  uint32_t sel_a, sel_b, m_a, m_hi, m_b, m_b2;
};

__device__ __forceinline__ ScaleSel scale_selectors(int c) {
  ScaleSel s;
  const uint32_t j = 2u * (uint32_t)c;
  if (c < 2) {
    // all four fields are the low 6 bits of S[j], S[j+1], S[j+4], S[j+5]
    s.sel_a = j | (j + 1) << 8 | (j + 4) << 16 | (j + 5) << 24;
    s.sel_b = 0x03020100u;
    s.m_a = 0x3F3F3F3Fu;
    s.m_hi = 0u;
    s.m_b = 0u;
    s.m_b2 = 0u;
  } else {
    // top bits: S[j-4], S[j-3] (scales) and S[j], S[j+1] (mins), bits 6..7
    s.sel_a = (j - 4) | (j - 3) << 8 | j << 16 | (j + 1) << 24;
    // low bits: S[j+4], S[j+5] = bytes j-4, j-3 of S[8..11]; low nibble = scale, high = min
    const uint32_t b = j - 4;
    s.sel_b = b | (b + 1) << 8 | b << 16 | (b + 1) << 24;
    s.m_a = 0u;
    s.m_hi = 0x30303030u;
    s.m_b = 0x00000F0Fu;
    s.m_b2 = 0x0F0F0000u;
  }
  return s;
}

// s0_3, s4_7, s8_11: the three little-endian words of S. Returns the packed
// bytes [sc_2c, sc_2c+1, m_2c, m_2c+1].
__device__ __forceinline__ uint32_t unpack_scale_mins(uint32_t s0_3, uint32_t s4_7, uint32_t s8_11,
                                                      const ScaleSel &s) {
  // v_perm_b32 pool: bytes 0..3 from the second operand, 4..7 from the first,
  // so with (s4_7, s0_3) selector value k picks S[k].
  const uint32_t a = __builtin_amdgcn_perm(s4_7, s0_3, s.sel_a);
  const uint32_t b = __builtin_amdgcn_perm(s8_11, s8_11, s.sel_b);
  return (a & s.m_a) | ((a >> 2) & s.m_hi) | (b & s.m_b) | ((b >> 4) & s.m_b2);
}

// Padded LDS layout of a staged bf16 activation row: 16-byte granules, two
// 64-weight chunks (16 granules) per 17-granule slot. Granule g of chunk ci sits
// at (ci >> 1) * 17 + (ci & 1) * 8 + g, so 16 lanes reading granule g of 16
// consecutive chunks hit 16 distinct bank groups (gfx950 serves 16 lanes of a
// 16-byte read per cycle over 64 banks) while the 8 granules of one chunk stay
// contiguous and are addressed with immediate offsets.
__device__ __forceinline__ int padded_granule(int gi) { return (gi >> 4) * 17 + (gi & 15); }
__host__ __device__ constexpr size_t padded_row_granules(int k) { return layout::q4k_row_granules(k); }

// ---------------------------------------------------------------------------
// Per-chunk arithmetic. A lane holds one 64-weight chunk c of a super-block
// (header `hdr`, quant bytes 32c..32c+31 in `qa`, `qb`) and adds, for each of
// the first `m_act` activation rows r,
//   (d sc_2c) S_lo - (dmin m_2c) X_2c + (d sc_2c+1) S_hi - (dmin m_2c+1) X_2c+1
// to acc[r], where S_lo / S_hi are the exact-quant dot products over the two
// 32-weight sub-blocks of the chunk and X_j the sub-block activation sums. The
// operation sequence per row does not depend on M or m_act.
// ---------------------------------------------------------------------------

// Unpacked header of one chunk: d*sc and dmin*m of its two sub-blocks.
struct ChunkScales {
  float a0, a1, b0, b1;
};

__device__ __forceinline__ ChunkScales chunk_scales(const uint4 hdr, const ScaleSel &sel) {
  const uint32_t scm = unpack_scale_mins(hdr.y, hdr.z, hdr.w, sel);
  const float d = fp16_bits_to_f32(hdr.x & 0xFFFFu);
  const float dmin = fp16_bits_to_f32(hdr.x >> 16);
  ChunkScales c;
  c.a0 = d * (float)(scm & 0xFFu);
  c.a1 = d * (float)((scm >> 8) & 0xFFu);
  c.b0 = dmin * (float)((scm >> 16) & 0xFFu);
  c.b1 = dmin * (float)(scm >> 24);
  return c;
}

}  // namespace qmv
