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

// Activations in bf16: xs holds rows of K/8 swizzled 16-byte granules (gpr per
// row), xsum rows of K/32 sub-block sums (nsub per row).
template <int M>
__device__ __forceinline__ void q4k_chunk_bf16(float (&acc)[M], const int m_act, const uint4 hdr, const uint4 qa,
                                               const uint4 qb, const int ci, const ScaleSel &sel,
                                               const uint4 *__restrict__ xs, const float *__restrict__ xsum,
                                               const int gpr, const int nsub) {
  const ChunkScales cs = chunk_scales(hdr, sel);
  const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  bf16x2 lo[16], hi[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t l = qw[i] & 0x0F0F0F0Fu;
    const uint32_t h = (qw[i] >> 4) & 0x0F0F0F0Fu;
    lo[2 * i] = nibbles_to_bf16x2<false>(l);
    lo[2 * i + 1] = nibbles_to_bf16x2<true>(l);
    hi[2 * i] = nibbles_to_bf16x2<false>(h);
    hi[2 * i + 1] = nibbles_to_bf16x2<true>(h);
  }
#pragma unroll
  for (int r = 0; r < M; ++r) {
    if (r >= m_act) break;
    const uint4 *xr = xs + r * gpr;
    float s_lo = 0.0f, s_hi = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 v = xr[swizzle_granule(ci * 8 + g)];
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 0], __builtin_bit_cast(bf16x2, v.x), s_lo, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 1], __builtin_bit_cast(bf16x2, v.y), s_lo, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 2], __builtin_bit_cast(bf16x2, v.z), s_lo, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 3], __builtin_bit_cast(bf16x2, v.w), s_lo, false);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 v = xr[swizzle_granule(ci * 8 + 4 + g)];
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 0], __builtin_bit_cast(bf16x2, v.x), s_hi, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 1], __builtin_bit_cast(bf16x2, v.y), s_hi, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 2], __builtin_bit_cast(bf16x2, v.z), s_hi, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 3], __builtin_bit_cast(bf16x2, v.w), s_hi, false);
    }
    const float2 xsm = *reinterpret_cast<const float2 *>(xsum + r * nsub + 2 * ci);
    acc[r] = __builtin_fmaf(cs.a0, s_lo, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, xsm.y, acc[r]);
  }
}

// Swizzled position of fp32 granule g (4 activations) when a 64-weight chunk
// spans 16 granules: granule i of chunk c sits at slot i ^ (c & 15), so 16 lanes
// reading the same granule of consecutive chunks hit 16 different bank groups.
__device__ __forceinline__ int swizzle_granule_f32(int g) { return g ^ ((g >> 4) & 15); }

// Activations in fp32 (the MoE down projection's h): hs holds rows of K/4
// swizzled granules (gpr per row), hsum rows of K/32 sub-block sums.
template <int M>
__device__ __forceinline__ void q4k_chunk_f32(float (&acc)[M], const int m_act, const uint4 hdr, const uint4 qa,
                                              const uint4 qb, const int ci, const ScaleSel &sel,
                                              const uint4 *__restrict__ hs, const float *__restrict__ hsum,
                                              const int gpr, const int nsub) {
  const ChunkScales cs = chunk_scales(hdr, sel);
  const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  float s_lo[M], s_hi[M];
#pragma unroll
  for (int r = 0; r < M; ++r) s_lo[r] = s_hi[r] = 0.0f;
  // quant word g holds weights 4g..4g+3 of sub-block 2c (low nibbles) and of 2c+1 (high nibbles)
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const uint32_t w = qw[g];
    const float l0 = (float)(w & 0xFu), l1 = (float)((w >> 8) & 0xFu), l2 = (float)((w >> 16) & 0xFu),
                l3 = (float)((w >> 24) & 0xFu);
    const float h0 = (float)((w >> 4) & 0xFu), h1 = (float)((w >> 12) & 0xFu), h2 = (float)((w >> 20) & 0xFu),
                h3 = (float)(w >> 28);
#pragma unroll
    for (int r = 0; r < M; ++r) {
      if (r >= m_act) break;
      const uint4 v = hs[r * gpr + swizzle_granule_f32(ci * 16 + g)];
      s_lo[r] = __builtin_fmaf(l0, __builtin_bit_cast(float, v.x), s_lo[r]);
      s_lo[r] = __builtin_fmaf(l1, __builtin_bit_cast(float, v.y), s_lo[r]);
      s_lo[r] = __builtin_fmaf(l2, __builtin_bit_cast(float, v.z), s_lo[r]);
      s_lo[r] = __builtin_fmaf(l3, __builtin_bit_cast(float, v.w), s_lo[r]);
      const uint4 u = hs[r * gpr + swizzle_granule_f32(ci * 16 + 8 + g)];
      s_hi[r] = __builtin_fmaf(h0, __builtin_bit_cast(float, u.x), s_hi[r]);
      s_hi[r] = __builtin_fmaf(h1, __builtin_bit_cast(float, u.y), s_hi[r]);
      s_hi[r] = __builtin_fmaf(h2, __builtin_bit_cast(float, u.z), s_hi[r]);
      s_hi[r] = __builtin_fmaf(h3, __builtin_bit_cast(float, u.w), s_hi[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < M; ++r) {
    if (r >= m_act) break;
    const float2 hsm = *reinterpret_cast<const float2 *>(hsum + r * nsub + 2 * ci);
    acc[r] = __builtin_fmaf(cs.a0, s_lo[r], acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, hsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi[r], acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, hsm.y, acc[r]);
  }
}

// Stage M bf16 activation rows of K values (row r at x + r*K) into LDS: swizzled
// granules (gpr = K/8 per row) then, after a barrier, each row's K/32 sub-block
// sums read back from LDS and summed in index order. Loads are batched eight
// granules per thread so their latencies overlap. Ends with a barrier.
template <int M, int NT>
__device__ __forceinline__ void stage_bf16_rows_lds(const uint16_t *__restrict__ x, uint4 *xs, float *xsum,
                                                    const int gpr, const int nsub) {
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const int total = M * gpr;
  for (int base = 0; base < total; base += NT * 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = base + (int)threadIdx.x + i * NT;
      v[i] = xg[g < total ? g : 0];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = base + (int)threadIdx.x + i * NT;
      if (g < total) {
        int r = 0;
#pragma unroll
        for (int q = 1; q < M; ++q) r += g >= q * gpr;
        const int gi = g - r * gpr;
        xs[r * gpr + swizzle_granule(gi)] = v[i];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < M * nsub; t += NT) {
    int r = 0;
#pragma unroll
    for (int q = 1; q < M; ++q) r += t >= q * nsub;
    const int sb = t - r * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xs[r * gpr + swizzle_granule(4 * sb + q)];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += bf16_bits_to_f32(wv[e] & 0xFFFFu);
        s += bf16_bits_to_f32(wv[e] >> 16);
      }
    }
    xsum[r * nsub + sb] = s;
  }
  __syncthreads();
}

// Stage one bf16 activation row (K values) into LDS as swizzled granules plus
// its sub-block sums (fp32, summed in index order), cooperatively.
__device__ __forceinline__ void stage_bf16_row(const uint16_t *__restrict__ x, uint4 *xs, float *xsum, const int gpr,
                                               const int nsub, const int tid, const int nthreads) {
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  for (int g = tid; g < gpr; g += nthreads) xs[swizzle_granule(g)] = xg[g];
  for (int sb = tid; sb < nsub; sb += nthreads) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xg[4 * sb + q];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s += bf16_bits_to_f32(wv[e] & 0xFFFFu);
        s += bf16_bits_to_f32(wv[e] >> 16);
      }
    }
    xsum[sb] = s;
  }
}

// Stage one fp32 activation row (K values) the same way (granules of 4 floats).
__device__ __forceinline__ void stage_f32_row(const float *__restrict__ h, uint4 *hs, float *hsum, const int gpr,
                                              const int nsub, const int tid, const int nthreads) {
  const uint4 *hg = reinterpret_cast<const uint4 *>(h);
  for (int g = tid; g < gpr; g += nthreads) hs[swizzle_granule_f32(g)] = hg[g];
  for (int sb = tid; sb < nsub; sb += nthreads) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = reinterpret_cast<const float4 *>(h)[8 * sb + q];
      s += v.x;
      s += v.y;
      s += v.z;
      s += v.w;
    }
    hsum[sb] = s;
  }
}

}  // namespace qmv
