// IQ4_XS device helpers shared by the GEMV and the routed-expert MoE kernels.
//
// A 136-byte super-block holds 256 weights along K (public GGUF layout; the
// memra README's model support table lists its 35B-A3B MoE in IQ4_XS):
//   bytes 0..1   fp16 d
//   bytes 2..3   H: bits 2j..2j+1 are bits 4..5 of the 6-bit scale ls_j
//   bytes 4..7   L: bits 4j..4j+3 of this little-endian word are bits 0..3 of ls_j
//   bytes 8..135 grid indices: sub-block j (32 weights) owns 16 bytes; byte i of
//                them holds weight 32j + i (low nibble) and 32j + 16 + i (high)
// and weight = d * (ls_j - 32) * grid[index] with a fixed 16-value grid.
#pragma once

#include "qmv_device.h"

namespace qmv {
namespace iq4xs {

constexpr int kIQ4XSBlockBytes = 136;
constexpr int kTableEntries = 256;  // LDS table: one bf16 pair per index byte

// The format's 16 grid values, packed as signed bytes (index 4w + b in byte b of word w).
constexpr uint32_t kGrid0 = 0xBFAD9881u;  // -127, -104,  -83,  -65
constexpr uint32_t kGrid1 = 0xF6EADDCFu;  //  -49,  -35,  -22,  -10
constexpr uint32_t kGrid2 = 0x26190D01u;  //    1,   13,   25,   38
constexpr uint32_t kGrid3 = 0x71594535u;  //   53,   69,   89,  113

__device__ __forceinline__ uint32_t grid_bf16(uint32_t idx) {
  const uint32_t w = idx < 4 ? kGrid0 : idx < 8 ? kGrid1 : idx < 12 ? kGrid2 : kGrid3;
  const int v = (int)(int8_t)(uint8_t)(w >> (8 * (idx & 3)));
  return __builtin_bit_cast(uint32_t, (float)v) >> 16;   // exact: |v| < 2^8
}

// x staging: row r's sub-block s lives at granule r * row_gran + 4 s + (s >> 2)
// (one pad granule after every 4 sub-blocks: the 16 lanes of a row reading
// granule q of 16 consecutive sub-blocks hit 16 distinct bank groups).
__device__ __forceinline__ int x_slot(int s) { return 4 * s + (s >> 2); }
__host__ __device__ constexpr int row_granules(int nsub) { return layout::iq4xs_row_granules(nsub); }

// Pair-interleave one 32-value sub-block: in granules g0..g3 hold x[0..31]; out
// granule t holds the pairs (x[4t + e], x[16 + 4t + e]) for e < 4.
__device__ __forceinline__ void interleave(const uint4 g0, const uint4 g1, const uint4 g2, const uint4 g3,
                                           uint4 (&o)[4]) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;   // (b.lo16, a.lo16), (b.hi16, a.hi16)
  o[0] = make_uint4(__builtin_amdgcn_perm(g2.x, g0.x, kLo), __builtin_amdgcn_perm(g2.x, g0.x, kHi),
                    __builtin_amdgcn_perm(g2.y, g0.y, kLo), __builtin_amdgcn_perm(g2.y, g0.y, kHi));
  o[1] = make_uint4(__builtin_amdgcn_perm(g2.z, g0.z, kLo), __builtin_amdgcn_perm(g2.z, g0.z, kHi),
                    __builtin_amdgcn_perm(g2.w, g0.w, kLo), __builtin_amdgcn_perm(g2.w, g0.w, kHi));
  o[2] = make_uint4(__builtin_amdgcn_perm(g3.x, g1.x, kLo), __builtin_amdgcn_perm(g3.x, g1.x, kHi),
                    __builtin_amdgcn_perm(g3.y, g1.y, kLo), __builtin_amdgcn_perm(g3.y, g1.y, kHi));
  o[3] = make_uint4(__builtin_amdgcn_perm(g3.z, g1.z, kLo), __builtin_amdgcn_perm(g3.z, g1.z, kHi),
                    __builtin_amdgcn_perm(g3.w, g1.w, kLo), __builtin_amdgcn_perm(g3.w, g1.w, kHi));
}

// Scale of sub-block j of a super-block whose first 8 bytes are hdr:
// d * (ls_j - 32), exact in fp32 (11 + 6 significant bits).
__device__ __forceinline__ float sub_scale(const uint2 hdr, const int sh_lo, const int sh_hi) {
  const uint32_t ls = ((hdr.y >> sh_lo) & 15u) | (((hdr.x >> sh_hi) & 3u) << 4);
  return fp16_bits_to_f32(hdr.x & 0xFFFFu) * (float)((int)ls - 32);
}

// One unit's global data for a lane: the block's 8 header bytes and the
// sub-block's 16 index bytes (blocks are only 8-byte aligned: 8-byte loads).
struct Unit {
  uint2 hdr, q0, q1;
};

// bp: the super-block; qoff = 8 + 16 j: the lane's sub-block j.
__device__ __forceinline__ void load_unit(const uint8_t *__restrict__ bp, const int qoff, Unit &r) {
  r.hdr = *reinterpret_cast<const uint2 *>(bp);
  r.q0 = *reinterpret_cast<const uint2 *>(bp + qoff);
  r.q1 = *reinterpret_cast<const uint2 *>(bp + qoff + 8);
}

// Byte B of w times 4 (the table's byte offset for that index byte) in one
// instruction: the shift reads the byte through an SDWA source select.
template <int B>
__device__ __forceinline__ uint32_t byte_x4(const uint32_t w) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, 2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  return r;
}

// Byte B of w times 8 (the offset of a table of 8-byte entries), one instruction.
template <int B>
__device__ __forceinline__ uint32_t byte_x8(const uint32_t w) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  else if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  else if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  return r;
}

template <int B>
__device__ __forceinline__ bf16x2 table_pair(const uint8_t *__restrict__ tbl_bytes, const uint32_t w) {
  return __builtin_bit_cast(bf16x2, *reinterpret_cast<const uint32_t *>(tbl_bytes + byte_x4<B>(w)));
}

// The four table entries of index word w (four index bytes).
struct Pairs {
  bf16x2 e[4];
};

__device__ __forceinline__ Pairs word_pairs(const uint8_t *__restrict__ tbl_bytes, const uint32_t w) {
  return Pairs{{table_pair<0>(tbl_bytes, w), table_pair<1>(tbl_bytes, w), table_pair<2>(tbl_bytes, w),
                table_pair<3>(tbl_bytes, w)}};
}

__device__ __forceinline__ float pairs_dot(const Pairs &p, const uint4 xp, float s) {
  s = __builtin_amdgcn_fdot2_f32_bf16(p.e[0], __builtin_bit_cast(bf16x2, xp.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p.e[1], __builtin_bit_cast(bf16x2, xp.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p.e[2], __builtin_bit_cast(bf16x2, xp.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(p.e[3], __builtin_bit_cast(bf16x2, xp.w), s, false);
  return s;
}

}  // namespace iq4xs
}  // namespace qmv
