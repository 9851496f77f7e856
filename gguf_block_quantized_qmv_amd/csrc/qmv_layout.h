// Sizes the host works out before a launch: the LDS a kernel stages its
// activations in, the workspace layouts of the routed-expert entry points and
// the K-split plan of the prefill GEMM. Plain C++ with no HIP dependency, so
// the argument checks (qmv_api.cpp, built with g++) and the kernel files use
// the same arithmetic: a size the host checks is the size the kernel uses.
// Every function depends on its arguments only -- never on the device -- so a
// call's numerical program is fixed by its shape.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/qmv.h"

#if defined(__HIPCC__)
#define QMV_HD __host__ __device__
#else
#define QMV_HD
#endif

namespace qmv {
namespace layout {

constexpr size_t kLdsBudget = QMV_LDS_X_BYTES;   // dynamic LDS any one workgroup may take
constexpr size_t kLdsPerCu = 160 * 1024;          // LDS of one gfx950 compute unit

// Largest matrix any entry point takes: launch grids and row indices stay
// inside 32 bits with room to spare (2^40 weights are far beyond one GPU).
constexpr bool matrix_in_range(int n, int k) {
  return n <= QMV_MAX_MATRIX_ROWS && k <= QMV_MAX_MATRIX_K && (size_t)n * (size_t)k <= ((size_t)1 << 40);
}

// ---- dense GEMV activation staging ----------------------------------------

// Q4_K / Q5_K / Q4_0: a bf16 row in 16-byte granules, two 64-weight chunks
// (16 granules) per 17-granule slot, then the row's per-32 sums (fp32).
QMV_HD constexpr size_t q4k_row_granules(int k) { return (size_t)(k >> 7) * 17; }
constexpr size_t q4k_x_lds(int m, int k) {
  return (size_t)m * (q4k_row_granules(k) * 16 + (size_t)(k >> 5) * 4);
}

// Q6_K: a bf16 row with an XOR swizzle and no pad, then the per-16 sums.
constexpr size_t q6k_x_lds(int m, int k) { return (size_t)m * ((size_t)k * 2 + (size_t)(k >> 4) * 4); }

// Q8_0: the fp32 rows as they are.
constexpr size_t q80_x_lds(int m, int k) { return (size_t)m * (size_t)k * 4; }

// IQ4_XS: pair-interleaved bf16 sub-blocks, one pad granule after every 4
// sub-blocks, next to a static 256-entry (1 KiB) LDS table of bf16 pairs.
QMV_HD constexpr int iq4xs_row_granules(int nsub) { return 4 * nsub + nsub / 4; }
constexpr size_t kIq4xsTableBytes = 256 * 4;
constexpr size_t iq4xs_gemv_dyn_lds(int m, int k) { return (size_t)m * iq4xs_row_granules((k >> 8) * 8) * 16; }
constexpr size_t iq4xs_gemv_lds(int m, int k) { return kIq4xsTableBytes + iq4xs_gemv_dyn_lds(m, k); }

// ---- routed-expert decode (Q4_K and IQ4_XS experts) ------------------------

// Workspace: the routing tables launch 1 writes for launch 2, then h as fp32
// [t * top_k][ffn] in gather-list order.
constexpr size_t kMoeTableBytes = 4096;
constexpr size_t moe_workspace(int t, int ffn, int top_k) {
  return kMoeTableBytes + (size_t)t * (size_t)top_k * (size_t)ffn * 4;
}
// The gate/up launch routes every token in LDS: one row of 8-byte composite
// keys per token, QMV_MOE_MAX_EXPERTS of them.
constexpr size_t kMoeRouteBytesPerToken = (size_t)QMV_MOE_MAX_EXPERTS * 8;
// Q4_K: x rows staged as in the dense GEMV, then the routing rows; h rows in
// 64-value chunks of 17 granules (fp32) plus their per-32 sums. Static LDS
// stays under 4 KiB.
constexpr size_t q4k_moe_gate_up_lds(int t, int hidden) {
  return q4k_x_lds(t, hidden) + (size_t)t * kMoeRouteBytesPerToken;
}
constexpr size_t q4k_moe_down_lds(int pairs, int ffn) {
  return (size_t)pairs * ((size_t)(ffn >> 6) * 17 * 16 + (size_t)(ffn >> 5) * 4);
}
constexpr bool q4k_moe_fits_lds(int t, int hidden, int ffn, int top_k) {
  return q4k_moe_gate_up_lds(t, hidden) <= kLdsBudget - 4096 && q4k_moe_down_lds(t * top_k, ffn) <= kLdsBudget - 4096;
}
// Device scratch of the allocation-free routed-expert entry point: one fixed
// array per GPU. Every call that passes q4k_moe_fits_lds fits in it: the down
// stage holds t * top_k * ffn * 4.375 bytes of h rows and sums in LDS, at most
// kLdsBudget - 4096, so h (4 bytes per value) is at most 146,051 bytes and the
// workspace at most 4096 + 146,051 < 160 KiB.
constexpr size_t kMoeNoAllocBytes = QMV_MOE_NOALLOC_BYTES;
static_assert(kMoeNoAllocBytes == 160 * 1024, "the bound derived above");
// IQ4_XS: x rows pair-interleaved as in its GEMV; h in fp32 with a 144-byte
// sub-block stride. Static LDS stays under 8 KiB.
constexpr size_t iq4xs_moe_gate_up_lds(int t, int hidden) {
  return (size_t)t * iq4xs_row_granules(hidden >> 5) * 16 + (size_t)t * kMoeRouteBytesPerToken;
}
constexpr size_t iq4xs_moe_down_lds(int pairs, int ffn) { return (size_t)pairs * (size_t)(ffn >> 5) * 9 * 16; }
constexpr bool iq4xs_moe_fits_lds(int t, int hidden, int ffn, int top_k) {
  return iq4xs_moe_gate_up_lds(t, hidden) <= kLdsBudget - 8192 &&
         iq4xs_moe_down_lds(t * top_k, ffn) <= kLdsBudget - 8192;
}

// ---- routed-expert prefill (grouped-expert products) ----------------------

constexpr int kGroupChunk = 16;     // pairs per chunk (the MFMA's M)
constexpr int kGroupChunk32 = 32;   // pairs per wide gate/up chunk

// Workspace regions, each 256-byte aligned: routing (ids, weights), per-expert
// counts and offsets, the two chunk lists, the pair list, h [P][ffn] fp32 and
// the per-pair down products z [P][hidden] fp32, P = t * top_k.
struct GroupLayout {
  size_t ids, wts, cnt, off, choff, chunks, choff32, chunks32, plist, h, z, total;
};
constexpr size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
inline GroupLayout group_layout(int t, int hidden, int ffn, int n_experts, int top_k) {
  GroupLayout L{};
  const size_t P = (size_t)t * (size_t)top_k, E = (size_t)n_experts;
  const size_t maxch = (P + kGroupChunk - 1) / kGroupChunk + E;
  const size_t maxch32 = (P + kGroupChunk32 - 1) / kGroupChunk32 + E;
  size_t o = 0;
  L.ids = o; o += round256(P * 4);
  L.wts = o; o += round256(P * 4);
  L.cnt = o; o += round256(E * 4);
  L.off = o; o += round256(E * 4);
  L.choff = o; o += round256((E + 1) * 4);
  L.chunks = o; o += round256(maxch * 8);
  L.choff32 = o; o += round256((E + 1) * 4);
  L.chunks32 = o; o += round256(maxch32 * 8);
  L.plist = o; o += round256(P * 4);
  L.h = o; o += round256(P * (size_t)ffn * 4);
  L.z = o; o += round256(P * (size_t)hidden * 4);
  L.total = o;
  return L;
}
// LDS: chunk rows of x (bf16) and their per-32 sums; for down, h as three bf16
// parts and its per-32 sums. Rows are padded by kGroupRowPad granules, so that
// a row's stride is 1 mod 16 granules: the MFMA fragment reads (16 lanes, one
// granule of 16 consecutive rows) fall in 16 distinct 16-byte bank groups
// (gfx950 serves 16 lanes of a 16-byte LDS read per clock, group = granule mod
// 16). A pad of 4 put those 16 lanes in 4 groups, a 4-way conflict.
// The per-32 sums are rows of K/32 + kGroupSumPad floats: each 4-byte read
// takes the sums of 4 pair rows 4 apart (one per 16-lane group), and an odd
// row stride puts them in 4 distinct banks (with K/32 floats per row, a
// multiple of 8, they shared a bank or two).
constexpr int kGroupRowPad = 1, kGroupSumPad = 1;
constexpr size_t group_gate_up_lds(int chunk, int hidden) {
  return (size_t)chunk * ((size_t)(hidden >> 3) + kGroupRowPad) * 16 +
         (size_t)chunk * ((size_t)(hidden >> 5) + kGroupSumPad) * 4;
}
constexpr size_t group_down_lds(int ffn) {
  return (size_t)3 * kGroupChunk * ((size_t)(ffn >> 3) + kGroupRowPad) * 16 +
         (size_t)kGroupChunk * ((size_t)(ffn >> 5) + kGroupSumPad) * 4;
}
constexpr bool group_fits_lds(int hidden, int ffn) {
  return group_gate_up_lds(kGroupChunk, hidden) <= kLdsBudget && group_down_lds(ffn) <= kLdsBudget;
}

// ---- prefill GEMM: tiles and the K split of the last round -----------------

// 256 x 128 output tiles, one 1024-thread workgroup each. The plan assumes the
// workgroup slots of a 256-CU MI355X at one workgroup per CU; it is a fixed
// constant, not a device query, so the summation order -- and so the bits --
// depends only on (m, n, k).
constexpr int kPrefillTileM = 256, kPrefillTileN = 128;
constexpr int kPrefillSlots = 256;

// Tiles [0, t_main) run whole. The r_tiles tiles after them (when the tile
// count is not a multiple of the slots) run as `splits` parts of whole
// 256-value K blocks each, so that the last round fills the slots; a second
// launch adds a tile's parts in K order. splits == 0: every tile whole.
struct PrefillPlan {
  int t_main, r_tiles, splits;
};
inline size_t prefill_tiles(int m, int n) {
  return (((size_t)n + kPrefillTileN - 1) / kPrefillTileN) * (((size_t)m + kPrefillTileM - 1) / kPrefillTileM);
}
// The caller has bounded prefill_tiles(m, n) to fit an int.
inline PrefillPlan prefill_plan(int m, int n, int k) {
  const int tiles = (int)prefill_tiles(m, n);
  PrefillPlan p{tiles, 0, 0};
  const int t_main = tiles / kPrefillSlots * kPrefillSlots, r = tiles - t_main;
  if (r == 0) return p;
  const int nkb = k / 256;   // parts are runs of whole K blocks
  const int most = kPrefillSlots / r < nkb ? kPrefillSlots / r : nkb;
  if (most < 2) return p;
  // the longest part decides the round; the fewest parts that reach it keep
  // the partial sums (and the second launch's reads) smallest
  const int longest = (nkb + most - 1) / most;
  int splits = (nkb + longest - 1) / longest;
  if (splits < 2) splits = 2;
  return PrefillPlan{t_main, r, splits};
}
inline size_t prefill_plan_bytes(const PrefillPlan &p) {
  return (size_t)p.splits * (size_t)p.r_tiles * kPrefillTileM * kPrefillTileN * sizeof(float);
}
// Largest product the prefill takes: activation granules (8 bf16) are indexed
// in 32 bits (every index below m * k / 8) and the tile count must fit an int.
inline bool prefill_in_range(int m, int n, int k) {
  return (size_t)m * (size_t)(k >> 3) <= ((size_t)1 << 32) && prefill_tiles(m, n) <= (size_t)INT32_MAX;
}

}  // namespace layout
}  // namespace qmv
