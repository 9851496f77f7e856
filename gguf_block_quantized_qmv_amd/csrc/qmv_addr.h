// Where every kernel reads its quantized weights: the launch plan of each entry
// point (template choice, workgroup size, grid) and, per lane, the byte offset
// of every weight load it issues. Plain C++ with no HIP dependency: the kernels
// form their load addresses with these functions, and a host program built
// with g++ enumerates the same functions over every lane, step and
// instantiation a launch uses and checks that each load stays inside the
// weights. Offsets are in bytes from the start of the weight array the entry
// point receives.
//
// Block formats are the public GGUF ones (memra summary page, the format
// table): Q4_K 144 bytes per 256 weights, Q5_K 176, Q6_K 210, IQ4_XS 136,
// Q4_0 and Q8_0 18 and 34 bytes per 32.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qmv_layout.h"

#if defined(__HIPCC__)
#define QMV_HDI __host__ __device__ inline __attribute__((always_inline))
#else
#define QMV_HDI inline
#endif

namespace qmv {
namespace addr {

constexpr int kQ4KBytes = 144, kQ5KBytes = 176, kQ6KBytes = 210, kIQ4XSBytes = 136;
constexpr int kQ40Bytes = 18, kQ80Bytes = 34;

// A byte range [off, off + len) relative to some base; len 0: nothing read.
struct Window {
  int off, len;
};

// ---- dense GEMV: Q4_K, Q5_K, Q4_0 ---------------------------------------------
//
// G lanes (16 or 32) own one output row; at step s lane j reads chunk j % 4 of
// block (G/4) s + j / 4 of its row (for Q4_0 a "block" is a group of eight
// 18-byte blocks, 144 bytes). Loads that have no block of their own -- steps
// past the row, lanes past a partial last step, rows past the matrix -- read
// the last block of the lane's row (of the last row past the matrix).

constexpr int kFmtQ4K = 0, kFmtQ5K = 1, kFmtQ40 = 2;
QMV_HDI constexpr int dense_block_bytes(int fmt) { return fmt == kFmtQ5K ? kQ5KBytes : kQ4KBytes; }

// Steps of loads in flight (the register ring), by format, rows m and lanes G.
QMV_HDI constexpr int dense_depth(int fmt, int m, int G) {
  return fmt == kFmtQ5K ? (m == 1 ? (G == 16 ? 5 : 2) : 4) : (G == 16 ? 5 : 2);
}
constexpr int kDenseMinThreads = 256;
QMV_HDI constexpr int dense_max_threads(int m) { return m == 1 ? 512 : 768; }
QMV_HDI constexpr int q6_max_threads(int m) { return m == 1 ? 512 : 640; }

// Rows per workgroup: every CU gets the same rows when n splits over 256 CUs
// into q workgroups of whole waves with min..max threads that fit the LDS q at
// a time; otherwise min threads.
inline int balanced_rows(int n, int G, size_t lds, int max_threads) {
  const int dflt = kDenseMinThreads / G;
  if (n % 256 != 0) return dflt;
  const int per_cu = n / 256;
  for (int q = 1; q <= 8; ++q) {
    if (per_cu % q != 0) continue;
    const int threads = (per_cu / q) * G;
    if (threads > max_threads || threads % 64 != 0) continue;
    if (threads < kDenseMinThreads || (size_t)q * lds > layout::kLdsBudget) break;
    return per_cu / q;
  }
  return dflt;
}

// ns > 0: rows of exactly ns steps, the step loop unrolled; ns == 0: runtime
// step loop (full: every step whole).
struct GemvPlan {
  int G, ns, depth, rows;
  bool full;
  unsigned grid;
};
// 16 lanes per row up to k = 8192 (1..8 steps of 4 blocks), 32 beyond (5..9
// steps of 8 blocks unrolled up to k = 18432, a runtime loop after).
inline GemvPlan dense_gemv_plan(int fmt, int m, int n, int k) {
  GemvPlan p{};
  const int nblk = k >> 8;
  if (k <= 8192) {
    p.G = 16;
    p.ns = (nblk + 3) / 4;
  } else {
    p.G = 32;
    const int s = (nblk + 7) / 8;
    p.ns = s <= 9 ? s : 0;
    p.full = p.ns == 0 && nblk % 8 == 0;
  }
  p.depth = dense_depth(fmt, m, p.G);
  p.rows = balanced_rows(n, p.G, layout::q4k_x_lds(m, k), dense_max_threads(m));
  p.grid = (unsigned)((n + p.rows - 1) / p.rows);
  return p;
}

// Output row of thread tid of workgroup bid (nthreads per workgroup).
QMV_HDI int lane_row(int bid, int tid, int nthreads, int G) { return bid * (nthreads / G) + tid / G; }

// Two matrices of n rows on one activation (qmv_q4_k_pair): the launch covers
// 2n rows, rows [0, n) of matrix 0 then [n, 2n) of matrix 1; each is row `row`
// of its own matrix (rows past 2n are past matrix 1, inactive in dense_lane).
struct PairRow {
  int half, row;
};
QMV_HDI PairRow pair_row(int row2, int n) { return row2 < n ? PairRow{0, row2} : PairRow{1, row2 - n}; }

struct DenseLane {
  int c, jb, nsteps;
  bool active, last_ok;
  size_t row_base, blk_off;   // the lane's row, and its block at step 0 within the row
  size_t fb;                  // the fallback block
};
// j: the lane's index within its row's G lanes.
QMV_HDI DenseLane dense_lane(int G, int ns, int fmt, int n, int nblk, int row, int j) {
  const int bps = G / 4, bb = dense_block_bytes(fmt);
  DenseLane l;
  l.c = j & 3;
  l.jb = j >> 2;
  l.active = row < n;
  l.nsteps = ns > 0 ? ns : (nblk + bps - 1) / bps;
  // with ns > 0 only the last step can be partial: lanes past its blocks skip it
  l.last_ok = l.jb < nblk - (l.nsteps - 1) * bps;
  l.fb = ((size_t)(l.active ? row : n - 1) * (size_t)nblk + (size_t)(nblk - 1)) * bb;
  l.row_base = (size_t)(l.active ? row : 0) * (size_t)nblk * bb;
  l.blk_off = (size_t)l.jb * bb;
  return l;
}
// Whether step t of a lane (active, last_ok, nsteps, jb as in DenseLane) has
// a block of its own.
QMV_HDI bool dense_step_ok(bool active, bool last_ok, int nsteps, int jb, int ns, bool full, int G, int nblk, int t) {
  if (ns > 0) return active && t < ns && (t < ns - 1 || last_ok);
  return active && t < nsteps && (full || t * (G / 4) + jb < nblk);
}
// Bytes from the lane's block at step 0 to its block at step t. The block step
// t reads is row_base + blk_off + dense_step_offset when dense_step_ok, else
// the fallback fb.
QMV_HDI size_t dense_step_offset(int G, int fmt, int t) { return (size_t)(t * (G / 4)) * dense_block_bytes(fmt); }
// The two ranges one step reads from its block, for chunk c: [0] the block
// header (Q5_K: with its 32 bytes of fifth bits; Q4_0: the chunk's pair of
// 18-byte blocks, header and quants together), [1] the chunk's 32 quant bytes.
QMV_HDI constexpr Window dense_window(int fmt, int c, int i) {
  if (fmt == kFmtQ40) return i == 0 ? Window{36 * c, 36} : Window{36 * c, 0};
  if (fmt == kFmtQ5K) return i == 0 ? Window{0, 48} : Window{48 + 32 * c, 32};
  return i == 0 ? Window{0, 16} : Window{16 + 32 * c, 32};
}

// ---- Q6_K GEMV -----------------------------------------------------------------
//
// As the dense GEMV, with units (h, p) of a 210-byte block in place of chunks.
// 210 = 2 mod 4, so a block starts 0 or 2 bytes into a dword; a step moves an
// even number of blocks, so that offset (sb) is fixed per lane, and the
// fallback of a lane is block 0 or 1 of the matrix, whichever has its offset.

QMV_HDI constexpr int q6_depth(int m, int G) { return m == 1 ? (G == 16 ? 5 : 2) : 3; }

inline GemvPlan q6_gemv_plan(int m, int n, int k) {
  GemvPlan p{};
  const int nblk = k >> 8;
  if (k <= 8192) {
    p.G = 16;
    p.ns = (nblk + 3) / 4;
  } else {
    p.G = 32;
    const int s = (nblk + 7) / 8;
    p.ns = s <= 9 ? s : 0;
  }
  p.depth = q6_depth(m, p.G);
  p.rows = balanced_rows(n, p.G, layout::q6k_x_lds(m, k), q6_max_threads(m));
  p.grid = (unsigned)((n + p.rows - 1) / p.rows);
  return p;
}

struct Q6Lane {
  int h, p, jb, nsteps, sb;
  bool active, last_ok;
  size_t base, fb;
};
QMV_HDI Q6Lane q6_lane(int G, int ns, int n, int nblk, int row, int j) {
  const int bps = G / 4;
  Q6Lane l;
  const int u = j & 3;
  l.h = u >> 1;
  l.p = u & 1;
  l.jb = j >> 2;
  l.active = row < n;
  l.nsteps = ns > 0 ? ns : (nblk + bps - 1) / bps;
  l.last_ok = l.jb < nblk - (l.nsteps - 1) * bps;
  // parity of the lane's block index row * nblk + jb (a one-block matrix has
  // only block 0, whose offset is 0)
  const int r = l.active ? row : 0;
  const int par = (n > 1 || nblk > 1) ? (((r & nblk) ^ l.jb) & 1) : 0;
  l.sb = 2 * par;
  l.fb = (size_t)par * kQ6KBytes;
  l.base = ((size_t)r * (size_t)nblk + (size_t)l.jb) * kQ6KBytes;
  return l;
}
QMV_HDI bool q6_step_ok(const Q6Lane &l, int G, int nblk, int t) {
  return l.active && t < l.nsteps && t * (G / 4) + l.jb < nblk;
}
// The block step t reads: base + q6_step_offset when q6_step_ok, else fb.
QMV_HDI size_t q6_step_offset(int G, int t) { return (size_t)(t * (G / 4)) * kQ6KBytes; }
// The reads of unit (h, p) of a block. q6_run: the first five, relative to the
// dword-aligned start of the block's window (the block's first byte minus sb):
// three 20-byte windows around the quant runs, the two dwords at the scales,
// and one more dword (the third when the scales start mid-dword, the second
// again otherwise). q6_window: all six relative to the block's first byte, the
// last being the 2-byte d.
// Each offset is a base, a part fixed by h and a part fixed by p: the kernel
// adds them to its pointer one at a time, which keeps its address registers
// fewest.
QMV_HDI int q6_run_base(int i) {
  switch (i) {
    case 0: return 0;
    case 1: return 32;
    case 2: return 128;
    default: return 192;
  }
}
QMV_HDI int q6_run_h(int h, int i) { return i < 2 ? 64 * h : (i == 2 ? 32 * h : 8 * h); }
QMV_HDI int q6_run_p(int p, int i) { return i < 3 ? 16 * p : 0; }
QMV_HDI int q6_run(int sb, int h, int p, int i) {
  return q6_run_base(i) + q6_run_h(h, i) + q6_run_p(p, i) + (i == 4 ? (sb ? 8 : 4) : 0);
}
QMV_HDI Window q6_window(int sb, int h, int p, int i) {
  if (i == 5) return Window{208, 2};
  return Window{q6_run(sb, h, p, i) - sb, i < 3 ? 20 : (i == 3 ? 8 : 4)};
}
constexpr int kQ6Windows = 6;

// ---- IQ4_XS GEMV -----------------------------------------------------------------
//
// G lanes (16 or 32) own one row; lane l takes the 32-weight sub-blocks
// l + G t, i.e. sub-block l & 7 of block (l >> 3) + (G / 8) t. Units past the
// lane's last re-read sub-block l & 7 of the row's first block (of row 0 past
// the matrix).

constexpr int kIq4GemvDepth = 2;   // units of loads in flight per lane
struct Iq4Plan {
  int G, threads, depth;
  unsigned grid;
};
inline Iq4Plan iq4_gemv_plan(int m, int n, int k) {
  Iq4Plan p{};
  p.depth = kIq4GemvDepth;
  if (k <= 8192) p.G = 16, p.threads = 256;
  else if (2 * layout::iq4xs_gemv_lds(m, k) > layout::kLdsPerCu) p.G = 32, p.threads = 512;
  else p.G = 32, p.threads = 256;
  const int rows = p.threads / p.G;
  p.grid = (unsigned)((n + rows - 1) / rows);
  return p;
}

struct Iq4Lane {
  size_t row_base, lane_base;
  int qoff, nlive, unit_bytes;
};
// row: the row the lane reads, counted from the start of the array (an
// expert's rows follow the previous expert's); the caller has already put a
// row that exists in place of one past its matrix.
QMV_HDI Iq4Lane iq4_lane(int G, int nblk, size_t row, int l) {
  Iq4Lane r;
  const size_t row_bytes = (size_t)nblk * kIQ4XSBytes;
  r.row_base = row * row_bytes;
  r.lane_base = r.row_base + (size_t)(l >> 3) * kIQ4XSBytes;
  r.qoff = 8 + 16 * (l & 7);
  const int nsub = nblk * 8;
  r.nlive = l < nsub ? (nsub - l + G - 1) / G : 0;
  r.unit_bytes = (G / 8) * kIQ4XSBytes;
  return r;
}
// Unit t: live (t < nlive) at lane_base + iq4_unit_offset, else the row's
// first block (row_base).
QMV_HDI size_t iq4_unit_offset(int t, int unit_bytes) { return (size_t)t * unit_bytes; }
// Unit slots a lane runs through, the ring refilled depth units ahead.
QMV_HDI int iq4_slots(int G, int nblk, int depth) {
  const int nmax = (nblk * 8 + G - 1) / G;
  return (nmax + depth - 1) / depth * depth;
}
// A unit's reads from its block: the 8-byte header and the sub-block's 16
// quant bytes (two 8-byte loads).
QMV_HDI Window iq4_window(int qoff, int i) { return i == 0 ? Window{0, 8} : Window{qoff, 16}; }

// ---- routed-expert decode (Q4_K experts) ---------------------------------------
//
// Gate/up: workgroup (x, y) takes rows R x .. R x + R - 1 of the y-th distinct
// expert e, L lanes per row (L / 4 blocks per step), every load guarded by the
// row and block existing: L = 32 and R = 8 for one token, L = 16 and R = 16
// for two to four. One token's few expert rows then spread over twice the
// workgroups (768 for the 35B-A3B layer, three per CU, where 384 left half the
// CUs with two and half with one). Down: 4 lanes per W_down row (lane c reads
// chunk c of each block), units (expert slot, block) in order, guarded by the
// unit existing.

constexpr int kMoeThreads = 256, kMoeUpDepth = 2;
QMV_HDI constexpr int moe_up_lanes(int t) { return t == 1 ? 32 : 16; }
QMV_HDI constexpr int moe_up_rows(int t) { return (kMoeThreads / 64) * (64 / moe_up_lanes(t)); }
constexpr int kMoeDnRows = 8, kMoeDnGroups = 8, kMoeDnDepth = 6;

struct MoeUpLane {
  int f, c, jb, nsteps, bps;   // bps: blocks per step (lanes per row / 4)
  bool active;
  size_t base;   // the lane's block at step 0 in the chosen expert's gate (or up) matrix
};
QMV_HDI MoeUpLane moe_up_lane(int lanes, int e, int ffn, int hidden, int bx, int tid) {
  MoeUpLane l;
  const int lane = tid & 63, wave = tid >> 6, j = lane & (lanes - 1);
  l.c = j & 3;
  l.jb = j >> 2;
  l.bps = lanes / 4;
  l.f = bx * ((kMoeThreads / 64) * (64 / lanes)) + wave * (64 / lanes) + lane / lanes;
  l.active = l.f < ffn;
  const int nblk = hidden >> 8;
  const size_t row_bytes = (size_t)nblk * kQ4KBytes;
  l.base = (size_t)e * (size_t)ffn * row_bytes + (size_t)(l.active ? l.f : 0) * row_bytes + (size_t)l.jb * kQ4KBytes;
  l.nsteps = (nblk + l.bps - 1) / l.bps;
  return l;
}
QMV_HDI bool moe_up_step_ok(const MoeUpLane &l, int nblk, int s) {
  return l.active && s < l.nsteps && l.bps * s + l.jb < nblk;
}
// Step s's block from the lane's base (an offset or an address); its reads are
// the Q4_K windows of dense_window.
template <class P>
QMV_HDI P moe_up_step_at(P base, int bps, int s) { return base + (size_t)(bps * s) * kQ4KBytes; }

struct MoeDnLane {
  int grp, c, n, my_slots, units;
  size_t row;   // chunk c of block 0 of the lane's W_down row in expert 0
};
QMV_HDI MoeDnLane moe_dn_lane(int hidden, int ffn, int n_slots, int bx, int tid) {
  MoeDnLane l;
  l.grp = tid >> 5;
  l.c = tid & 3;
  l.n = bx * kMoeDnRows + ((tid & 31) >> 2);
  const int nblk = ffn >> 8;
  const size_t row_bytes = (size_t)nblk * kQ4KBytes;
  // rows past the matrix read row 0 (their results are never stored)
  l.row = (size_t)(l.n < hidden ? l.n : 0) * row_bytes + 32 * l.c;
  l.my_slots = n_slots > l.grp ? (n_slots - l.grp + kMoeDnGroups - 1) / kMoeDnGroups : 0;
  l.units = l.my_slots * nblk;
  return l;
}
// Unit (expert e, block lb) from the lane's row (an offset or an address):
// chunk c of the block, whose header sits 32 c bytes before it.
template <class P>
QMV_HDI P moe_dn_unit_at(P row, int e, size_t expert_bytes, int lb) {
  return row + (size_t)e * expert_bytes + (size_t)lb * kQ4KBytes;
}
// A lane's units run expert slot by expert slot, all blocks of one before the
// next: from (slot grp, block 0), each step to the next block, and past the
// last block to block 0 of slot + groups.
QMV_HDI void moe_dn_next(int &slot, int &blk, int nblk, int groups) {
  if (++blk == nblk) {
    blk = 0;
    slot += groups;
  }
}
// Reads relative to the unit address: the header, then the chunk's quants.
QMV_HDI Window moe_dn_window(int c, int i) { return i == 0 ? Window{-32 * c, 16} : Window{16, 32}; }

// ---- routed-expert decode (IQ4_XS experts) -------------------------------------

constexpr int kIq4MoeUpDepth = 2;
// Lanes per gate/up row: 32 for one token (8 rows per 256-thread workgroup),
// 16 for two to four (16 rows), as for the Q4_K experts.
QMV_HDI constexpr int iq4_moe_up_lanes(int t) { return t == 1 ? 32 : 16; }
QMV_HDI constexpr int iq4_moe_up_rows(int t) { return 256 / iq4_moe_up_lanes(t); }
constexpr int kIq4MoeDnRows = 8, kIq4MoeDnLanes = 8, kIq4MoeDnWaves = 4, kIq4MoeDnDepth = 4;

// Gate/up: `lanes` lanes per row, rows past ffn read row 0 of the expert.
QMV_HDI Iq4Lane iq4_moe_up_lane(int lanes, int e, int ffn, int hidden, int bx, int tid) {
  const int f = bx * (256 / lanes) + tid / lanes;
  return iq4_lane(lanes, hidden >> 8, (size_t)e * (size_t)ffn + (size_t)(f < ffn ? f : 0), tid % lanes);
}
// Down: lane (row i, sub-block j) of a wave; unit (slot, block) of W_down.
struct Iq4DnLane {
  int wave, qoff, my_slots, units;
  size_t row;
};
QMV_HDI Iq4DnLane iq4_moe_dn_lane(int hidden, int ffn, int n_slots, int bx, int tid) {
  Iq4DnLane l;
  const int lane = tid & 63;
  l.wave = tid >> 6;
  const int j = lane & (kIq4MoeDnLanes - 1), i_row = lane / kIq4MoeDnLanes;
  const int n = bx * kIq4MoeDnRows + i_row;
  const int nblk = ffn >> 8;
  l.row = (size_t)(n < hidden ? n : 0) * (size_t)nblk * kIQ4XSBytes;
  l.qoff = 8 + 16 * j;
  l.my_slots = n_slots > l.wave ? (n_slots - l.wave + kIq4MoeDnWaves - 1) / kIq4MoeDnWaves : 0;
  l.units = l.my_slots * nblk;
  return l;
}
// Unit (expert e, block lb) from the lane's row (an offset or an address);
// units past the lane's last re-read block 0 of the first slot's expert.
template <class P>
QMV_HDI P iq4_moe_dn_unit_at(P row, int e, size_t expert_bytes, int lb) {
  return row + (size_t)e * expert_bytes + (size_t)lb * kIQ4XSBytes;
}

// ---- prefill GEMM ------------------------------------------------------------------

constexpr int kPrefillBK = 64, kPrefillHalf = 512;

// Tile t of an m_tiles x n_tiles grid as (mt, nt). When the M tiles divide 8,
// tile t goes where block t of a one-tile-per-block launch runs -- workgroups
// are dealt to the 8 XCDs round robin by launch order -- and XCD x works only
// on M tile x % m_tiles, so the X rows of a tile stay in that XCD's L2 for all
// its N tiles; otherwise row-major over N.
QMV_HDI void tile_of(int t, int m_tiles, int n_tiles, int &mt, int &nt) {
  if (8 % m_tiles == 0 && n_tiles % (8 / m_tiles) == 0) {
    const int xcd = t & 7, per = 8 / m_tiles;
    mt = xcd % m_tiles;
    nt = (xcd / m_tiles) + per * (t >> 3);
  } else {
    nt = t % n_tiles;
    mt = t / n_tiles;
  }
}
// Workgroup blk's tile and K steps [s_begin, s_begin + nsteps).
struct PrefillWork {
  int tile, s_begin, nsteps, slot;
};
QMV_HDI PrefillWork prefill_work(int blk, int K, int t_main, int r_tiles, int splits) {
  PrefillWork w{blk, 0, K / kPrefillBK, -1};
  if (blk >= t_main) {
    const int rb = blk - t_main, r = rb % r_tiles, sp = rb / r_tiles, nkb = K >> 8;
    w.tile = t_main + r;
    w.s_begin = 4 * (sp * nkb / splits);
    w.nsteps = 4 * ((sp + 1) * nkb / splits) - w.s_begin;
    w.slot = sp * r_tiles + r;
  }
  return w;
}
// Producer thread pt (0 .. kPrefillHalf - 1) of a tile with first W row n0: block 0 of its
// work's K range in its W row (rows past N read row 0).
QMV_HDI size_t prefill_w_row(int n0, int N, int K, int s_begin, int pt, int threads_per_row) {
  const int nblk = K >> 8, w_row = pt / threads_per_row;
  return (size_t)(n0 + w_row < N ? n0 + w_row : 0) * (size_t)nblk * kQ4KBytes + (size_t)(s_begin >> 2) * kQ4KBytes;
}
// Step s (clamped to the last) of that row: the block offset from the row
// base, then the header and the thread's quant bytes of chunk s % 4.
QMV_HDI int prefill_clamp(int s, int nsteps) { return s < nsteps ? s : nsteps - 1; }
QMV_HDI size_t prefill_w_step(int s) { return (size_t)(s >> 2) * kQ4KBytes; }
QMV_HDI Window prefill_w_window(int s, int pt, int threads_per_row, int i) {
  const int qbytes = 32 / threads_per_row;
  return i == 0 ? Window{0, 16} : Window{16 + 32 * (s & 3) + qbytes * (pt % threads_per_row), qbytes};
}
// X granule (8 bf16) of producer thread pt's i-th load at step s, counted from
// granule s_begin * 8 of row 0: rows past M read row 0.
QMV_HDI uint32_t prefill_x_granule(int pt, int i, int m0, int M, int gpr, int s) {
  const int g = pt + kPrefillHalf * i;
  const int row = m0 + (g >> 3);
  return (uint32_t)(row < M ? row : 0) * (uint32_t)gpr + (uint32_t)(s * 8 + (g & 7));
}

// ---- routed-expert prefill (grouped products) ------------------------------------

constexpr int kGroupTile = 16;

// Tiles of 16 rows per wave, by pair count.
QMV_HDI int group_tiles_per_wave(int P) { return P >= 2048 ? 4 : (P >= 256 ? 2 : 1); }
// The wide (32-pair) gate/up form: waves per workgroup and tiles per wave.
constexpr int kGroupWideWaves = 8, kGroupWideTiles = 1;
// Lane l of wave wv in workgroup bx (waves per workgroup: nwaves): its W row
// for tile tt of expert e (rows of the expert: rows).
QMV_HDI size_t group_row(int e, int rows, int bx, int nwaves, int wv, int tpw, int tt, int l) {
  const int rb = (bx * nwaves + wv) * (tpw * kGroupTile);
  return (size_t)e * (size_t)rows + (size_t)(rb + kGroupTile * tt + (l & 15));
}
// Block b of a row, clamped to the last (the load ahead of the last block
// re-reads it).
QMV_HDI size_t group_block(int b, int nblk) { return (size_t)(b < nblk ? b : nblk - 1) * kQ4KBytes; }
// Reads of lane group kg (l >> 4) from a block: the header, and 8 quant bytes
// of each of the four chunks.
QMV_HDI Window group_window(int kg, int i) { return i == 0 ? Window{0, 16} : Window{16 + 32 * (i - 1) + 8 * kg, 8}; }
constexpr int kGroupWindows = 5;

// ---- Q8_0 GEMV and the dequantization kernels --------------------------------------

// Q8_0 block at byte off (even): read as the dword-aligned window around it.
QMV_HDI Window q80_window(size_t off) {
  const int a = (int)(off & 3);
  return a ? Window{-a, 36} : Window{0, 34};
}

}  // namespace addr
}  // namespace qmv
