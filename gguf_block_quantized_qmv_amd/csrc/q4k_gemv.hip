// Q4_K matrix x bf16 activation rows (decode M=1, speculative verify M=2..4), gfx950.
// The same kernel body, with the block format as a template parameter, serves
// Q5_K (the Q4_K header and nibbles plus a 32-byte plane of fifth bits) and
// Q4_0 (eight 18-byte blocks are 256 weights in 144 bytes, so a group of eight
// is stepped over exactly like a Q4_K super-block; see q40_chunk).
//
// Work mapping. A group of G lanes (16 for rows up to 8192 weights, 32 beyond)
// owns one output row. Lane j of a group reads, at step s, 64-weight chunk
// c = j % 4 of super-block b = (G/4) s + j / 4 of its row: the 16-byte block
// header and the 32 quant bytes of that chunk, as 16-byte loads (the four lanes
// of a block cover its 144 bytes). Rows of 5120 weights are 5 steps of 16 lanes,
// rows of 17408 are 8.5 steps of 32 lanes. The chunk fixes the lane's two
// sub-blocks (2c, 2c+1), so each lane unpacks two scales and two mins per step.
// A workgroup is 256..512 threads (768 for M > 1) of whole rows, sized so that
// every CU gets the same rows when the row count allows it.
//
// Arithmetic per chunk and activation row r:
//   S_lo = sum q_i x_i over the 32 weights of sub-block 2c   (v_dot2 on exact bf16 q)
//   S_hi = the same over sub-block 2c+1
//   acc_r += (d sc_2c) S_lo - (dmin m_2c) X_2c + (d sc_2c+1) S_hi - (dmin m_2c+1) X_2c+1
// where X_j = sum of the 32 activations of sub-block j, precomputed once per
// workgroup. The quants are converted exactly (q is an e4m3 value q*2^-9 scaled
// by 2^9), products of q with bf16 x are exact in fp32, and accumulation is fp32.
//
// LDS holds only the activations: M rows of bf16 in a padded layout of 16-byte
// granules, then the M x K/32 sub-block sums. Each row is reduced inside its
// G-lane group (DPP, then cross-row shuffles for G = 32); nothing crosses waves.
//
// Batch invariance: the instruction sequence applied to activation row r does
// not depend on M or on the workgroup shape (every row runs the same unrolled
// body, explicit fma/dot builtins, no reassociation), so row r is bit-identical
// for M = 1..4.
#include "q4k_common.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

// Block formats of this kernel body.
using addr::kFmtQ4K;
using addr::kFmtQ5K;
using addr::kFmtQ40;


template <int M>
__host__ __device__ constexpr size_t dense_lds_bytes(int k) {
  return layout::q4k_x_lds(M, k);
}

// Activation staging, in two parts so the weight loads can be issued in
// between. Granule g of the M concatenated rows (row r = g / gpr) goes to LDS
// slot r * gpp + padded_granule(g - r * gpr).
template <int M>
__device__ __forceinline__ void store_x_granule(uint4 *xs, const int g, const int gpr, const int gpp, const uint4 v) {
  int r = 0;
#pragma unroll
  for (int q = 1; q < M; ++q) r += g >= q * gpr;
  xs[r * gpp + padded_granule(g - r * gpr)] = v;
}

// Part 1: the first kXHead granules of this thread (g = tid + i * nthreads),
// loaded into registers before any weight load is issued. Vector loads return
// in issue order, so waiting for these never waits for the weights behind them.
template <int kXHead>
__device__ __forceinline__ void load_x_head(const uint4 *__restrict__ xg, const int total, const int nthreads,
                                            uint4 (&v)[kXHead]) {
#pragma unroll
  for (int i = 0; i < kXHead; ++i) {
    const int g = (int)threadIdx.x + i * nthreads;
    v[i] = xg[g < total ? g : 0];  // unconditional, like the weight loads behind it
  }
}

// Part 2: write the head to LDS (no barrier yet).
template <int M, int kXHead>
__device__ __forceinline__ void store_x_head(const uint4 (&v)[kXHead], uint4 *xs, const int gpr, const int gpp,
                                             const int nthreads) {
  const int total = M * gpr;
#pragma unroll
  for (int i = 0; i < kXHead; ++i) {
    const int g = (int)threadIdx.x + i * nthreads;
    if (g < total) store_x_granule<M>(xs, g, gpr, gpp, v[i]);
  }
}

// Part 3: stage the granules beyond the head (rows longer than it covers), BATCH
// per thread per round trip.
template <int M, int kXHead, int BATCH>
__device__ __forceinline__ void stage_x_tail(const uint4 *__restrict__ xg, uint4 *xs, const int gpr, const int gpp,
                                             const int nthreads) {
  const int total = M * gpr;
  for (int base = kXHead * nthreads; base < total; base += nthreads * BATCH) {
    uint4 t[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int g = base + (int)threadIdx.x + i * nthreads;
      t[i] = xg[g < total ? g : 0];
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int g = base + (int)threadIdx.x + i * nthreads;
      if (g < total) store_x_granule<M>(xs, g, gpr, gpp, t[i]);
    }
  }
}

// Part 4: after a barrier, each row's K/32 sub-block sums from LDS, summed in
// index order. Ends with a barrier.
template <int M>
__device__ __forceinline__ void x_sums(const uint4 *xs, float *xsum, const int gpp, const int nsub, const int nthreads) {
  __syncthreads();
  for (int t = threadIdx.x; t < M * nsub; t += nthreads) {
    int r = 0;
#pragma unroll
    for (int q = 1; q < M; ++q) r += t >= q * nsub;
    const int sb = t - r * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 g = xs[r * gpp + padded_granule(4 * sb + q)];
      const uint32_t wv[4] = {g.x, g.y, g.z, g.w};
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

// One 64-weight chunk against M activation rows: xc points at the chunk's first
// granule in row 0 (its 8 granules are xc[0..7]), xsc at its two sub-block sums.
// Quant words 2g, 2g+1 hold weights 8g..8g+7 of both sub-blocks; they are
// converted right before the dot products that use them, so only 8 converted
// pairs are live at a time. Each row keeps four dot2 chains (two per sub-block)
// joined in a fixed order; the chain order does not depend on M.
// Q5_K (Q5 = true): the quants are 5-bit, q = nibble + 16 h with h from the
// high-bit plane (hb0, hb1: its 32 bytes; bit hsh = 2c of byte l belongs to
// weight 64c + l, bit 2c + 1 to weight 64c + 32 + l). q in [0, 31] is not exact
// through the fp8 conversion, so each bf16 quant is built as 128 + q (bits
// 0x43 | q: exact) with one byte permute per pair, and 128 X_j is taken off
// per sub-block: acc += (d sc) (S' - 128 X) - (dmin m) X, S' = sum (128 + q) x.
__device__ __forceinline__ bf16x2 biased_q5_pair_lo(const uint32_t q) {
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, q, 0x04010400u));
}
__device__ __forceinline__ bf16x2 biased_q5_pair_hi(const uint32_t q) {
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, q, 0x04030402u));
}

// Q4_0: the lane's chunk is the pair of 18-byte blocks at byte 36c of a group
// of eight (w0..w3 = w03, w4..w7 = w47, w8). Block A (weights 64c .. 64c + 31,
// sub-block 2c) has d in the low half of w0 and its 16 quant bytes at pair
// bytes 2..17 (realigned by 16 bits); block B (sub-block 2c + 1) has d in the
// high half of w4 and its quant bytes in w5..w8. Byte i of a block holds weight
// i in its low nibble and weight 16 + i in its high nibble; a weight is
// d (q - 8), so per block acc += d S - 8 d X with S = sum q x over the block
// (exact bf16 nibbles, exact products) and X its activation sum.
template <int M>
__device__ __forceinline__ void q40_chunk(float (&acc)[M], const uint4 w03, const uint4 w47, const uint32_t w8,
                                          const uint4 *__restrict__ xc, const int gpp, const float *__restrict__ xsc,
                                          const int nsub) {
  const uint32_t qa[4] = {__builtin_amdgcn_alignbit(w03.y, w03.x, 16), __builtin_amdgcn_alignbit(w03.z, w03.y, 16),
                          __builtin_amdgcn_alignbit(w03.w, w03.z, 16), __builtin_amdgcn_alignbit(w47.x, w03.w, 16)};
  const uint32_t qb[4] = {w47.y, w47.z, w47.w, w8};
  const float da = fp16_bits_to_f32(w03.x & 0xFFFFu), db = fp16_bits_to_f32(w47.x >> 16);
  float sa_lo[M], sa_hi[M], sb_lo[M], sb_hi[M];
#pragma unroll
  for (int r = 0; r < M; ++r) sa_lo[r] = sa_hi[r] = sb_lo[r] = sb_hi[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t la = qa[i] & 0x0F0F0F0Fu, ha = (qa[i] >> 4) & 0x0F0F0F0Fu;
    const uint32_t lb = qb[i] & 0x0F0F0F0Fu, hb = (qb[i] >> 4) & 0x0F0F0F0Fu;
    const bf16x2 la0 = nibbles_to_bf16x2<false>(la), la1 = nibbles_to_bf16x2<true>(la);
    const bf16x2 ha0 = nibbles_to_bf16x2<false>(ha), ha1 = nibbles_to_bf16x2<true>(ha);
    const bf16x2 lb0 = nibbles_to_bf16x2<false>(lb), lb1 = nibbles_to_bf16x2<true>(lb);
    const bf16x2 hb0 = nibbles_to_bf16x2<false>(hb), hb1 = nibbles_to_bf16x2<true>(hb);
#pragma unroll
    for (int r = 0; r < M; ++r) {
      // weights 4i .. 4i + 3 (low nibbles) and 16 + 4i .. 16 + 4i + 3 (high)
      const uint4 xal = xc[r * gpp + (i >> 1)], xah = xc[r * gpp + 2 + (i >> 1)];
      const uint4 xbl = xc[r * gpp + 4 + (i >> 1)], xbh = xc[r * gpp + 6 + (i >> 1)];
      const uint32_t al0 = (i & 1) ? xal.z : xal.x, al1 = (i & 1) ? xal.w : xal.y;
      const uint32_t ah0 = (i & 1) ? xah.z : xah.x, ah1 = (i & 1) ? xah.w : xah.y;
      const uint32_t bl0 = (i & 1) ? xbl.z : xbl.x, bl1 = (i & 1) ? xbl.w : xbl.y;
      const uint32_t bh0 = (i & 1) ? xbh.z : xbh.x, bh1 = (i & 1) ? xbh.w : xbh.y;
      sa_lo[r] = __builtin_amdgcn_fdot2_f32_bf16(la0, __builtin_bit_cast(bf16x2, al0), sa_lo[r], false);
      sa_hi[r] = __builtin_amdgcn_fdot2_f32_bf16(ha0, __builtin_bit_cast(bf16x2, ah0), sa_hi[r], false);
      sb_lo[r] = __builtin_amdgcn_fdot2_f32_bf16(lb0, __builtin_bit_cast(bf16x2, bl0), sb_lo[r], false);
      sb_hi[r] = __builtin_amdgcn_fdot2_f32_bf16(hb0, __builtin_bit_cast(bf16x2, bh0), sb_hi[r], false);
      sa_lo[r] = __builtin_amdgcn_fdot2_f32_bf16(la1, __builtin_bit_cast(bf16x2, al1), sa_lo[r], false);
      sa_hi[r] = __builtin_amdgcn_fdot2_f32_bf16(ha1, __builtin_bit_cast(bf16x2, ah1), sa_hi[r], false);
      sb_lo[r] = __builtin_amdgcn_fdot2_f32_bf16(lb1, __builtin_bit_cast(bf16x2, bl1), sb_lo[r], false);
      sb_hi[r] = __builtin_amdgcn_fdot2_f32_bf16(hb1, __builtin_bit_cast(bf16x2, bh1), sb_hi[r], false);
    }
  }
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float2 xsm = *reinterpret_cast<const float2 *>(xsc + r * nsub);
    acc[r] = __builtin_fmaf(da, sa_lo[r] + sa_hi[r], acc[r]);
    acc[r] = __builtin_fmaf(-8.0f * da, xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(db, sb_lo[r] + sb_hi[r], acc[r]);
    acc[r] = __builtin_fmaf(-8.0f * db, xsm.y, acc[r]);
  }
}

template <int M, int F>
__device__ __forceinline__ void dense_chunk(float (&acc)[M], const uint4 hdr, const uint4 qa, const uint4 qb,
                                            const uint4 hb0, const uint4 hb1, const int hsh, const ScaleSel &sel,
                                            const uint4 *__restrict__ xc, const int gpp,
                                            const float *__restrict__ xsc, const int nsub) {
  if constexpr (F == kFmtQ40) {
    q40_chunk<M>(acc, hdr, qa, qb.x, xc, gpp, xsc, nsub);
    return;
  }
  const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  const uint32_t hw[8] = {hb0.x, hb0.y, hb0.z, hb0.w, hb1.x, hb1.y, hb1.z, hb1.w};
  float s_lo0[M], s_lo1[M], s_hi0[M], s_hi1[M];
#pragma unroll
  for (int r = 0; r < M; ++r) s_lo0[r] = s_lo1[r] = s_hi0[r] = s_hi1[r] = 0.0f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t l0 = qw[2 * g] & 0x0F0F0F0Fu, h0 = (qw[2 * g] >> 4) & 0x0F0F0F0Fu;
    const uint32_t l1 = qw[2 * g + 1] & 0x0F0F0F0Fu, h1 = (qw[2 * g + 1] >> 4) & 0x0F0F0F0Fu;
    bf16x2 lo0, lo1, lo2, lo3, hi0, hi1, hi2, hi3;
    if constexpr (F == kFmtQ5K) {
      // bit 0 of each byte of t: the low-nibble weight's fifth bit; bit 1: the high-nibble weight's
      const uint32_t t0 = hw[2 * g] >> hsh, t1 = hw[2 * g + 1] >> hsh;
      const uint32_t ql0 = l0 | ((t0 << 4) & 0x10101010u), qh0 = h0 | ((t0 << 3) & 0x10101010u);
      const uint32_t ql1 = l1 | ((t1 << 4) & 0x10101010u), qh1 = h1 | ((t1 << 3) & 0x10101010u);
      lo0 = biased_q5_pair_lo(ql0), lo1 = biased_q5_pair_hi(ql0);
      lo2 = biased_q5_pair_lo(ql1), lo3 = biased_q5_pair_hi(ql1);
      hi0 = biased_q5_pair_lo(qh0), hi1 = biased_q5_pair_hi(qh0);
      hi2 = biased_q5_pair_lo(qh1), hi3 = biased_q5_pair_hi(qh1);
    } else {
      lo0 = nibbles_to_bf16x2<false>(l0), lo1 = nibbles_to_bf16x2<true>(l0);
      lo2 = nibbles_to_bf16x2<false>(l1), lo3 = nibbles_to_bf16x2<true>(l1);
      hi0 = nibbles_to_bf16x2<false>(h0), hi1 = nibbles_to_bf16x2<true>(h0);
      hi2 = nibbles_to_bf16x2<false>(h1), hi3 = nibbles_to_bf16x2<true>(h1);
    }
#pragma unroll
    for (int r = 0; r < M; ++r) {
      const uint4 v = xc[r * gpp + g];
      const uint4 u = xc[r * gpp + 4 + g];
      s_lo0[r] = __builtin_amdgcn_fdot2_f32_bf16(lo0, __builtin_bit_cast(bf16x2, v.x), s_lo0[r], false);
      s_hi0[r] = __builtin_amdgcn_fdot2_f32_bf16(hi0, __builtin_bit_cast(bf16x2, u.x), s_hi0[r], false);
      s_lo1[r] = __builtin_amdgcn_fdot2_f32_bf16(lo1, __builtin_bit_cast(bf16x2, v.y), s_lo1[r], false);
      s_hi1[r] = __builtin_amdgcn_fdot2_f32_bf16(hi1, __builtin_bit_cast(bf16x2, u.y), s_hi1[r], false);
      s_lo0[r] = __builtin_amdgcn_fdot2_f32_bf16(lo2, __builtin_bit_cast(bf16x2, v.z), s_lo0[r], false);
      s_hi0[r] = __builtin_amdgcn_fdot2_f32_bf16(hi2, __builtin_bit_cast(bf16x2, u.z), s_hi0[r], false);
      s_lo1[r] = __builtin_amdgcn_fdot2_f32_bf16(lo3, __builtin_bit_cast(bf16x2, v.w), s_lo1[r], false);
      s_hi1[r] = __builtin_amdgcn_fdot2_f32_bf16(hi3, __builtin_bit_cast(bf16x2, u.w), s_hi1[r], false);
    }
  }
  const ChunkScales cs = chunk_scales(hdr, sel);
#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float s_lo = s_lo0[r] + s_lo1[r], s_hi = s_hi0[r] + s_hi1[r];
    const float2 xsm = *reinterpret_cast<const float2 *>(xsc + r * nsub);
    acc[r] = __builtin_fmaf(cs.a0, s_lo, acc[r]);
    if constexpr (F == kFmtQ5K) acc[r] = __builtin_fmaf(-cs.a0, 128.0f * xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi, acc[r]);
    if constexpr (F == kFmtQ5K) acc[r] = __builtin_fmaf(-cs.a1, 128.0f * xsm.y, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, xsm.y, acc[r]);
  }
}

// The 16-byte weight loads of one step for the lane holding chunk c of the
// block at bp: the block header (for Q5_K with the 32 bytes of the high-bit
// plane that every chunk's lane reads; for Q4_0 the chunk's pair of 18-byte
// blocks, read as nine dwords) and the chunk's 32 quant bytes -- the windows
// addr::dense_window describes (checked below). The offsets are written out
// here: the same offsets formed through the window function cost registers.
template <int F>
constexpr int kQuantBase = F == kFmtQ5K ? 48 : 16;

template <int F>
__device__ __forceinline__ void load_step(const uint8_t *__restrict__ bp, const int c, uint4 &hdr, uint4 &qa,
                                          uint4 &qb, uint4 &hb0, uint4 &hb1) {
  if constexpr (F == kFmtQ40) {
    // the pair of 18-byte blocks at byte 36c: 4-byte aligned, read as dwords
    const uint32_t *p = reinterpret_cast<const uint32_t *>(bp + 36 * c);
    hdr = make_uint4(p[0], p[1], p[2], p[3]);
    qa = make_uint4(p[4], p[5], p[6], p[7]);
    qb = make_uint4(p[8], 0u, 0u, 0u);
    return;
  }
  hdr = *reinterpret_cast<const uint4 *>(bp);
  if constexpr (F == kFmtQ5K) {
    hb0 = *reinterpret_cast<const uint4 *>(bp + 16);
    hb1 = *reinterpret_cast<const uint4 *>(bp + 32);
  }
  qa = *reinterpret_cast<const uint4 *>(bp + kQuantBase<F> + 32 * c);
  qb = *reinterpret_cast<const uint4 *>(bp + kQuantBase<F> + 32 * c + 16);
}

constexpr bool load_step_reads_the_windows() {
  for (int c = 0; c < 4; ++c) {
    const addr::Window q4h = addr::dense_window(kFmtQ4K, c, 0), q4q = addr::dense_window(kFmtQ4K, c, 1);
    const addr::Window q5h = addr::dense_window(kFmtQ5K, c, 0), q5q = addr::dense_window(kFmtQ5K, c, 1);
    const addr::Window q0 = addr::dense_window(kFmtQ40, c, 0), q0q = addr::dense_window(kFmtQ40, c, 1);
    if (q4h.off != 0 || q4h.len != 16 || q4q.off != kQuantBase<kFmtQ4K> + 32 * c || q4q.len != 32) return false;
    if (q5h.off != 0 || q5h.len != 48 || q5q.off != kQuantBase<kFmtQ5K> + 32 * c || q5q.len != 32) return false;
    if (q0.off != 36 * c || q0.len != 36 || q0q.len != 0) return false;
  }
  return true;
}
static_assert(load_step_reads_the_windows(), "load_step reads exactly the windows of addr::dense_window");

// Block address of step t for this lane (addr::dense_step_ok and
// addr::dense_step_offset), or the fallback block wfb when the step has no
// block of its own.
template <bool FULL, int NS, int kBlocksPerStep, int F>
__device__ __forceinline__ const uint8_t *step_ptr(const uint8_t *wfb, const uint8_t *wl, const bool active, const int t,
                                                   const int nsteps, const int jb, const int nblk,
                                                   const bool last_ok) {
  const bool ok = addr::dense_step_ok(active, last_ok, nsteps, jb, NS, FULL, 4 * kBlocksPerStep, nblk, t);
  return ok ? wl + addr::dense_step_offset(4 * kBlocksPerStep, F, t) : wfb;
}

// G lanes own one output row (G = 16 or 32): a step covers G/4 super-blocks of
// the row, lane j holding chunk j % 4 of block j / 4. A wave owns 64/G rows.
//
// Prologue order: the first kXHead activation granules per thread are
// requested, then the first D steps of weights; the activations are written to
// LDS (and the sub-block sums formed) as soon as they arrive, while the weights
// are still in flight. Afterwards a ring of D steps stays in flight.
//
// Every weight load is issued unconditionally -- a step past the row, blocks
// past a partial last step and rows past the matrix read the last block of the
// lane's row (or of the matrix) instead and are never used -- so the number of
// loads in flight is known at every point and each step waits only for its own
// ring slot.
//
// NS > 0: the row is exactly NS steps (the last one possibly partial) and the
// step loop is unrolled, which keeps the ring in fixed registers and every wait
// exact. NS == 0: rows of any length, runtime step loop (FULL: a whole number of
// steps, so no lane needs a block-range test).
//
// kXHead: activation granules per thread loaded ahead of the weights -- enough
// for the rows the launcher sends to each G (K <= 8192 with G = 16, K <= 18432
// otherwise) at M = 1, capped at 9 so the head never sets the register peak.
// Workgroups have kMinThreads..kMaxThreads threads (addr::balanced_rows).
// Ring depths (addr::dense_depth): at M = 1 a 5-step row of 16 lanes (K = 5120)
// keeps every load in flight from the start and the 9-step rows of 32 lanes are
// fastest with 2; Q5_K at M = 2..4 (more registers per step) takes 4 for both.
constexpr int kMinThreads = addr::kDenseMinThreads;
constexpr int kMaxThreads = addr::dense_max_threads(1);       // M = 1
constexpr int kMaxThreadsRows = addr::dense_max_threads(2);   // M = 2..4: register use allows 3 waves per SIMD

template <int M, int G>
constexpr int x_head() { return (G == 16 ? 4 * M : 9 * M) < 9 ? (G == 16 ? 4 * M : 9 * M) : 9; }

// PAIR: w and w1 are two matrices of n rows on the same activations, the grid
// covers 2n rows (addr::pair_row), and matrix 1's rows go to y1; each row runs
// exactly the instruction sequence of the one-matrix launch.
template <int M, int G, int D, bool FULL, int NS, int F, bool PAIR = false>
__device__ __forceinline__ void gemv_body(const uint8_t *__restrict__ w, const uint16_t *__restrict__ x,
                                          float *__restrict__ y, const int n, const int k,
                                          const uint8_t *__restrict__ w1 = nullptr, float *__restrict__ y1 = nullptr) {
  constexpr int kBlocksPerStep = G / 4;
  constexpr int kStepGranules = (G / 2) * 17;   // padded LDS granules per step
  extern __shared__ uint4 lds[];
  const int nblk = k >> 8;
  const int gpr = k >> 3;
  const int gpp = (int)padded_row_granules(k);
  const int nsub = k >> 5;
  uint4 *xs = lds;
  float *xsum = reinterpret_cast<float *>(lds + (size_t)M * gpp);

  const int lane = threadIdx.x & 63;
  const int j = lane & (G - 1);
  // blockDim.x = (rows per workgroup) * G; the last wave may be partial
  const int nthreads = (int)blockDim.x;
  int row = addr::lane_row(blockIdx.x, threadIdx.x, nthreads, G);
  if constexpr (PAIR) {
    const addr::PairRow pr = addr::pair_row(row, n);
    row = pr.row;
    if (pr.half) w = w1, y = y1;
  }
  // loads with no block of their own (past the row, past the matrix, past a
  // partial last step) read the last block of the lane's row (of the last row
  // when the row is past the matrix), which the same or a recent load also reads
  const addr::DenseLane ln = addr::dense_lane(G, NS, F, n, nblk, row, j);
  const int c = ln.c, jb = ln.jb;
  const bool active = ln.active, last_ok = ln.last_ok;
  const int nsteps = ln.nsteps;
  const uint8_t *wl = w + ln.row_base + ln.blk_off, *wfb = w + ln.fb;

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  constexpr int kXHead = x_head<M, G>();
  uint4 xv[kXHead];
  load_x_head<kXHead>(xg, M * gpr, nthreads, xv);
  uint4 hdr[D], qa[D], qb[D], hb0[D], hb1[D];
  if constexpr (M == 1) {
    // One step of weights goes out behind the activation head; the rest of the
    // ring only after the head has arrived and is in LDS. Requests queue in the
    // memory system in issue order, so every weight request issued before a
    // wave's activations are back delays them (and with them its first step).
    load_step<F>(step_ptr<FULL, NS, kBlocksPerStep, F>(wfb, wl, active, 0, nsteps, jb, nblk, last_ok), c, hdr[0], qa[0], qb[0],
                  hb0[0], hb1[0]);
    store_x_head<M, kXHead>(xv, xs, gpr, gpp, nthreads);
#pragma unroll
    for (int u = 1; u < D; ++u)
      load_step<F>(step_ptr<FULL, NS, kBlocksPerStep, F>(wfb, wl, active, u, nsteps, jb, nblk, last_ok), c, hdr[u], qa[u], qb[u],
                    hb0[u], hb1[u]);
    // rows up to NS steps are covered by the head when this holds, and the
    // loop that stages the rest is compiled out
    if constexpr (NS == 0 || NS * G * 8 > kXHead * kMinThreads) stage_x_tail<M, kXHead, 2>(xg, xs, gpr, gpp, nthreads);
  } else {
    // Several rows fill most of the LDS and allow few workgroups per CU: all the
    // activations are staged (eight granules per thread per round trip) before
    // the first weight request, so no staging load waits behind the weights.
    store_x_head<M, kXHead>(xv, xs, gpr, gpp, nthreads);
    stage_x_tail<M, kXHead, 8>(xg, xs, gpr, gpp, nthreads);
#pragma unroll
    for (int u = 0; u < D; ++u)
      load_step<F>(step_ptr<FULL, NS, kBlocksPerStep, F>(wfb, wl, active, u, nsteps, jb, nblk, last_ok), c, hdr[u], qa[u], qb[u],
                    hb0[u], hb1[u]);
  }
  x_sums<M>(xs, xsum, gpp, nsub, nthreads);
  if (!active) return;

  const ScaleSel sel = scale_selectors(c);
  const uint4 *xb = xs + (j >> 1) * 17 + (j & 1) * 8;
  const float *sb = xsum + 2 * j;
  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;

  if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      constexpr int kD = D;
      const int u = s % kD;
      if (s < NS - 1 || last_ok)
        dense_chunk<M, F>(acc, hdr[u], qa[u], qb[u], hb0[u], hb1[u], 2 * c, sel, xb + s * kStepGranules, gpp,
                           sb + s * 2 * G, nsub);
      if (s + D < NS)
        load_step<F>(step_ptr<FULL, NS, kBlocksPerStep, F>(wfb, wl, active, s + D, nsteps, jb, nblk, last_ok), c, hdr[u], qa[u],
                      qb[u], hb0[u], hb1[u]);
    }
  } else {
    for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        const int s = s0 + u;
        if (s < nsteps && (FULL || s * kBlocksPerStep + jb < nblk))
          dense_chunk<M, F>(acc, hdr[u], qa[u], qb[u], hb0[u], hb1[u], 2 * c, sel, xb + s * kStepGranules, gpp,
                             sb + s * 2 * G, nsub);
        load_step<F>(step_ptr<FULL, NS, kBlocksPerStep, F>(wfb, wl, active, s + D, nsteps, jb, nblk, last_ok), c, hdr[u], qa[u],
                      qb[u], hb0[u], hb1[u]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float v = group_sum<G>(acc[r]);
    if (j == r) y[(size_t)r * n + row] = v;
  }
}

template <int M, int G, int D, bool FULL, int NS>
__global__ __launch_bounds__(M == 1 ? kMaxThreads : kMaxThreadsRows) void q4k_gemv_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  gemv_body<M, G, D, FULL, NS, kFmtQ4K>(w, x, y, n, k);
}

template <int M, int G, int D, bool FULL, int NS>
__global__ __launch_bounds__(M == 1 ? kMaxThreads : kMaxThreadsRows) void q4k_gemv_pair_kernel(
    const uint8_t *__restrict__ w0, const uint8_t *__restrict__ w1, const uint16_t *__restrict__ x,
    float *__restrict__ y0, float *__restrict__ y1, const int n, const int k) {
  gemv_body<M, G, D, FULL, NS, kFmtQ4K, true>(w0, x, y0, n, k, w1, y1);
}

template <int M, int G, int D, bool FULL, int NS>
__global__ __launch_bounds__(M == 1 ? kMaxThreads : kMaxThreadsRows) void q40_gemv_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  gemv_body<M, G, D, FULL, NS, kFmtQ40>(w, x, y, n, k);
}

template <int M, int G, int D, bool FULL, int NS>
__global__ __launch_bounds__(M == 1 ? kMaxThreads : kMaxThreadsRows) void q5k_gemv_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  gemv_body<M, G, D, FULL, NS, kFmtQ5K>(w, x, y, n, k);
}

// The plan (lanes per row, steps, ring depth, rows per workgroup, grid) is
// addr::dense_gemv_plan; rows per workgroup balance the rows over the 256 CUs
// (10 rows of 32 lanes for N = 5120 at M = 1, 20 rows at M = 2..4 where the
// activations fill the LDS). Each instantiation below is the one the plan
// names: G and NS by the switch, D = addr::dense_depth(F, M, G).
template <int M, int G, bool FULL, int NS, int F, bool PAIR = false>
int launch_cfg(const addr::GemvPlan &p, const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream,
               const void *w1 = nullptr, float *y1 = nullptr) {
  constexpr int D = addr::dense_depth(F, M, G);
  const size_t lds = dense_lds_bytes<M>(k);
  if constexpr (PAIR) {
    static_assert(F == kFmtQ4K, "the pair form is built for Q4_K");
    static LdsGrant granted_pair;
    if (allow_dynamic_lds(reinterpret_cast<const void *>(&q4k_gemv_pair_kernel<M, G, D, FULL, NS>), lds, granted_pair,
                          "q4k_gemv_pair_kernel"))
      return QMV_ERR_HIP;
    return launch_kernel("q4k_gemv_pair_kernel", q4k_gemv_pair_kernel<M, G, D, FULL, NS>, dim3(p.grid),
                         dim3(p.rows * G), lds, stream, w, w1, x, y, y1, n, k);
  }
  // only the launched format's kernel is instantiated
  void (*fn)(const uint8_t *, const uint16_t *, float *, int, int);
  const char *name;
  if constexpr (F == kFmtQ5K) fn = q5k_gemv_kernel<M, G, D, FULL, NS>, name = "q5k_gemv_kernel";
  else if constexpr (F == kFmtQ40) fn = q40_gemv_kernel<M, G, D, FULL, NS>, name = "q40_gemv_kernel";
  else fn = q4k_gemv_kernel<M, G, D, FULL, NS>, name = "q4k_gemv_kernel";
  static LdsGrant granted;
  if (allow_dynamic_lds(reinterpret_cast<const void *>(fn), lds, granted, name)) return QMV_ERR_HIP;
  return launch_kernel(name, fn, dim3(p.grid), dim3(p.rows * G), lds, stream, w, x, y, n, k);
}

// PAIR: w1 and y1 are the second matrix and its output; the plan covers 2n
// rows (the same G, NS and D as one matrix: they depend on k and M only).
template <int M, int F, bool PAIR = false>
int launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream, const void *w1 = nullptr,
             float *y1 = nullptr) {
  const addr::GemvPlan p = addr::dense_gemv_plan(F, M, PAIR ? 2 * n : n, k);
  if (p.G == 16) {
    switch (p.ns) {
      case 1: return launch_cfg<M, 16, false, 1, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 2: return launch_cfg<M, 16, false, 2, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 3: return launch_cfg<M, 16, false, 3, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 4: return launch_cfg<M, 16, false, 4, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 5: return launch_cfg<M, 16, false, 5, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 6: return launch_cfg<M, 16, false, 6, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      case 7: return launch_cfg<M, 16, false, 7, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
      default: return launch_cfg<M, 16, false, 8, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    }
  }
  switch (p.ns) {
    case 5: return launch_cfg<M, 32, false, 5, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    case 6: return launch_cfg<M, 32, false, 6, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    case 7: return launch_cfg<M, 32, false, 7, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    case 8: return launch_cfg<M, 32, false, 8, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    case 9: return launch_cfg<M, 32, false, 9, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
    default:
      return p.full ? launch_cfg<M, 32, true, 0, F, PAIR>(p, w, x, y, n, k, stream, w1, y1)
                    : launch_cfg<M, 32, false, 0, F, PAIR>(p, w, x, y, n, k, stream, w1, y1);
  }
}

}  // namespace

int launch_q4_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1, kFmtQ4K>(w, x, y, n, k, s);
    case 2: return launch_m<2, kFmtQ4K>(w, x, y, n, k, s);
    case 3: return launch_m<3, kFmtQ4K>(w, x, y, n, k, s);
    case 4: return launch_m<4, kFmtQ4K>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_q4_k_gemv_pair(const void *w0, const void *w1, const uint16_t *x, float *y0, float *y1, int m, int n, int k,
                          void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1, kFmtQ4K, true>(w0, x, y0, n, k, s, w1, y1);
    case 2: return launch_m<2, kFmtQ4K, true>(w0, x, y0, n, k, s, w1, y1);
    case 3: return launch_m<3, kFmtQ4K, true>(w0, x, y0, n, k, s, w1, y1);
    case 4: return launch_m<4, kFmtQ4K, true>(w0, x, y0, n, k, s, w1, y1);
    default: return QMV_ERR_RANGE;
  }
}

int launch_q5_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1, kFmtQ5K>(w, x, y, n, k, s);
    case 2: return launch_m<2, kFmtQ5K>(w, x, y, n, k, s);
    case 3: return launch_m<3, kFmtQ5K>(w, x, y, n, k, s);
    case 4: return launch_m<4, kFmtQ5K>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_q4_0_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1, kFmtQ40>(w, x, y, n, k, s);
    case 2: return launch_m<2, kFmtQ40>(w, x, y, n, k, s);
    case 3: return launch_m<3, kFmtQ40>(w, x, y, n, k, s);
    case 4: return launch_m<4, kFmtQ40>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

}  // namespace qmv
