// Routed-expert MoE feed-forward on Q4_K experts, gfx950.
//
// The workload is the memra README speed table's 35B-A3B MoE decode (hidden
// 2048, 128 experts, top-8) and the memra-bench card's K=2 drafts on it: per
// token, the top-k router logits pick experts, their softmax (restricted to
// the chosen k) weights the experts' silu-gated FFN outputs.
//
// Two launches on the caller's stream, no host round trip:
//
//  1. moe_gate_up_kernel, grid (F/16 row tiles) x (max distinct experts).
//     The activations of all T tokens and the router logits are requested at
//     once; the workgroup then routes every token in one pass (each expert
//     ranked by counting the token's larger composite keys -- logit, then the
//     lower id -- the K of rank below K chosen in rank order), and every wave
//     sorts the (expert, token) pairs in registers (rank by comparison,
//     forward lane permute), forms their weights (the softmax over each
//     token's chosen logits) and finds its workgroup's distinct expert, the
//     s-th smallest, and the tokens that chose it. Workgroup (0, 0)
//     writes the routing outputs and the tables launch 2 reads. The expert's
//     gate and up rows are requested as soon as the expert is known; the
//     activation sub-block sums are formed in LDS while they arrive. Each
//     16-row tile stores h = silu(W_gate x) * (W_up x) in fp32 per pair.
//  2. moe_down_kernel, grid H/8 row tiles. Four lanes own one W_down row and
//     the workgroup's eight groups of 32 lanes share its 8 rows, group g taking
//     the distinct experts g, g + 8, ...; every pair's h is staged in LDS
//     together with the routing tables, then the first (expert, block) weight
//     loads go out and the h sub-block sums are formed while they arrive. Each
//     (pair, row) result z lands in LDS, and y_t = sum over token t's experts,
//     in routing rank order (largest logit first), of weight * z, accumulated
//     with fma from zero.
//
// Each selected expert's weights are read once per call. A token's result is
// bit-identical whatever other tokens share the call: the arithmetic applied
// to one (expert, token) pair does not depend on which lanes or waves run it,
// and a token's experts are combined in its own rank order.
#include <limits.h>

#include "moe_routing.h"
#include "q4k_common.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

using namespace moe;

constexpr int kWaves = 4;
constexpr int kThreads = addr::kMoeThreads;
// gate/up: 16 lanes per W row, 4 rows per wave, 16 rows per workgroup
constexpr int kUpDepth = addr::kMoeUpDepth;  // steps of gate + up loads in flight
// down: 4 lanes per W row; a workgroup owns 8 rows, and its 8 lane groups of
// 32 lanes (8 rows x 4 chunks) split the distinct experts
constexpr int kDnRows = addr::kMoeDnRows;
constexpr int kDnGroups = addr::kMoeDnGroups;
constexpr int kDnDepth = addr::kMoeDnDepth;  // (expert, block) units of loads in flight per lane
static_assert(kThreads == kRouteThreads, "the gate/up workgroup routes with every thread");
static_assert(kThreads == 64 * kWaves && kDnGroups == kThreads / (4 * kDnRows), "the shapes the addressing assumes");

// The gate (or up) loads of one step at bp: the block header and chunk c's 32
// quant bytes (the Q4_K windows of addr::dense_window).
__device__ __forceinline__ void load_up_step(const uint8_t *__restrict__ bp, const int c, uint4 &h, uint4 &a,
                                             uint4 &b) {
  const addr::Window wh = addr::dense_window(addr::kFmtQ4K, c, 0), wq = addr::dense_window(addr::kFmtQ4K, c, 1);
  h = *reinterpret_cast<const uint4 *>(bp + wh.off);
  a = *reinterpret_cast<const uint4 *>(bp + wq.off);
  b = *reinterpret_cast<const uint4 *>(bp + wq.off + 16);
}

// The W_down loads of one unit at bp (the block's first byte plus 32 c): the
// header and chunk c's 32 quant bytes (addr::moe_dn_window).
__device__ __forceinline__ void load_dn_unit(const uint8_t *__restrict__ bp, const int c, uint4 &h, uint4 &a,
                                             uint4 &b) {
  const addr::Window wh = addr::moe_dn_window(c, 0), wq = addr::moe_dn_window(c, 1);
  h = *reinterpret_cast<const uint4 *>(bp + wh.off);
  a = *reinterpret_cast<const uint4 *>(bp + wq.off);
  b = *reinterpret_cast<const uint4 *>(bp + wq.off + 16);
}

typedef float floatx2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Launch 1: gate and up projections, silu gating
// ---------------------------------------------------------------------------

// One 64-weight chunk of a W row against the bf16 activations of `m_act`
// tokens: token r's chunk granules at xc + xoff[r] (8 contiguous granules of
// the padded layout), its two sub-block sums at xsc + soff[r].
template <int T>
__device__ __forceinline__ void chunk_bf16(float (&acc)[T], const int m_act, const uint4 hdr, const uint4 qa,
                                           const uint4 qb, const ScaleSel &sel, const uint4 *__restrict__ xc,
                                           const int (&xoff)[T], const float *__restrict__ xsc, const int (&soff)[T]) {
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
  for (int r = 0; r < T; ++r) {
    if (r >= m_act) break;
    const uint4 *xr = xc + xoff[r];
    float s_lo = 0.0f, s_hi = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 v = xr[g];
      const uint4 u = xr[4 + g];
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 0], __builtin_bit_cast(bf16x2, v.x), s_lo, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 0], __builtin_bit_cast(bf16x2, u.x), s_hi, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 1], __builtin_bit_cast(bf16x2, v.y), s_lo, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 1], __builtin_bit_cast(bf16x2, u.y), s_hi, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 2], __builtin_bit_cast(bf16x2, v.z), s_lo, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 2], __builtin_bit_cast(bf16x2, u.z), s_hi, false);
      s_lo = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 3], __builtin_bit_cast(bf16x2, v.w), s_lo, false);
      s_hi = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 3], __builtin_bit_cast(bf16x2, u.w), s_hi, false);
    }
    const float2 xsm = *reinterpret_cast<const float2 *>(xsc + soff[r]);
    acc[r] = __builtin_fmaf(cs.a0, s_lo, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, xsm.y, acc[r]);
  }
}

constexpr int kStageBatch = 4;  // activation granules per thread per batch

template <int T>
__device__ __forceinline__ void load_x_batch(const uint4 *__restrict__ xg, const int base, const int total,
                                             uint4 (&v)[kStageBatch]) {
#pragma unroll
  for (int i = 0; i < kStageBatch; ++i) {
    const int g = base + (int)threadIdx.x + i * kThreads;
    v[i] = xg[g < total ? g : 0];
  }
}

// Lanes past the end hold granule 0 (their load was clamped) and store it to
// granule 0's slot again: no store is guarded, so the compiler cannot sink a
// load into a store's branch, where each load would wait before the next.
template <int T>
__device__ __forceinline__ void store_x_batch(uint4 *xs, const int base, const int total, const int gpr,
                                              const int gpp, const uint4 (&v)[kStageBatch]) {
#pragma unroll
  for (int i = 0; i < kStageBatch; ++i) {
    const int g0 = base + (int)threadIdx.x + i * kThreads;
    const int g = g0 < total ? g0 : 0;
    int r = 0;
#pragma unroll
    for (int q = 1; q < T; ++q) r += g >= q * gpr;
    xs[r * gpp + padded_granule(g - r * gpr)] = v[i];
  }
}

// Workgroup (tile, slot) of launch 1: rows R tile .. R tile + R - 1 of the
// slot-th distinct expert's W_gate and W_up, L lanes per row (addr::moe_up_rows,
// addr::moe_up_lanes: 8 rows of 32 lanes for one token, 16 rows of 16 lanes for
// more). Returns with every thread of the workgroup past its last barrier
// (threads without a row return early).
//
// Both lane widths give every row the same bits, so a token's result does not
// depend on how many tokens share the call: a lane's blocks are summed in two
// chains, blocks b with b / 4 even and with b / 4 odd (for 32 lanes the two
// chains sit in lanes j and j ^ 16, for 16 lanes in one lane's alternate
// steps), the two chains are added, then summed over the 16 lanes of the
// row's (block mod 4, chunk) positions in one fixed DPP tree.
template <int T>
__device__ __forceinline__ void gate_up_body(const uint8_t *__restrict__ w_gate, const uint8_t *__restrict__ w_up,
                                             const float *__restrict__ logits, const uint16_t *__restrict__ x,
                                             int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
                                             int32_t *__restrict__ pairs_out, uint8_t *__restrict__ ws,
                                             const int hidden, const int ffn, const int E, const int K,
                                             const int tile, const int slot, RouteLds &rl, uint4 *lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gpr = hidden >> 3, nsub = hidden >> 5;
  const int gpp = (int)padded_row_granules(hidden);
  uint4 *xs = lds;
  float *xsum = reinterpret_cast<float *>(lds + (size_t)T * gpp);
  uint32_t *kr = reinterpret_cast<uint32_t *>(xsum + (size_t)T * nsub);   // routing rows

  // every token's activations and the router logits are requested together
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const int total = T * gpr;
  uint4 v[kStageBatch];
  load_x_batch<T>(xg, 0, total, v);
  const WgLogits<T> lg = load_logits_wg<T>(logits, E);
  store_x_batch<T>(xs, 0, total, gpr, gpp, v);
  store_keys<T>(lg, E, kr, rl);
  for (int base = kStageBatch * kThreads; base < total; base += kStageBatch * kThreads) {
    uint4 vb[kStageBatch];
    load_x_batch<T>(xg, base, total, vb);
    store_x_batch<T>(xs, base, total, gpr, gpp, vb);
  }
  __syncthreads();
  route_wave<T>(kr, E, K, rl);
  __syncthreads();

  const int P = T * K;
  const PairRank pr = pair_ranks<T>(rl, P);
  const Slot<T> sl = my_slot<T>(pr, slot, P);
  if (sl.p0 < 0) return;  // fewer distinct experts than the grid allows for (uniform over the workgroup)

  constexpr int kUpLanes = addr::moe_up_lanes(T), kBps = kUpLanes / 4;
  const int j = lane & (kUpLanes - 1);
  const addr::MoeUpLane ln = addr::moe_up_lane(kUpLanes, sl.e, ffn, hidden, tile, threadIdx.x);
  const int c = ln.c, jb = ln.jb, f = ln.f;
  const bool active = ln.active;
  const int nblk = hidden >> 8;
  const uint8_t *gl = w_gate + ln.base;
  const uint8_t *ul = w_up + ln.base;
  const int nsteps = ln.nsteps;

  uint4 gh[kUpDepth], ga[kUpDepth], gb[kUpDepth], uh[kUpDepth], ua[kUpDepth], ub[kUpDepth];
#pragma unroll
  for (int u = 0; u < kUpDepth; ++u) {
    if (addr::moe_up_step_ok(ln, nblk, u)) {
      load_up_step(addr::moe_up_step_at(gl, kBps, u), c, gh[u], ga[u], gb[u]);
      load_up_step(addr::moe_up_step_at(ul, kBps, u), c, uh[u], ua[u], ub[u]);
    }
  }
  // the weights (softmax) and the routing outputs, off the path to the loads
  // above: the last wave of workgroup (0, 0), whose waves all hold the expert
  // of slot 0
  if (tile == 0 && slot == 0 && wave == kWaves - 1)
    write_routing(with_weights(sorted_pairs(pr, P), rl, P, K), P, topk_ids, topk_w, pairs_out,
                  reinterpret_cast<Table *>(ws));

  // sub-block sums of every staged token (index order) while the weights arrive
  for (int t = threadIdx.x; t < T * nsub; t += kThreads) {
    int r = 0;
#pragma unroll
    for (int q = 1; q < T; ++q) r += t >= q * nsub;
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
  if (!active) return;

  const ScaleSel sel = scale_selectors(c);
  int xoff[T], soff[T];
#pragma unroll
  for (int r = 0; r < T; ++r) {
    xoff[r] = sl.tok[r] * gpp;
    soff[r] = sl.tok[r] * nsub;
  }
  // chunk 4 kBps s + j of the row sits at padded granule 34 kBps s + (j >> 1) * 17 + (j & 1) * 8
  const uint4 *xb = xs + (j >> 1) * 17 + (j & 1) * 8;
  const float *sb = xsum + 2 * j;
  // chain 0: blocks b with b / 4 even; chain 1: b / 4 odd (16 lanes: odd steps)
  float acc_g[2][T], acc_u[2][T];
#pragma unroll
  for (int r = 0; r < T; ++r) acc_g[0][r] = acc_u[0][r] = acc_g[1][r] = acc_u[1][r] = 0.0f;

  static_assert(kUpDepth == 2, "16 lanes: step parity is the ring slot");
  for (int s0 = 0; s0 < nsteps; s0 += kUpDepth) {
#pragma unroll
    for (int u = 0; u < kUpDepth; ++u) {
      const int s = s0 + u;
      constexpr int kOdd = kBps == 4 ? 1 : 0;   // chain of the ring slot u = 1
      if (s < nsteps && kBps * s + jb < nblk) {
        chunk_bf16<T>(acc_g[u * kOdd], sl.ntok, gh[u], ga[u], gb[u], sel, xb + s * 34 * kBps, xoff,
                      sb + 8 * kBps * s, soff);
        chunk_bf16<T>(acc_u[u * kOdd], sl.ntok, uh[u], ua[u], ub[u], sel, xb + s * 34 * kBps, xoff,
                      sb + 8 * kBps * s, soff);
      }
      const int sn = s + kUpDepth;
      if (addr::moe_up_step_ok(ln, nblk, sn)) {   // active holds for every lane that gets here
        load_up_step(addr::moe_up_step_at(gl, kBps, sn), c, gh[u], ga[u], gb[u]);
        load_up_step(addr::moe_up_step_at(ul, kBps, sn), c, uh[u], ua[u], ub[u]);
      }
    }
  }

  float *h = reinterpret_cast<float *>(ws + kTableBytes);
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if (r >= sl.ntok) break;
    float vg, vu;
    if constexpr (kUpLanes == 32) {   // lane j ^ 16 holds the other chain
      vg = acc_g[0][r] + __shfl_xor(acc_g[0][r], 16);
      vu = acc_u[0][r] + __shfl_xor(acc_u[0][r], 16);
    } else {
      vg = acc_g[0][r] + acc_g[1][r];
      vu = acc_u[0][r] + acc_u[1][r];
    }
    const float g = row16_sum(vg);
    const float u = row16_sum(vu);
    if (j == r) h[(size_t)(sl.p0 + r) * ffn + f] = g / (1.0f + expf(-g)) * u;
  }
}

template <int T>
__global__ __launch_bounds__(kThreads) void moe_gate_up_kernel(
    const uint8_t *__restrict__ w_gate, const uint8_t *__restrict__ w_up, const float *__restrict__ logits,
    const uint16_t *__restrict__ x, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ pairs_out, uint8_t *__restrict__ ws, const int hidden, const int ffn, const int E,
    const int K) {
  __shared__ __align__(16) RouteLds rl;
  extern __shared__ uint4 lds[];
  gate_up_body<T>(w_gate, w_up, logits, x, topk_ids, topk_w, pairs_out, ws, hidden, ffn, E, K, (int)blockIdx.x,
                  (int)blockIdx.y, rl, lds);
}

// ---------------------------------------------------------------------------
// Launch 2: down projection and the weighted combine
// ---------------------------------------------------------------------------

// One 64-weight chunk of a W_down row against the fp32 h of `m_act` pairs:
// pair r's chunk at hc + r * stride (16 contiguous granules), its two sub-block
// sums at hsc + r * nsub. Quants become exact fp32 two at a time (a nibble byte
// read as e4m3 is q * 2^-9; the conversion scales by 2^9).
template <int T>
__device__ __forceinline__ void chunk_f32(float (&acc)[T], const int m_act, const uint4 hdr, const uint4 qa,
                                          const uint4 qb, const ScaleSel &sel, const uint4 *__restrict__ hc,
                                          const int stride, const float *__restrict__ hsc, const int nsub) {
  const ChunkScales cs = chunk_scales(hdr, sel);
  const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  float s_lo[T], s_hi[T];
#pragma unroll
  for (int r = 0; r < T; ++r) s_lo[r] = s_hi[r] = 0.0f;
  // quant word g: weights 4g..4g+3 of sub-block 2c (low nibbles) and of 2c+1 (high nibbles)
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const uint32_t l = qw[g] & 0x0F0F0F0Fu;
    const uint32_t hb = (qw[g] >> 4) & 0x0F0F0F0Fu;
    const floatx2 l01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, false);
    const floatx2 l23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(l, 512.0f, true);
    const floatx2 h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb, 512.0f, false);
    const floatx2 h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb, 512.0f, true);
#pragma unroll
    for (int r = 0; r < T; ++r) {
      if (r >= m_act) break;
      const uint4 v = hc[r * stride + g];
      const uint4 u = hc[r * stride + 8 + g];
      s_lo[r] = __builtin_fmaf(l01.x, __builtin_bit_cast(float, v.x), s_lo[r]);
      s_hi[r] = __builtin_fmaf(h01.x, __builtin_bit_cast(float, u.x), s_hi[r]);
      s_lo[r] = __builtin_fmaf(l01.y, __builtin_bit_cast(float, v.y), s_lo[r]);
      s_hi[r] = __builtin_fmaf(h01.y, __builtin_bit_cast(float, u.y), s_hi[r]);
      s_lo[r] = __builtin_fmaf(l23.x, __builtin_bit_cast(float, v.z), s_lo[r]);
      s_hi[r] = __builtin_fmaf(h23.x, __builtin_bit_cast(float, u.z), s_hi[r]);
      s_lo[r] = __builtin_fmaf(l23.y, __builtin_bit_cast(float, v.w), s_lo[r]);
      s_hi[r] = __builtin_fmaf(h23.y, __builtin_bit_cast(float, u.w), s_hi[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if (r >= m_act) break;
    const float2 hsm = *reinterpret_cast<const float2 *>(hsc + r * nsub);
    acc[r] = __builtin_fmaf(cs.a0, s_lo[r], acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, hsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi[r], acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, hsm.y, acc[r]);
  }
}

// h of all pairs in LDS: chunk q (64 values, 16 granules) of the concatenated
// pair rows at granules 17q .. 17q + 15. Four lanes of a row read granule i of
// four consecutive chunks: bank groups (q + i) mod 16, all distinct.
__device__ __forceinline__ int h_slot(int g) { return (g >> 4) * 17 + (g & 15); }

constexpr int kTableWords = (int)(sizeof(Table) / 4);
static_assert(kTableWords <= kThreads, "one table word per thread");

constexpr int kHBatch = 4;  // h granules per thread per batch

__device__ __forceinline__ void load_h_batch(const uint4 *__restrict__ hg, const int base, const int total,
                                             uint4 (&v)[kHBatch]) {
#pragma unroll
  for (int i = 0; i < kHBatch; ++i) {
    const int g = base + (int)threadIdx.x + i * kThreads;
    v[i] = hg[g < total ? g : 0];
  }
}

// Lanes past the end store their clamped load (granule 0) to granule 0's slot
// (unguarded, as in store_x_batch).
__device__ __forceinline__ void store_h_batch(uint4 *hs, const int base, const int total,
                                              const uint4 (&v)[kHBatch]) {
#pragma unroll
  for (int i = 0; i < kHBatch; ++i) {
    const int g = base + (int)threadIdx.x + i * kThreads;
    hs[h_slot(g < total ? g : 0)] = v[i];
  }
}

// Every pair's h from the workspace into LDS, two batches per round trip; no
// other load is waited for in between, so each round's waits are exact.
__device__ __forceinline__ void stage_h(const uint4 *__restrict__ hg, const int total, uint4 *hs) {
  for (int base = 0; base < total; base += 2 * kHBatch * kThreads) {
    uint4 hb0[kHBatch], hb1[kHBatch];
    load_h_batch(hg, base, total, hb0);
    load_h_batch(hg, base + kHBatch * kThreads, total, hb1);
    store_h_batch(hs, base, total, hb0);
    store_h_batch(hs, base + kHBatch * kThreads, total, hb1);
  }
}

// Workgroup `tile` of launch 2: W_down rows 8 tile .. + 7 for every pair, then
// the weighted combine.
template <int T>
__device__ __forceinline__ void down_body(const uint8_t *__restrict__ w_down, const uint8_t *__restrict__ ws,
                                          float *__restrict__ y, const int hidden, const int ffn, const int P,
                                          const int tile, Table &R, float (&zbuf)[kMaxPairs][kDnRows], uint4 *lds) {
  const int tid = threadIdx.x;
  const int cpr = ffn >> 6;   // 64-value chunks per h row
  const int nsub = ffn >> 5;
  const int nblk = ffn >> 8;
  uint4 *hs = lds;
  float *hsum = reinterpret_cast<float *>(lds + (size_t)P * cpr * 17);

  // The tables and every pair's h are in LDS before the barrier; no load is
  // outstanding yet, so each round's waits are exact and its loads are all in
  // flight together.
  {
    const int tword = reinterpret_cast<const int *>(ws)[tid < kTableWords ? tid : 0];
    stage_h(reinterpret_cast<const uint4 *>(ws + kTableBytes), P * (ffn >> 2), hs);
    reinterpret_cast<int *>(&R)[tid < kTableWords ? tid : 0] = tword;  // lanes past the table rewrite word 0
  }
  __syncthreads();

  // lane group grp (32 lanes: 8 rows x 4 chunks) takes distinct experts grp, grp + 8, ...
  const addr::MoeDnLane ln = addr::moe_dn_lane(hidden, ffn, R.n_slots, tile, tid);
  const int grp = ln.grp;
  const int c = ln.c;
  const int i_row = (tid & 31) >> 2;
  const size_t expert_bytes = (size_t)hidden * (size_t)nblk * kQ4KBlockBytes;
  // rows past the matrix read row 0 (their results are never stored)
  const uint8_t *wrow = w_down + ln.row;
  const int U = ln.units;  // units (expert, block), expert-major

  uint4 wh[kDnDepth], wa[kDnDepth], wb[kDnDepth];
  int ls = grp, lb = 0;  // next unit to load
#pragma unroll
  for (int u = 0; u < kDnDepth; ++u) {
    if (u < U) {
      load_dn_unit(addr::moe_dn_unit_at(wrow, R.slot_expert[ls], expert_bytes, lb), c, wh[u], wa[u], wb[u]);
      addr::moe_dn_next(ls, lb, nblk, kDnGroups);
    }
  }

  // sub-block sums (32 values each, index order); sub-block t is half t & 1 of chunk t >> 1
  for (int t = tid; t < P * nsub; t += kThreads) {
    const uint4 *src = hs + (t >> 1) * 17 + (t & 1) * 8;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 g = src[q];
      s += __builtin_bit_cast(float, g.x);
      s += __builtin_bit_cast(float, g.y);
      s += __builtin_bit_cast(float, g.z);
      s += __builtin_bit_cast(float, g.w);
    }
    hsum[t] = s;
  }
  __syncthreads();

  const ScaleSel sel = scale_selectors(c);
  const int stride = cpr * 17;
  float acc[T];
#pragma unroll
  for (int r = 0; r < T; ++r) acc[r] = 0.0f;
  int cs_ = grp, cb = 0;  // unit being computed
  for (int u0 = 0; u0 < U; u0 += kDnDepth) {
#pragma unroll
    for (int u = 0; u < kDnDepth; ++u) {
      if (u0 + u < U) {
        const int p0 = R.slot_pair0[cs_], ntok = R.slot_ntok[cs_];
        const int ci = 4 * cb + c;
        chunk_f32<T>(acc, ntok, wh[u], wa[u], wb[u], sel, hs + (p0 * cpr + ci) * 17, stride,
                     hsum + p0 * nsub + 2 * ci, nsub);
        if (u0 + u + kDnDepth < U) {
          load_dn_unit(addr::moe_dn_unit_at(wrow, R.slot_expert[ls], expert_bytes, lb), c, wh[u], wa[u], wb[u]);
          addr::moe_dn_next(ls, lb, nblk, kDnGroups);
        }
        if (++cb == nblk) {
          // the expert's row is complete: one z per token, reduced over the row's four lanes (one quad)
#pragma unroll
          for (int r = 0; r < T; ++r) {
            if (r >= ntok) break;
            const float z = row4_sum(acc[r]);
            if (c == r) zbuf[p0 + r][i_row] = z;
            acc[r] = 0.0f;
          }
          cb = 0;
          cs_ += kDnGroups;
        }
      }
    }
  }
  __syncthreads();

  // y[t][n] = sum over token t's experts in routing rank order of weight * z
  if (tid < T * kDnRows) {
    const int t = tid / kDnRows, i = tid % kDnRows;
    const int nn = tile * kDnRows + i;
    const int K = P / T;
    float out = 0.0f;
    for (int j = 0; j < K; ++j) {
      const int p = R.rank_pair[t * K + j];
      out = __builtin_fmaf(R.pair_weight[p], zbuf[p][i], out);
    }
    if (nn < hidden) y[(size_t)t * hidden + nn] = out;
  }
}


template <int T>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const uint8_t *__restrict__ w_down,
                                                            const uint8_t *__restrict__ ws, float *__restrict__ y,
                                                            const int hidden, const int ffn, const int P) {
  __shared__ Table R;
  __shared__ float zbuf[kMaxPairs][kDnRows];
  extern __shared__ uint4 lds[];
  down_body<T>(w_down, ws, y, hidden, ffn, P, (int)blockIdx.x, R, zbuf, lds);
}

template <int T>
int launch_t(const void *w_gate, const void *w_up, const void *w_down, const float *logits, const uint16_t *x,
             float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int hidden, int ffn,
             int n_experts, int top_k, hipStream_t s) {
  static LdsGrant granted_a, granted_b;
  const size_t lds_a = layout::q4k_moe_gate_up_lds(T, hidden), lds_b = layout::q4k_moe_down_lds(T * top_k, ffn);
  const int max_slots = n_experts < T * top_k ? n_experts : T * top_k;
  constexpr int kUpRows = addr::moe_up_rows(T);
  const dim3 grid_a((unsigned)((ffn + kUpRows - 1) / kUpRows), (unsigned)max_slots);
  const dim3 grid_b((unsigned)((hidden + kDnRows - 1) / kDnRows));
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&moe_gate_up_kernel<T>), lds_a, granted_a,
                        "moe_gate_up_kernel lds") ||
      allow_dynamic_lds(reinterpret_cast<const void *>(&moe_down_kernel<T>), lds_b, granted_b, "moe_down_kernel lds"))
    return QMV_ERR_HIP;
  int rc = launch_kernel("moe_gate_up_kernel", moe_gate_up_kernel<T>, grid_a, dim3(kThreads), lds_a, s, w_gate, w_up,
                         logits, x, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k);
  if (rc) return rc;
  return launch_kernel("moe_down_kernel", moe_down_kernel<T>, grid_b, dim3(kThreads), lds_b, s, w_down, ws, y,
                       hidden, ffn, T * top_k);
}

}  // namespace

namespace {

// Scratch of qmv_q4_k_moe_noalloc: the routing tables and h of one call, in a
// fixed device array instead of a caller's workspace. Each GPU the library
// runs on holds its own copy until the process ends. Host code never passes
// the array's name to a kernel (on the host it only stands in for the symbol):
// it uses the device address hipGetSymbolAddress returns, looked up once per
// device and kept here.
static __device__ __align__(256) uint8_t scratch[layout::kMoeNoAllocBytes];
std::atomic<void *> g_scratch_addr[LdsGrant::kDevices];

// Device address of `scratch` on the current device, or nullptr after
// recording the HIP error.
void *scratch_address() {
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e == hipSuccess && (d < 0 || d >= LdsGrant::kDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    set_error_detail("qmv_q4_k_moe_noalloc device", (int)e, hipGetErrorString(e));
    return nullptr;
  }
  void *p = g_scratch_addr[d].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    set_error_detail("qmv_q4_k_moe_noalloc scratch address", (int)e, hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_addr[d].store(p, std::memory_order_release);
  return p;
}

}  // namespace

int launch_q4_k_moe(const void *w_gate, const void *w_up, const void *w_down, const float *logits, const uint16_t *x,
                    float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int t, int hidden, int ffn,
                    int n_experts, int top_k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (t) {
    case 1: return launch_t<1>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 2: return launch_t<2>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 3: return launch_t<3>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 4: return launch_t<4>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_q4_k_moe_noalloc(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                            const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, int t,
                            int hidden, int ffn, int n_experts, int top_k, void *stream) {
  // the launches write every table and h value they read, so nothing in the
  // array needs clearing between calls
  void *ws = scratch_address();
  if (!ws) return QMV_ERR_HIP;
  return launch_q4_k_moe(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, t, hidden, ffn, n_experts,
                         top_k, stream);
}

}  // namespace qmv
