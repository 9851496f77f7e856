// Routed-expert MoE feed-forward on IQ4_XS experts, gfx950.
//
// The memra README's model support table lists its 35B-A3B MoE (hidden 2048,
// 128 experts, top-8; the speed table's MoE decode row) in IQ4_XS. The
// routing, its tables and the two-launch structure are those of the Q4_K form
// (moe_routing.h): per token the top-k router logits pick experts, their
// softmax restricted to the chosen k weights the experts' silu-gated FFN
// outputs.
//
//  1. iq4xs_moe_gate_up_kernel, grid (F/16 row tiles) x (max distinct experts).
//     The activations of all T tokens (pair-interleaved, as in the IQ4_XS GEMV)
//     and the router logits are requested at once; the workgroup routes every
//     token in one pass (as the Q4_K form does); after one barrier every wave
//     sorts the pairs and finds its workgroup's distinct expert and the tokens
//     that chose it. 16 lanes own a W_gate and a
//     W_up row, lane l taking sub-blocks l, l + 16, ... of both; each index
//     byte becomes a bf16 weight pair through a 256-entry LDS table and meets
//     its activation pair in one dot2. h = silu(W_gate x) * (W_up x) in fp32
//     per (expert, token) pair goes to the workspace.
//  2. iq4xs_moe_down_kernel, grid H/8 row tiles. Every pair's h (fp32) is
//     staged in LDS with the routing tables; 8 lanes own a W_down row, lane j
//     taking sub-block j of each super-block, and the workgroup's four waves
//     share its 8 rows, wave w taking the distinct experts w, w + 4, ... Each
//     index byte becomes an fp32 weight pair through a 256-entry LDS table of
//     float pairs; products with h accumulate in fp32 (fma). y_t = sum over
//     token t's experts, in routing rank order, of weight * z, from zero.
//
// Each selected expert's weights are read once per call, and a token's result
// is bit-identical whatever other tokens share the call: the arithmetic of an
// (expert, token) pair does not depend on which lanes or waves run it.
#include "iq4xs_common.h"
#include "moe_routing.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

using namespace iq4xs;
using namespace moe;

constexpr int kWaves = addr::kIq4MoeDnWaves;
constexpr int kThreads = 64 * kWaves;
static_assert(kThreads == kTableEntries, "one table entry per thread");
static_assert(kThreads == kRouteThreads, "the gate/up workgroup routes with every thread");
// gate/up: 16 lanes per W row, 4 rows per wave, 16 rows per workgroup
constexpr int kUpDepth = addr::kIq4MoeUpDepth;   // units (gate and up) of loads in flight per lane
// down: 8 lanes per W row (one sub-block each), 8 rows per wave and workgroup
constexpr int kDnLanes = addr::kIq4MoeDnLanes;
constexpr int kDnRows = addr::kIq4MoeDnRows;
constexpr int kDnDepth = addr::kIq4MoeDnDepth;   // (expert, super-block) units of loads in flight per lane
static_assert(kThreads == 256 && kDnRows == 64 / kDnLanes, "the shapes the addressing assumes");
constexpr int kTableWords = (int)(sizeof(Table) / 4);
static_assert(kTableWords <= kThreads, "one table word per thread");

// ---------------------------------------------------------------------------
// Launch 1: gate and up projections, silu gating
// ---------------------------------------------------------------------------

template <int T>
__global__ __launch_bounds__(kThreads) void iq4xs_moe_gate_up_kernel(
    const uint8_t *__restrict__ w_gate, const uint8_t *__restrict__ w_up, const float *__restrict__ logits,
    const uint16_t *__restrict__ x, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ pairs_out, uint8_t *__restrict__ ws, const int hidden, const int ffn, const int E,
    const int K) {
  __shared__ __align__(16) RouteLds rl;
  __shared__ uint32_t tbl[kTableEntries];
  extern __shared__ uint4 xs[];
  const uint8_t *tbl_bytes = reinterpret_cast<const uint8_t *>(tbl);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nblk = hidden >> 8, nsub = nblk * 8, rg = row_granules(nsub);

  // every token's first sub-blocks and the router logits are requested together
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const int total = T * nsub;
  uint4 g[4];
  {
    const int t = tid < total ? tid : 0;   // a clamped lane re-stages sub-block 0
    const int r = t / nsub, s = t - r * nsub;
#pragma unroll
    for (int q = 0; q < 4; ++q) g[q] = xg[(size_t)r * (hidden >> 3) + 4 * s + q];
  }
  const WgLogits<T> lg = load_logits_wg<T>(logits, E);
  {
    const int t = tid < total ? tid : 0;
    const int r = t / nsub, s = t - r * nsub;
    uint4 o[4];
    interleave(g[0], g[1], g[2], g[3], o);
#pragma unroll
    for (int q = 0; q < 4; ++q) xs[r * rg + x_slot(s) + q] = o[q];
  }
  tbl[tid] = grid_bf16((uint32_t)tid & 15u) | (grid_bf16((uint32_t)tid >> 4) << 16);
  uint32_t *kr = reinterpret_cast<uint32_t *>(xs + (size_t)T * rg);   // routing rows
  store_keys<T>(lg, E, kr, rl);
  for (int t = tid + kThreads; t < total; t += kThreads) {
    const int r = t / nsub, s = t - r * nsub;
    const uint4 *src = xg + (size_t)r * (hidden >> 3) + 4 * s;
    uint4 o[4];
    interleave(src[0], src[1], src[2], src[3], o);
#pragma unroll
    for (int q = 0; q < 4; ++q) xs[r * rg + x_slot(s) + q] = o[q];
  }
  __syncthreads();
  route_wave<T>(kr, E, K, rl);
  __syncthreads();

  const int P = T * K;
  const PairRank pr = pair_ranks<T>(rl, P);
  const Slot<T> sl = my_slot<T>(pr, (int)blockIdx.y, P);
  if (sl.p0 < 0) return;  // fewer distinct experts than the grid allows for (uniform over the workgroup)

  // kUpLanes lanes per row: 32 for one token, 16 for more. Both give a row the
  // same bits: a lane's units are summed in two chains by unit parity for 16
  // lanes (sub-blocks l + 32 t and l + 16 + 32 t), which for 32 lanes are lanes
  // l and l + 16; the chains are added, then summed over 16 lanes.
  constexpr int kUpLanes = addr::iq4_moe_up_lanes(T), kUpRows = addr::iq4_moe_up_rows(T);
  const int l = tid % kUpLanes;
  const int f = blockIdx.x * kUpRows + tid / kUpLanes;
  // lane l: sub-blocks u = l + 16 t -> super-block (l >> 3) + 2 t, sub-block j = l & 7
  const addr::Iq4Lane ln = addr::iq4_moe_up_lane(kUpLanes, sl.e, ffn, hidden, blockIdx.x, tid);
  const uint8_t *grow = w_gate + ln.row_base, *urow = w_up + ln.row_base;
  const uint8_t *gl = w_gate + ln.lane_base, *ul = w_up + ln.lane_base;
  const int j = l & 7, qoff = ln.qoff;
  const int nlive = ln.nlive;
  const int nslots = addr::iq4_slots(kUpLanes, nblk, kUpDepth);
  constexpr int kXStride = 4 * kUpLanes + kUpLanes / 4;
  const int x_l = x_slot(l < nsub ? l : 0);

  Unit rg_[kUpDepth], ru_[kUpDepth];
#pragma unroll
  for (int d = 0; d < kUpDepth; ++d) {
    load_unit((d < nlive ? gl + addr::iq4_unit_offset(d, ln.unit_bytes) : grow), qoff, rg_[d]);
    load_unit((d < nlive ? ul + addr::iq4_unit_offset(d, ln.unit_bytes) : urow), qoff, ru_[d]);
  }
  // the weights (softmax) and the routing outputs, off the path to the loads
  // above: the last wave of workgroup (0, 0)
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid >= kThreads - 64)
    write_routing(with_weights(sorted_pairs(pr, P), rl, P, K), P, topk_ids, topk_w, pairs_out,
                  reinterpret_cast<Table *>(ws));

  int xoff[T];
#pragma unroll
  for (int r = 0; r < T; ++r) xoff[r] = sl.tok[r] * rg;
  const int sh_lo = 4 * j, sh_hi = 16 + 2 * j;
  float acc_g[2][T], acc_u[2][T];   // the two chains (32 lanes: chain 0 only)
#pragma unroll
  for (int r = 0; r < T; ++r) acc_g[0][r] = acc_u[0][r] = acc_g[1][r] = acc_u[1][r] = 0.0f;
  static_assert(kUpDepth == 2, "16 lanes: unit parity is the ring slot");
  constexpr int kOdd = kUpLanes == 16 ? 1 : 0;
  for (int t0 = 0; t0 < nslots; t0 += kUpDepth) {
#pragma unroll
    for (int d = 0; d < kUpDepth; ++d) {
      const int t = t0 + d;
      const bool live = t < nlive;
      const float dg_raw = sub_scale(rg_[d].hdr, sh_lo, sh_hi);
      const float du_raw = sub_scale(ru_[d].hdr, sh_lo, sh_hi);
      const float dg = live ? dg_raw : 0.0f, du = live ? du_raw : 0.0f;
      const int xg0 = live ? x_l + t * kXStride : x_l;
      const Pairs g0 = word_pairs(tbl_bytes, rg_[d].q0.x), g1 = word_pairs(tbl_bytes, rg_[d].q0.y);
      const Pairs g2 = word_pairs(tbl_bytes, rg_[d].q1.x), g3 = word_pairs(tbl_bytes, rg_[d].q1.y);
      const Pairs u0 = word_pairs(tbl_bytes, ru_[d].q0.x), u1 = word_pairs(tbl_bytes, ru_[d].q0.y);
      const Pairs u2 = word_pairs(tbl_bytes, ru_[d].q1.x), u3 = word_pairs(tbl_bytes, ru_[d].q1.y);
      {
        const int tn = t + kUpDepth;
        load_unit((tn < nlive ? gl + addr::iq4_unit_offset(tn, ln.unit_bytes) : grow), qoff, rg_[d]);
        load_unit((tn < nlive ? ul + addr::iq4_unit_offset(tn, ln.unit_bytes) : urow), qoff, ru_[d]);
      }
#pragma unroll
      for (int r = 0; r < T; ++r) {
        if (r >= sl.ntok) break;
        const uint4 *xp = xs + xoff[r] + xg0;
        const uint4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
        float a0 = pairs_dot(g0, x0, 0.0f), a1 = pairs_dot(g1, x1, 0.0f);
        a0 = pairs_dot(g2, x2, a0);
        a1 = pairs_dot(g3, x3, a1);
        float b0 = pairs_dot(u0, x0, 0.0f), b1 = pairs_dot(u1, x1, 0.0f);
        b0 = pairs_dot(u2, x2, b0);
        b1 = pairs_dot(u3, x3, b1);
        acc_g[d * kOdd][r] = __builtin_fmaf(dg, a0 + a1, acc_g[d * kOdd][r]);
        acc_u[d * kOdd][r] = __builtin_fmaf(du, b0 + b1, acc_u[d * kOdd][r]);
      }
    }
  }

  float *h = reinterpret_cast<float *>(ws + kTableBytes);
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if (r >= sl.ntok) break;
    float vg, vu;
    if constexpr (kUpLanes == 32) {   // lane l ^ 16 holds the other chain
      vg = acc_g[0][r] + __shfl_xor(acc_g[0][r], 16);
      vu = acc_u[0][r] + __shfl_xor(acc_u[0][r], 16);
    } else {
      vg = acc_g[0][r] + acc_g[1][r];
      vu = acc_u[0][r] + acc_u[1][r];
    }
    const float gv = group_sum<16>(vg);
    const float uv = group_sum<16>(vu);
    if (l == r && f < ffn) h[(size_t)(sl.p0 + r) * ffn + f] = gv / (1.0f + expf(-gv)) * uv;
  }
}

// ---------------------------------------------------------------------------
// Launch 2: down projection and the weighted combine
// ---------------------------------------------------------------------------

// h of all pairs in LDS: sub-block s (32 floats, 8 granules) of the concatenated
// pair rows at granules 9 s .. 9 s + 7. The 8 lanes of a row read granule q of
// 8 consecutive sub-blocks: 144-byte strides put them in 8 distinct bank groups.
__device__ __forceinline__ int h_slot(int g) { return (g >> 3) * 9 + (g & 7); }

constexpr int kHBatch = 4;  // h granules per thread per batch

__device__ __forceinline__ void load_h_batch(const uint4 *__restrict__ hg, const int base, const int total,
                                             uint4 (&v)[kHBatch]) {
#pragma unroll
  for (int i = 0; i < kHBatch; ++i) {
    const int g = base + (int)threadIdx.x + i * kThreads;
    v[i] = hg[g < total ? g : 0];
  }
}

// Lanes past the end store their clamped load (granule 0) to granule 0's slot:
// no store is guarded, so no load waits inside a store's branch.
__device__ __forceinline__ void store_h_batch(uint4 *hs, const int base, const int total,
                                              const uint4 (&v)[kHBatch]) {
#pragma unroll
  for (int i = 0; i < kHBatch; ++i) {
    const int g = base + (int)threadIdx.x + i * kThreads;
    hs[h_slot(g < total ? g : 0)] = v[i];
  }
}

// The 8 fp32 weight pairs (grid[lo], grid[hi]) of index word w, scaled later.
struct FPairs {
  float2 e[4];
};
template <int B>
__device__ __forceinline__ float2 table_fpair(const uint8_t *__restrict__ tblf_bytes, const uint32_t w) {
  return *reinterpret_cast<const float2 *>(tblf_bytes + byte_x8<B>(w));
}
__device__ __forceinline__ FPairs word_fpairs(const uint8_t *__restrict__ tblf_bytes, const uint32_t w) {
  return FPairs{{table_fpair<0>(tblf_bytes, w), table_fpair<1>(tblf_bytes, w), table_fpair<2>(tblf_bytes, w),
                 table_fpair<3>(tblf_bytes, w)}};
}

// sum over index word q's 8 weights of grid * h: lo weights meet h[4q .. 4q+3]
// (granule q of the sub-block), hi weights h[16 + 4q ..] (granule 4 + q)
__device__ __forceinline__ void fpairs_fma(const FPairs &p, const uint4 lo, const uint4 hi, float &s_lo,
                                           float &s_hi) {
  s_lo = __builtin_fmaf(p.e[0].x, __builtin_bit_cast(float, lo.x), s_lo);
  s_hi = __builtin_fmaf(p.e[0].y, __builtin_bit_cast(float, hi.x), s_hi);
  s_lo = __builtin_fmaf(p.e[1].x, __builtin_bit_cast(float, lo.y), s_lo);
  s_hi = __builtin_fmaf(p.e[1].y, __builtin_bit_cast(float, hi.y), s_hi);
  s_lo = __builtin_fmaf(p.e[2].x, __builtin_bit_cast(float, lo.z), s_lo);
  s_hi = __builtin_fmaf(p.e[2].y, __builtin_bit_cast(float, hi.z), s_hi);
  s_lo = __builtin_fmaf(p.e[3].x, __builtin_bit_cast(float, lo.w), s_lo);
  s_hi = __builtin_fmaf(p.e[3].y, __builtin_bit_cast(float, hi.w), s_hi);
}

template <int T>
__global__ __launch_bounds__(kThreads) void iq4xs_moe_down_kernel(const uint8_t *__restrict__ w_down,
                                                                  const uint8_t *__restrict__ ws,
                                                                  float *__restrict__ y, const int hidden,
                                                                  const int ffn, const int P) {
  __shared__ Table R;
  __shared__ float zbuf[kMaxPairs][kDnRows];
  __shared__ float2 tblf[kTableEntries];
  extern __shared__ uint4 hs[];
  const uint8_t *tblf_bytes = reinterpret_cast<const uint8_t *>(tblf);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nblk = ffn >> 8, nsub = nblk * 8;

  // tables and every pair's h before the barrier, two h batches per round trip
  const uint4 *hg = reinterpret_cast<const uint4 *>(ws + kTableBytes);
  const int total = P * (ffn >> 2);
  {
    const int tword = reinterpret_cast<const int *>(ws)[tid < kTableWords ? tid : 0];
    for (int base = 0; base < total; base += 2 * kHBatch * kThreads) {
      uint4 hb0[kHBatch], hb1[kHBatch];
      load_h_batch(hg, base, total, hb0);
      load_h_batch(hg, base + kHBatch * kThreads, total, hb1);
      store_h_batch(hs, base, total, hb0);
      store_h_batch(hs, base + kHBatch * kThreads, total, hb1);
    }
    reinterpret_cast<int *>(&R)[tid < kTableWords ? tid : 0] = tword;  // lanes past the table rewrite word 0
    tblf[tid] = make_float2(__builtin_bit_cast(float, grid_bf16((uint32_t)tid & 15u) << 16),
                            __builtin_bit_cast(float, grid_bf16((uint32_t)tid >> 4) << 16));
  }
  __syncthreads();

  // wave w takes distinct experts w, w + 4, ...; lane: row i_row, sub-block j
  const int j = lane & (kDnLanes - 1), i_row = lane / kDnLanes;
  const addr::Iq4DnLane ln = addr::iq4_moe_dn_lane(hidden, ffn, R.n_slots, blockIdx.x, tid);
  const size_t expert_bytes = (size_t)hidden * (size_t)nblk * kIQ4XSBlockBytes;
  const uint8_t *wrow = w_down + ln.row;   // rows past the matrix read row 0
  const int qoff = ln.qoff;
  const int U = ln.units;   // units (expert, super-block), expert-major

  Unit ring[kDnDepth];
  int ls = wave, lb = 0;   // next unit to load; units past U re-read this row of the first slot's expert
#pragma unroll
  for (int u = 0; u < kDnDepth; ++u) {
    const bool ok = u < U;
    load_unit(addr::iq4_moe_dn_unit_at(wrow, R.slot_expert[ok ? ls : 0], expert_bytes, ok ? lb : 0), qoff, ring[u]);
    if (ok) addr::moe_dn_next(ls, lb, nblk, kWaves);
  }

  const int sh_lo = 4 * j, sh_hi = 16 + 2 * j;
  float acc[T];
#pragma unroll
  for (int r = 0; r < T; ++r) acc[r] = 0.0f;
  int cs = wave, cb = 0;   // unit being computed
  for (int u0 = 0; u0 < U; u0 += kDnDepth) {
#pragma unroll
    for (int u = 0; u < kDnDepth; ++u) {
      if (u0 + u < U) {
        const int p0 = R.slot_pair0[cs], ntok = R.slot_ntok[cs];
        const float dl = sub_scale(ring[u].hdr, sh_lo, sh_hi);
        const FPairs w0 = word_fpairs(tblf_bytes, ring[u].q0.x), w1 = word_fpairs(tblf_bytes, ring[u].q0.y);
        const FPairs w2 = word_fpairs(tblf_bytes, ring[u].q1.x), w3 = word_fpairs(tblf_bytes, ring[u].q1.y);
        {
          const bool ok = u0 + u + kDnDepth < U;
          load_unit(addr::iq4_moe_dn_unit_at(wrow, R.slot_expert[ok ? ls : 0], expert_bytes, ok ? lb : 0), qoff,
                    ring[u]);
          if (ok) addr::moe_dn_next(ls, lb, nblk, kWaves);
        }
        const int sb = 8 * cb + j;
#pragma unroll
        for (int r = 0; r < T; ++r) {
          if (r >= ntok) break;
          const uint4 *hp = hs + ((p0 + r) * nsub + sb) * 9;
          float s_lo = 0.0f, s_hi = 0.0f;
          fpairs_fma(w0, hp[0], hp[4], s_lo, s_hi);
          fpairs_fma(w1, hp[1], hp[5], s_lo, s_hi);
          fpairs_fma(w2, hp[2], hp[6], s_lo, s_hi);
          fpairs_fma(w3, hp[3], hp[7], s_lo, s_hi);
          acc[r] = __builtin_fmaf(dl, s_lo + s_hi, acc[r]);
        }
        if (++cb == nblk) {
          // the expert's row is complete: one z per token, reduced over the row's 8 lanes
#pragma unroll
          for (int r = 0; r < T; ++r) {
            if (r >= ntok) break;
            const float z = group_sum<kDnLanes>(acc[r]);
            if (j == r) zbuf[p0 + r][i_row] = z;
            acc[r] = 0.0f;
          }
          cb = 0;
          cs += kWaves;
        }
      }
    }
  }
  __syncthreads();

  // y[t][n] = sum over token t's experts in routing rank order of weight * z
  if (tid < T * kDnRows) {
    const int t = tid / kDnRows, i = tid % kDnRows;
    const int nn = blockIdx.x * kDnRows + i;
    const int K = P / T;
    float out = 0.0f;
    for (int jj = 0; jj < K; ++jj) {
      const int p = R.rank_pair[t * K + jj];
      out = __builtin_fmaf(R.pair_weight[p], zbuf[p][i], out);
    }
    if (nn < hidden) y[(size_t)t * hidden + nn] = out;
  }
}


template <int T>
int launch_t(const void *w_gate, const void *w_up, const void *w_down, const float *logits, const uint16_t *x,
             float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int hidden, int ffn,
             int n_experts, int top_k, hipStream_t s) {
  static LdsGrant granted_a, granted_b;
  const size_t lds_a = layout::iq4xs_moe_gate_up_lds(T, hidden), lds_b = layout::iq4xs_moe_down_lds(T * top_k, ffn);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&iq4xs_moe_gate_up_kernel<T>), lds_a, granted_a,
                        "iq4xs_moe_gate_up_kernel lds") ||
      allow_dynamic_lds(reinterpret_cast<const void *>(&iq4xs_moe_down_kernel<T>), lds_b, granted_b,
                        "iq4xs_moe_down_kernel lds"))
    return QMV_ERR_HIP;
  const int max_slots = n_experts < T * top_k ? n_experts : T * top_k;
  constexpr int kUpRows = addr::iq4_moe_up_rows(T);
  const dim3 grid_a((unsigned)((ffn + kUpRows - 1) / kUpRows), (unsigned)max_slots);
  int rc = launch_kernel("iq4xs_moe_gate_up_kernel", iq4xs_moe_gate_up_kernel<T>, grid_a, dim3(kThreads), lds_a, s,
                         w_gate, w_up, logits, x, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k);
  if (rc) return rc;
  const dim3 grid_b((unsigned)((hidden + kDnRows - 1) / kDnRows));
  return launch_kernel("iq4xs_moe_down_kernel", iq4xs_moe_down_kernel<T>, grid_b, dim3(kThreads), lds_b, s, w_down,
                       ws, y, hidden, ffn, T * top_k);
}

}  // namespace

int launch_iq4_xs_moe(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                      const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int t,
                      int hidden, int ffn, int n_experts, int top_k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (t) {
    case 1: return launch_t<1>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 2: return launch_t<2>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 3: return launch_t<3>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    case 4: return launch_t<4>(w_gate, w_up, w_down, logits, x, y, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k, s);
    default: return QMV_ERR_RANGE;
  }
}

}  // namespace qmv
