// Routing of the routed-expert MoE launches (shared by the Q4_K and IQ4_XS
// forms): top-k selection of the router logits inside one wave, the softmax
// over the chosen k, the (expert, token) pairs sorted in registers, and the
// tables the first launch leaves in the workspace for the second.
//
// The selection follows the memra README speed table's 35B-A3B MoE decode
// (128 experts, top-8): per token the k largest logits, ties to the lower
// expert id, weighted by their softmax restricted to the chosen k.
#pragma once

#include <limits.h>

#include "qmv_device.h"
#include "qmv_layout.h"
#include "../../include/qmv.h"

namespace qmv {
namespace moe {

constexpr int kMaxPairs = QMV_MOE_MAX_TOKENS * QMV_MOE_MAX_TOP_K;
constexpr int kTopK = QMV_MOE_MAX_TOP_K;

// Tables at the start of the workspace, written by launch 1 and read by launch 2.
struct Table {
  int n_pairs;
  int n_slots;
  int pair_expert[kMaxPairs];  // gather list: sorted by expert, then token
  int pair_token[kMaxPairs];
  float pair_weight[kMaxPairs];
  int slot_expert[kMaxPairs];  // distinct experts, ascending
  int slot_pair0[kMaxPairs];   // first gather-list position of each
  int slot_ntok[kMaxPairs];    // tokens that chose it
  int rank_pair[kMaxPairs];    // gather-list position of routing pair t*K + j (token t, rank j)
};
constexpr size_t kTableBytes = layout::kMoeTableBytes;
static_assert(sizeof(Table) <= kTableBytes, "routing tables exceed their workspace slot");
static_assert(sizeof(Table) % 4 == 0, "routing tables are copied as words");

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------

// Logits as order-preserving unsigned keys: for finite a, b (with -0 made +0
// first), a < b exactly when key(a) < key(b). Key 0 marks an absent or
// already chosen expert; every finite logit maps above it.
__device__ __forceinline__ uint32_t logit_key(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum of k over the wave: DPP butterfly inside each 16-lane row, then the
// four row maxima on the scalar side.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = max(k, dpp_u32<0xB1>(k));   // quad_perm [1,0,3,2]
  k = max(k, dpp_u32<0x4E>(k));   // quad_perm [2,3,0,1]
  k = max(k, dpp_u32<0x141>(k));  // row_half_mirror
  k = max(k, dpp_u32<0x140>(k));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)k, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Token t's logits for lanes l, l + 64, l + 128, l + 192: four loads in flight
// at once (clamped, never guarded).
struct Logits {
  float v[4];
};
__device__ __forceinline__ Logits load_logits(const float *__restrict__ logits, const int t, const int E) {
  const int lane = threadIdx.x & 63;
  Logits r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    r.v[i] = logits[(size_t)t * E + (e < E ? e : E - 1)];
  }
  return r;
}

// One wave routes token t from its logits. Lane l holds experts l, l + 64,
// l + 128, l + 192. Each of the k rounds takes the largest remaining logit (a
// wave-wide max of the keys) and, among the experts holding it, the lowest id
// (the first candidate slot i whose ballot is non-empty, lowest lane in it),
// then retires that expert. The softmax over the chosen logits follows:
// exp(l_j - l_0) summed in rank order, each divided by the sum. Writes
// sid[t][j], swt[t][j] for j < K when `write`; every wave routes, so that no
// wave's logit loads wait inside a branch. Logits must be finite.
__device__ __forceinline__ void route_token(const Logits &lg, const int t, const bool write, const int E, const int K,
                                            int (*sid)[kTopK], float (*swt)[kTopK]) {
  const int lane = threadIdx.x & 63;
  uint32_t kv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kv[i] = lane + 64 * i < E ? logit_key(lg.v[i]) : 0u;
  // kept in registers: every loop below is fully unrolled with K tested inside
  uint32_t selk[kTopK];
  int seli[kTopK];
#pragma unroll
  for (int j = 0; j < kTopK; ++j) {
    selk[j] = 0u;
    seli[j] = 0;
    if (j < K) {
      const uint32_t m = wave_max_u32(max(max(kv[0], kv[1]), max(kv[2], kv[3])));
      int id = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned long long b = __ballot(kv[i] == m);
        if (id < 0 && b) id = 64 * i + __ffsll((long long)b) - 1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == id) kv[i] = 0u;
      selk[j] = m;
      seli[j] = id;
    }
  }
  const float l0 = key_logit(selk[0]);
  float ex[kTopK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kTopK; ++j) {
    ex[j] = 0.0f;
    if (j < K) {
      ex[j] = expf(key_logit(selk[j]) - l0);
      sum += ex[j];
    }
  }
#pragma unroll
  for (int j = 0; j < kTopK; ++j)
    if (write && j < K && lane == j) {
      sid[t][j] = seli[j];
      swt[t][j] = ex[j] / sum;
    }
}

// ---------------------------------------------------------------------------
// Routing of every token of a decode call, one wave per token
// ---------------------------------------------------------------------------
//
// The same selection as route_token (the K largest logits, among equal logits
// the lower id first, in rank order), found in one pass. The 64 lanes hold
// the token's keys of experts l, l + 64, l + 128, l + 192. Each group of 8
// consecutive experts has a largest key; tau, the least of those maxima over
// the ceil(E / 8) groups, has at least that many experts at or above it, so
// when there are at least K groups every one of the K largest keys is >= tau.
// The experts at or above tau (usually little more than K) are listed with
// their composite key (logit key, then the complement of the id: distinct,
// and larger for the lower id among equal logits) and each is ranked by
// counting the larger composites of the list.

constexpr int kRouteThreads = 256;
static_assert(QMV_MOE_MAX_TOKENS <= kRouteThreads / 64, "one wave per token");
static_assert(QMV_MOE_MAX_EXPERTS <= kRouteThreads, "one logit per thread and token");
// Per token in LDS: the keys (QMV_MOE_MAX_EXPERTS 32-bit words, zero past E),
// then, over the same bytes once the keys are in registers, the candidate list
// (up to QMV_MOE_MAX_EXPERTS 64-bit composites).
constexpr int kRouteStride = 2 * QMV_MOE_MAX_EXPERTS;   // 32-bit words per token
static_assert(layout::kMoeRouteBytesPerToken == kRouteStride * sizeof(uint32_t), "the LDS the launch reserves");

// The routing state in LDS: per token the chosen experts and keys in rank
// order, and the pair keys (expert * 4 + token) in routing order.
struct RouteLds {
  int sid[QMV_MOE_MAX_TOKENS][kTopK];
  uint32_t skey[QMV_MOE_MAX_TOKENS][kTopK];
  int pkey[kMaxPairs];
};

// Thread tid's logits: expert tid (clamped) of every token; the loads are
// unconditional, so they can be issued with the activations.
template <int T>
struct WgLogits {
  float v[T];
};
template <int T>
__device__ __forceinline__ WgLogits<T> load_logits_wg(const float *__restrict__ logits, const int E) {
  const int e = (int)threadIdx.x < E ? (int)threadIdx.x : E - 1;
  WgLogits<T> r;
#pragma unroll
  for (int t = 0; t < T; ++t) r.v[t] = logits[(size_t)t * E + e];
  return r;
}

// The keys into LDS (kr[t * kRouteStride + e]), zero past E: below every finite
// logit's key (at least 2^23); the pair keys cleared. A barrier must follow.
template <int T>
__device__ __forceinline__ void store_keys(const WgLogits<T> &lg, const int E, uint32_t *kr, RouteLds &rl) {
  const int e = (int)threadIdx.x;
#pragma unroll
  for (int t = 0; t < T; ++t) kr[t * kRouteStride + e] = e < E ? logit_key(lg.v[t]) : 0u;
  if (e < kMaxPairs) rl.pkey[e] = INT_MAX;   // pair keys past P: above every real one
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t k) {
  k = min(k, dpp_u32<0xB1>(k));   // quad_perm [1,0,3,2]
  k = min(k, dpp_u32<0x4E>(k));   // quad_perm [2,3,0,1]
  k = min(k, dpp_u32<0x141>(k));  // row_half_mirror
  k = min(k, dpp_u32<0x140>(k));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)k, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)k, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)k, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)k, 48);
  return min(min(r0, r1), min(r2, r3));
}

// Wave t routes token t (t < T): records the expert and key at each rank j <
// K in sid[t][j], skey[t][j] and the pair key in pkey[t * K + j]. A barrier
// must follow before they are read by other waves.
template <int T>
__device__ __forceinline__ void route_wave(uint32_t *kr, const int E, const int K, RouteLds &rl) {
  const int lane = (int)threadIdx.x & 63, t = (int)threadIdx.x >> 6;
  if (t >= T) return;   // uniform per wave
  uint32_t *row = kr + t * kRouteStride;
  uint32_t k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) k[i] = row[lane + 64 * i];
  // tau: the least of the group maxima over groups of 16 experts when there
  // are at least K of them, else of 8, else 1 (every expert a candidate). An
  // empty group (all zero) does not count.
  const bool g16 = (E + 15) / 16 >= K;
  uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (64 * i >= E) break;   // uniform: slots past the experts hold only zeros
    uint32_t m = k[i];
    m = max(m, dpp_u32<0xB1>(m));   // quad_perm [1,0,3,2]
    m = max(m, dpp_u32<0x4E>(m));   // quad_perm [2,3,0,1]
    m = max(m, dpp_u32<0x141>(m));  // row_half_mirror: the 8-lane group's maximum
    if (g16) m = max(m, dpp_u32<0x140>(m));   // row_mirror: the 16-lane row's (uniform branch)
    lo = min(lo, m ? m : 0xFFFFFFFFu);
  }
  uint32_t tau = wave_min_u32(lo);
  if ((E + 7) / 8 < K) tau = 1u;
  // the candidates' composites over the keys (which are in registers now)
  uint64_t *cand = reinterpret_cast<uint64_t *>(row);
  if (lane < 32) cand[lane] = 0ull;   // zero (below every candidate) past a short list's end
  int n = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (64 * i >= E) break;   // uniform
    const bool c = k[i] >= tau;
    const unsigned long long b = __ballot(c);
    const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
    if (c) cand[pos] = ((uint64_t)k[i] << 32) | (uint64_t)(~(uint32_t)(lane + 64 * i));
    n += __popcll(b);
  }
  // rank of each candidate: the larger composites of the list. Up to 32
  // candidates, two lanes share one, each comparing every other pair of the
  // first 32 entries (zero past the list's end), all its reads in flight at
  // once; beyond 32, one lane per candidate.
  const uint4 *cand2 = reinterpret_cast<const uint4 *>(cand);
  int r = K;
  uint64_t my = 0;
  if (n <= 32) {   // uniform
    const int half = lane & 1, ci = lane >> 1;
    my = cand[ci < n ? ci : 0];
    uint4 two[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) two[j] = cand2[half + 2 * j];
    int c = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c += (((uint64_t)two[j].y << 32) | two[j].x) > my;
      c += (((uint64_t)two[j].w << 32) | two[j].z) > my;
    }
    c += __shfl_xor(c, 1);
    if (half == 0 && ci < n) r = c;
  } else {
    for (int ci = lane; ci < n; ci += 64) {
      const uint64_t m = cand[ci];
      int c = 0;
      for (int q = 0; q < n; q += 2) {
        const uint4 two = cand2[q >> 1];
        c += (((uint64_t)two.y << 32) | two.x) > m;
        c += q + 1 < n && (((uint64_t)two.w << 32) | two.z) > m;
      }
      if (c < K) {
        const int e = (int)~(uint32_t)m;
        rl.sid[t][c] = e;
        rl.skey[t][c] = (uint32_t)(m >> 32);
        rl.pkey[t * K + c] = e * QMV_MOE_MAX_TOKENS + t;
      }
    }
  }
  if (r < K) {
    const int e = (int)~(uint32_t)my;
    rl.sid[t][r] = e;
    rl.skey[t][r] = (uint32_t)(my >> 32);
    rl.pkey[t * K + r] = e * QMV_MOE_MAX_TOKENS + t;
  }
}

// Weight j of token t: the softmax over the token's K chosen logits, exp(l_q -
// l_0) summed in rank order, as route_token computes it.
__device__ __forceinline__ float route_weight(const uint32_t (*skey)[kTopK], const int t, const int j, const int K) {
  const float l0 = key_logit(skey[t][0]);
  float sum = 0.0f, mine = 0.0f;
#pragma unroll
  for (int q = 0; q < kTopK; ++q) {
    if (q < K) {
      const float ex = expf(key_logit(skey[t][q]) - l0);
      sum += ex;
      if (q == j) mine = ex;
    }
  }
  return mine / sum;
}

// The T*K (expert, token) pairs, sorted by expert then token, computed by one
// wave from the routing in LDS (sorted_pairs). Lane p < P holds pair p in
// routing order (token p / K, rank p % K); lane r < P holds the r-th pair of
// the sorted order.
struct SortedPairs {
  int key;                   // expert * 4 + token of this lane's pair in routing order (INT_MAX past P)
  float wgt;                 // its routing weight
  int rank;                  // gather-list position of this lane's pair
  int skey;                  // sorted order
  float sw;
  unsigned long long heads;  // sorted positions that start a new expert
};

// Lane p < P: pair p's key (routing order) and its position in the sorted
// order, by counting the smaller keys (read from LDS four at a time); lanes
// past P keep their own index, completing the permutation.
struct PairRank {
  int key, rank;
};
template <int T>
__device__ __forceinline__ PairRank pair_ranks(const RouteLds &rl, const int P) {
  constexpr int kP = T * kTopK;   // P <= kP; the keys past P are INT_MAX
  const int lane = threadIdx.x & 63;
  PairRank r;
  r.key = lane < P ? rl.pkey[lane] : INT_MAX;
  int rank = 0;
  const int4 *pk = reinterpret_cast<const int4 *>(rl.pkey);
  int4 v[kP / 4];
#pragma unroll
  for (int q4 = 0; q4 < kP / 4; ++q4) v[q4] = pk[q4];   // all in flight at once
#pragma unroll
  for (int q4 = 0; q4 < kP / 4; ++q4)
    rank += (v[q4].x < r.key) + (v[q4].y < r.key) + (v[q4].z < r.key) + (v[q4].w < r.key);
  r.rank = lane < P ? rank : lane;
  return r;
}

// The sorted pairs (the weights left at zero: with_weights adds them).
__device__ __forceinline__ SortedPairs sorted_pairs(const PairRank &pr, const int P) {
  const int lane = threadIdx.x & 63;
  SortedPairs s;
  s.key = pr.key;
  s.wgt = 0.0f;
  s.rank = pr.rank;
  s.skey = __builtin_amdgcn_ds_permute(pr.rank * 4, pr.key);
  s.sw = 0.0f;
  const int se = s.skey / QMV_MOE_MAX_TOKENS;
  const int prev = __shfl(se, (lane + 63) & 63);
  s.heads = __ballot(lane < P && (lane == 0 || se != prev));
  return s;
}

// The routing weights of the sorted pairs (routing order and sorted order).
__device__ __forceinline__ SortedPairs with_weights(SortedPairs s, const RouteLds &rl, const int P, const int K) {
  const int lane = threadIdx.x & 63;
  if (lane < P) {
    const int t = lane / K, j = lane - t * K;
    s.wgt = route_weight(rl.skey, t, j, K);
  }
  s.sw = __builtin_bit_cast(float, __builtin_amdgcn_ds_permute(s.rank * 4, __builtin_bit_cast(int, s.wgt)));
  return s;
}


// Distinct expert `slot` (ascending) of the sorted pairs: its id, first sorted
// position and token count, and its tokens in ascending order. p0 < 0 when
// fewer experts were chosen. All values are wave-uniform.
template <int T>
struct Slot {
  int e, p0, ntok;
  int tok[T];
};

template <int T>
__device__ __forceinline__ Slot<T> find_slot(const SortedPairs &s, const int slot, const int P) {
  const int lane = threadIdx.x & 63;
  const bool head = (s.heads >> lane) & 1ull;
  const int below = __popcll(s.heads & ((1ull << lane) - 1ull));
  const unsigned long long mine = __ballot(head && below == slot);
  Slot<T> r;
  r.p0 = __ffsll((long long)mine) - 1;
  r.e = 0;
  r.ntok = 0;
#pragma unroll
  for (int i = 0; i < T; ++i) r.tok[i] = 0;
  if (r.p0 < 0) return r;
  const unsigned long long after = s.heads & ~((2ull << r.p0) - 1ull);
  const int next = after ? __ffsll((long long)after) - 1 : P;
  r.ntok = next - r.p0;
  r.e = __builtin_amdgcn_readlane(s.skey, r.p0) / QMV_MOE_MAX_TOKENS;
#pragma unroll
  for (int i = 0; i < T; ++i)
    if (i < r.ntok) r.tok[i] = __builtin_amdgcn_readlane(s.skey, r.p0 + i) % QMV_MOE_MAX_TOKENS;
  return r;
}

// With one token every pair has its own expert, so distinct expert `slot` is
// the pair at sorted position `slot` (p0 < 0 when slot >= P).
__device__ __forceinline__ Slot<1> slot_of_rank(const PairRank &pr, const int slot, const int P) {
  const int lane = threadIdx.x & 63;
  Slot<1> r;
  r.p0 = slot < P ? slot : -1;
  r.ntok = slot < P ? 1 : 0;
  r.tok[0] = 0;
  const unsigned long long at = __ballot(lane < P && pr.rank == slot);
  r.e = at ? __builtin_amdgcn_readlane(pr.key, __ffsll((long long)at) - 1) / QMV_MOE_MAX_TOKENS : 0;
  return r;
}

// The workgroup's distinct expert: directly from the ranks with one token,
// else from the sorted pairs.
template <int T>
__device__ __forceinline__ Slot<T> my_slot(const PairRank &pr, const int slot, const int P) {
  if constexpr (T == 1) return slot_of_rank(pr, slot, P);
  else return find_slot<T>(sorted_pairs(pr, P), slot, P);
}

// Routing outputs and the tables of launch 2, written by one wave.
__device__ __forceinline__ void write_routing(const SortedPairs &s, const int P, int32_t *__restrict__ topk_ids,
                                              float *__restrict__ topk_w, int32_t *__restrict__ pairs_out,
                                              Table *__restrict__ tab) {
  const int lane = threadIdx.x & 63;
  const int se = s.skey / QMV_MOE_MAX_TOKENS, st = s.skey % QMV_MOE_MAX_TOKENS;
  if (lane < P) {
    if (topk_ids) topk_ids[lane] = s.key / QMV_MOE_MAX_TOKENS;
    if (topk_w) topk_w[lane] = s.wgt;
    if (pairs_out) {
      pairs_out[2 * lane] = se;
      pairs_out[2 * lane + 1] = st;
    }
    tab->pair_expert[lane] = se;
    tab->pair_token[lane] = st;
    tab->pair_weight[lane] = s.sw;
    tab->rank_pair[lane] = s.rank;
  }
  if ((s.heads >> lane) & 1ull) {
    const int slot = __popcll(s.heads & ((1ull << lane) - 1ull));
    const unsigned long long after = s.heads & ~((2ull << lane) - 1ull);
    const int next = after ? __ffsll((long long)after) - 1 : P;
    tab->slot_expert[slot] = se;
    tab->slot_pair0[slot] = lane;
    tab->slot_ntok[slot] = next - lane;
  }
  if (lane == 0) {
    tab->n_pairs = P;
    tab->n_slots = __popcll(s.heads);
  }
}

}  // namespace moe
}  // namespace qmv
