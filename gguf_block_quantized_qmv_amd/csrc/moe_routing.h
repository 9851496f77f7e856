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

// The T*K (expert, token) pairs, sorted by expert then token, computed by one
// wave from the routing in LDS. Lane p < P holds pair p in routing order
// (token p / K, rank p % K); lane r < P holds the r-th pair of the sorted order.
struct SortedPairs {
  int key;                   // expert * 4 + token of this lane's pair in routing order (INT_MAX past P)
  float wgt;                 // its routing weight
  int rank;                  // gather-list position of this lane's pair
  int skey;                  // sorted order
  float sw;
  unsigned long long heads;  // sorted positions that start a new expert
};

__device__ __forceinline__ SortedPairs sort_pairs(const int (*sid)[kTopK], const float (*swt)[kTopK], const int P,
                                            const int K) {
  const int lane = threadIdx.x & 63;
  SortedPairs s;
  s.key = INT_MAX;
  s.wgt = 0.0f;
  if (lane < P) {
    const int t = lane / K, j = lane - t * K;
    s.key = sid[t][j] * QMV_MOE_MAX_TOKENS + t;
    s.wgt = swt[t][j];
  }
  // keys are distinct (a token picks distinct experts), so ranks 0..P-1 are a
  // permutation; lanes past P keep their own index to complete it
  int rank = 0;
  for (int q = 0; q < P; ++q) rank += __builtin_amdgcn_readlane(s.key, q) < s.key;
  if (lane >= P) rank = lane;
  s.rank = rank;
  s.skey = __builtin_amdgcn_ds_permute(rank * 4, s.key);
  s.sw = __builtin_bit_cast(float, __builtin_amdgcn_ds_permute(rank * 4, __builtin_bit_cast(int, s.wgt)));
  const int se = s.skey / QMV_MOE_MAX_TOKENS;
  const int prev = __shfl(se, (lane + 63) & 63);
  s.heads = __ballot(lane < P && (lane == 0 || se != prev));
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
