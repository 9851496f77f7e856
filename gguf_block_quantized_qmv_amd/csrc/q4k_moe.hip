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
//     Every workgroup's first wave recomputes the routing of the <= 4 tokens
//     (k rounds of a wave-wide argmax over the logits, ties to the lower id)
//     and the gather list: all (expert, token) pairs sorted by expert, then
//     token. The expert ids live in LDS (next to the staged activations).
//     Workgroup (0, 0) also writes the routing outputs and the tables that
//     launch 2 reads. Workgroup (tile, s) then computes, for distinct expert s
//     (ascending id) and the tokens that chose it, 16 rows of W_gate x and
//     W_up x with the dense GEMV's per-chunk arithmetic (x staged in LDS) and
//     stores h = silu(g) * u in fp32 for each (expert, token) pair.
//  2. moe_down_kernel, grid H/16 row tiles. Each workgroup stages every pair's
//     h in LDS, walks the distinct experts in ascending id, streams 16 rows of
//     that expert's W_down once for all of its tokens, and accumulates
//     y_t += r_(t,e) * (W_down[e] h_(e,t)) per token in that fixed order.
//
// Each selected expert's weights are read once per call. A token's result is
// bit-identical whatever other tokens share the call: its experts are visited
// in the same ascending order and every token slot runs the same instructions.
#include <limits.h>

#include "q4k_common.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerWave = 64 / kLanesPerRow;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr int kMaxPairs = QMV_MOE_MAX_TOKENS * QMV_MOE_MAX_TOP_K;
constexpr size_t kTableBytes = 4096;  // routing tables at the start of the workspace

struct Routing {
  int n_pairs;
  int n_slots;
  int slot_expert[kMaxPairs];  // distinct experts, ascending
  int slot_pair0[kMaxPairs];   // first gather-list position of each distinct expert
  int slot_ntok[kMaxPairs];    // number of tokens that chose it
  int pair_expert[kMaxPairs];  // gather list: sorted by expert, then token
  int pair_token[kMaxPairs];
  float pair_weight[kMaxPairs];
  int sel_id[QMV_MOE_MAX_TOKENS][QMV_MOE_MAX_TOP_K];  // per token, rank order
  float sel_w[QMV_MOE_MAX_TOKENS][QMV_MOE_MAX_TOP_K];
};
static_assert(sizeof(Routing) <= kTableBytes, "routing tables exceed their workspace slot");
static_assert(sizeof(Routing) % 4 == 0, "routing tables are copied as words");

// Wave 0: top-k selection and renormalised weights for every token.
__device__ __forceinline__ void route_tokens(const float *__restrict__ logits, const int T, const int E, const int K, Routing *R) {
  const int lane = threadIdx.x;
  for (int t = 0; t < T; ++t) {
    float v[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      live[i] = e < E;
      v[i] = live[i] ? logits[(size_t)t * E + e] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < QMV_MOE_MAX_TOP_K; ++j) {
      if (j >= K) break;
      // this lane's best remaining candidate (ids ascend with i, so '>' keeps the lower id on ties)
      float bv = 0.0f;
      int bid = INT_MAX;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (live[i] && (bid == INT_MAX || v[i] > bv)) {
          bv = v[i];
          bid = lane + 64 * i;
        }
      // wave-wide argmax: larger logit wins, equal logits go to the lower id
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oid = __shfl_xor(bid, off);
        if (oid != INT_MAX && (bid == INT_MAX || ov > bv || (ov == bv && oid < bid))) {
          bv = ov;
          bid = oid;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == bid) live[i] = false;
      if (lane == 0) {
        R->sel_id[t][j] = bid;
        R->sel_w[t][j] = bv;  // the selected logit, turned into a weight below
      }
    }
    if (lane == 0) {
      // softmax over the selected logits, largest first: exp(l_j - l_0) / sum in rank order
      const float l0 = R->sel_w[t][0];
      float sum = 0.0f;
      for (int j = 0; j < K; ++j) {
        const float ex = expf(R->sel_w[t][j] - l0);
        R->sel_w[t][j] = ex;
        sum += ex;
      }
      for (int j = 0; j < K; ++j) R->sel_w[t][j] = R->sel_w[t][j] / sum;
    }
  }
}

// Wave 0, after route_tokens is visible: the sorted gather list and the distinct experts.
__device__ __forceinline__ void build_gather_list(const int T, const int K, Routing *R) {
  const int lane = threadIdx.x;
  const int P = T * K;
  if (lane < P) {
    const int t = lane / K, j = lane - t * K;
    const int e = R->sel_id[t][j];
    const int key = e * QMV_MOE_MAX_TOKENS + t;
    int rank = 0;
    for (int q = 0; q < P; ++q) {
      const int tq = q / K;
      rank += (R->sel_id[tq][q - tq * K] * QMV_MOE_MAX_TOKENS + tq) < key;
    }
    R->pair_expert[rank] = e;
    R->pair_token[rank] = t;
    R->pair_weight[rank] = R->sel_w[t][j];
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  const bool head = lane < P && (lane == 0 || R->pair_expert[lane] != R->pair_expert[lane - 1]);
  const unsigned long long mask = __ballot(head);
  if (head) {
    const int slot = __popcll(mask & ((1ull << lane) - 1ull));
    const unsigned long long later = (lane == 63) ? 0ull : (mask >> (lane + 1));
    const int next = later ? lane + 1 + __ffsll((long long)later) - 1 : P;
    R->slot_expert[slot] = R->pair_expert[lane];
    R->slot_pair0[slot] = lane;
    R->slot_ntok[slot] = next - lane;
  }
  if (lane == 0) {
    R->n_pairs = P;
    R->n_slots = __popcll(mask);
  }
}

template <int T>
__global__ __launch_bounds__(kThreads) void moe_gate_up_kernel(
    const uint8_t *__restrict__ w_gate, const uint8_t *__restrict__ w_up, const float *__restrict__ logits,
    const uint16_t *__restrict__ x, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ pairs_out, uint8_t *__restrict__ ws, const int hidden, const int ffn, const int E,
    const int K) {
  __shared__ Routing R;
  extern __shared__ uint4 lds[];
  if (threadIdx.x < 64) route_tokens(logits, T, E, K, &R);
  __syncthreads();
  if (threadIdx.x < 64) build_gather_list(T, K, &R);
  __syncthreads();

  if (blockIdx.x == 0 && blockIdx.y == 0) {
    const int P = T * K;
    for (int i = threadIdx.x; i < P; i += kThreads) {
      const int t = i / K, j = i - t * K;
      if (topk_ids) topk_ids[i] = R.sel_id[t][j];
      if (topk_w) topk_w[i] = R.sel_w[t][j];
      if (pairs_out) {
        pairs_out[2 * i] = R.pair_expert[i];
        pairs_out[2 * i + 1] = R.pair_token[i];
      }
    }
    const int *src = reinterpret_cast<const int *>(&R);
    int *dst = reinterpret_cast<int *>(ws);
    for (int i = threadIdx.x; i < (int)(sizeof(Routing) / 4); i += kThreads) dst[i] = src[i];
  }

  const int slot = blockIdx.y;
  if (slot >= R.n_slots) return;  // fewer distinct experts than the grid allows for
  const int e = R.slot_expert[slot], p0 = R.slot_pair0[slot], ntok = R.slot_ntok[slot];
  const int gpr = hidden >> 3, nsub = hidden >> 5;
  uint4 *xs = lds;
  float *xsum = reinterpret_cast<float *>(lds + T * gpr);
  for (int i = 0; i < ntok; ++i)
    stage_bf16_row(x + (size_t)R.pair_token[p0 + i] * hidden, xs + i * gpr, xsum + i * nsub, gpr, nsub, threadIdx.x,
                   kThreads);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);
  const int f = (blockIdx.x * kWaves + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanesPerRow;
  if (f >= ffn) return;
  const int c = j & 3;
  const ScaleSel sel = scale_selectors(c);
  const int nblk = hidden >> 8;
  const size_t row_bytes = (size_t)nblk * kQ4KBlockBytes;
  const size_t expert_bytes = (size_t)ffn * row_bytes;
  const uint8_t *grow = w_gate + (size_t)e * expert_bytes + (size_t)f * row_bytes;
  const uint8_t *urow = w_up + (size_t)e * expert_bytes + (size_t)f * row_bytes;
  const int nsteps = (nblk + 3) >> 2;

  float acc_g[T], acc_u[T];
#pragma unroll
  for (int r = 0; r < T; ++r) acc_g[r] = acc_u[r] = 0.0f;

  constexpr int D = 2;
  for (int s0 = 0; s0 < nsteps; s0 += D) {
    uint4 gh[D], ga[D], gb[D], uh[D], ua[D], ub[D];
    bool ok[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int b = (s0 + u) * 4 + (j >> 2);
      ok[u] = b < nblk;
      if (ok[u]) {
        const uint8_t *gp = grow + (size_t)b * kQ4KBlockBytes;
        const uint8_t *up = urow + (size_t)b * kQ4KBlockBytes;
        gh[u] = *reinterpret_cast<const uint4 *>(gp);
        ga[u] = *reinterpret_cast<const uint4 *>(gp + 16 + 32 * c);
        gb[u] = *reinterpret_cast<const uint4 *>(gp + 32 + 32 * c);
        uh[u] = *reinterpret_cast<const uint4 *>(up);
        ua[u] = *reinterpret_cast<const uint4 *>(up + 16 + 32 * c);
        ub[u] = *reinterpret_cast<const uint4 *>(up + 32 + 32 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
      if (ok[u]) {
        const int ci = (s0 + u) * 16 + j;
        q4k_chunk_bf16<T>(acc_g, ntok, gh[u], ga[u], gb[u], ci, sel, xs, xsum, gpr, nsub);
        q4k_chunk_bf16<T>(acc_u, ntok, uh[u], ua[u], ub[u], ci, sel, xs, xsum, gpr, nsub);
      }
  }

  float *h = reinterpret_cast<float *>(ws + kTableBytes);
#pragma unroll
  for (int r = 0; r < T; ++r) {
    if (r >= ntok) break;
    const float g = row16_sum(acc_g[r]);
    const float u = row16_sum(acc_u[r]);
    if (j == r) h[(size_t)(p0 + r) * ffn + f] = g / (1.0f + expf(-g)) * u;
  }
}

template <int T>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(const uint8_t *__restrict__ w_down,
                                                            const uint8_t *__restrict__ ws, float *__restrict__ y,
                                                            const int hidden, const int ffn) {
  __shared__ Routing R;
  extern __shared__ uint4 lds[];
  {
    const int *src = reinterpret_cast<const int *>(ws);
    int *dst = reinterpret_cast<int *>(&R);
    for (int i = threadIdx.x; i < (int)(sizeof(Routing) / 4); i += kThreads) dst[i] = src[i];
  }
  __syncthreads();
  const int P = R.n_pairs, n_slots = R.n_slots;
  const int gpr = ffn >> 2, nsub = ffn >> 5;
  uint4 *hs = lds;
  float *hsum = reinterpret_cast<float *>(lds + (size_t)P * gpr);
  const float *h = reinterpret_cast<const float *>(ws + kTableBytes);
  for (int p = 0; p < P; ++p)
    stage_f32_row(h + (size_t)p * ffn, hs + p * gpr, hsum + p * nsub, gpr, nsub, threadIdx.x, kThreads);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);
  const int n = (blockIdx.x * kWaves + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanesPerRow;
  if (n >= hidden) return;
  const int c = j & 3;
  const ScaleSel sel = scale_selectors(c);
  const int nblk = ffn >> 8;
  const size_t row_bytes = (size_t)nblk * kQ4KBlockBytes;
  const size_t expert_bytes = (size_t)hidden * row_bytes;
  const int nsteps = (nblk + 3) >> 2;

  float acc_y[T];
#pragma unroll
  for (int r = 0; r < T; ++r) acc_y[r] = 0.0f;

  constexpr int D = 4;  // distinct experts whose rows are loaded together
  for (int s0 = 0; s0 < n_slots; s0 += D) {
    float acc_z[D][T];
#pragma unroll
    for (int u = 0; u < D; ++u)
#pragma unroll
      for (int r = 0; r < T; ++r) acc_z[u][r] = 0.0f;
    for (int st = 0; st < nsteps; ++st) {
      const int b = st * 4 + (j >> 2);
      uint4 hh[D], qa[D], qb[D];
      bool ok[D];
#pragma unroll
      for (int u = 0; u < D; ++u) {
        ok[u] = (s0 + u < n_slots) && b < nblk;
        if (ok[u]) {
          const uint8_t *bp = w_down + (size_t)R.slot_expert[s0 + u] * expert_bytes + (size_t)n * row_bytes +
                              (size_t)b * kQ4KBlockBytes;
          hh[u] = *reinterpret_cast<const uint4 *>(bp);
          qa[u] = *reinterpret_cast<const uint4 *>(bp + 16 + 32 * c);
          qb[u] = *reinterpret_cast<const uint4 *>(bp + 32 + 32 * c);
        }
      }
#pragma unroll
      for (int u = 0; u < D; ++u)
        if (ok[u]) {
          const int p0 = R.slot_pair0[s0 + u];
          q4k_chunk_f32<T>(acc_z[u], R.slot_ntok[s0 + u], hh[u], qa[u], qb[u], st * 16 + j, sel, hs + p0 * gpr,
                           hsum + p0 * nsub, gpr, nsub);
        }
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (s0 + u >= n_slots) break;
      const int p0 = R.slot_pair0[s0 + u], ntok = R.slot_ntok[s0 + u];
#pragma unroll
      for (int r = 0; r < T; ++r) {
        if (r >= ntok) break;
        const float z = row16_sum(acc_z[u][r]);
        const int t = R.pair_token[p0 + r];
        const float wgt = R.pair_weight[p0 + r];
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
          if (tt == t) acc_y[tt] = __builtin_fmaf(wgt, z, acc_y[tt]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
    if (j == tt) y[(size_t)tt * hidden + n] = acc_y[tt];
}

size_t gate_up_lds(int t, int hidden) { return (size_t)t * ((size_t)(hidden >> 3) * 16 + (size_t)(hidden >> 5) * 4); }
size_t down_lds(int pairs, int ffn) { return (size_t)pairs * ((size_t)(ffn >> 2) * 16 + (size_t)(ffn >> 5) * 4); }

template <int T>
int launch_t(const void *w_gate, const void *w_up, const void *w_down, const float *logits, const uint16_t *x,
             float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int hidden, int ffn,
             int n_experts, int top_k, hipStream_t s) {
  static std::atomic<size_t> granted_a{0}, granted_b{0};
  const size_t lds_a = gate_up_lds(T, hidden), lds_b = down_lds(T * top_k, ffn);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&moe_gate_up_kernel<T>), lds_a, granted_a,
                        "moe_gate_up_kernel lds") ||
      allow_dynamic_lds(reinterpret_cast<const void *>(&moe_down_kernel<T>), lds_b, granted_b, "moe_down_kernel lds"))
    return QMV_ERR_HIP;
  const int max_slots = n_experts < T * top_k ? n_experts : T * top_k;
  const dim3 grid_a((unsigned)((ffn + kRowsPerGroup - 1) / kRowsPerGroup), (unsigned)max_slots);
  int rc = launch_kernel("moe_gate_up_kernel", moe_gate_up_kernel<T>, grid_a, dim3(kThreads), lds_a, s, w_gate, w_up,
                         logits, x, topk_ids, topk_w, pairs, ws, hidden, ffn, n_experts, top_k);
  if (rc) return rc;
  const dim3 grid_b((unsigned)((hidden + kRowsPerGroup - 1) / kRowsPerGroup));
  return launch_kernel("moe_down_kernel", moe_down_kernel<T>, grid_b, dim3(kThreads), lds_b, s, w_down, ws, y,
                       hidden, ffn);
}

}  // namespace

size_t moe_workspace_bytes(int t, int hidden, int ffn, int n_experts, int top_k) {
  (void)hidden;
  (void)n_experts;
  return kTableBytes + (size_t)t * (size_t)top_k * (size_t)ffn * sizeof(float);
}

bool moe_fits_lds(int t, int hidden, int ffn, int top_k) {
  const size_t budget = (size_t)QMV_LDS_X_BYTES - sizeof(Routing);
  return gate_up_lds(t, hidden) <= budget && down_lds(t * top_k, ffn) <= budget;
}

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

}  // namespace qmv
