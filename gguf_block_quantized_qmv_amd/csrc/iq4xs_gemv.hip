// IQ4_XS matrix times 1..4 bf16 activation rows, gfx950.
//
// The memra README's model support table ships its 35B-A3B MoE in IQ4_XS (the
// memra-bench card's Drafts section carries a UD-IQ4_XS draft of it). The pages
// print no layout; the one read here is the public GGUF format. A 136-byte
// super-block holds 256 weights along K:
//   bytes 0..1   fp16 d
//   bytes 2..3   H: bits 2j..2j+1 are bits 4..5 of the 6-bit scale ls_j
//   bytes 4..7   L: bits 4j..4j+3 of this little-endian word are bits 0..3 of ls_j
//   bytes 8..135 grid indices: sub-block j (32 weights) owns 16 bytes; byte i of
//                them holds weight 32j + i (low nibble) and 32j + 16 + i (high)
// and weight = d * (ls_j - 32) * grid[index] with a fixed 16-value grid.
//
// The grid is non-linear, so a nibble cannot be converted arithmetically. The
// kernel keeps a 256-entry LDS table indexed by a whole index byte: entry e is
// the bf16 pair (grid[e & 15], grid[e >> 4]) -- the weights i and 16 + i of a
// sub-block (exact: the grid values are integers below 2^8). The activations
// are staged in LDS pair-interleaved to match, (x[i], x[16 + i]) for i < 16 of
// every 32-value sub-block, so each table entry meets its activation pair in
// one v_dot2_f32_bf16. Per 32 weights a lane spends 16 table reads, 16 dot2
// per activation row and the scale decode; the sub-block sum is scaled by
// d * (ls - 32), which is exact in fp32, and accumulated in fp32.
//
// Work mapping: G lanes per W row (16, or 32 for long rows), T / G rows per
// workgroup of T threads; lane l of a row takes the row's sub-blocks l, l + G,
// ... Loads run kDepth units ahead through a register ring; they are
// unconditional (units past the row re-read the row's first sub-block with a
// zero scale) and the unit loop is unrolled by kDepth, so every wait is exact.
// Row r of the output is computed by the same instruction sequence for every M.
#include "iq4xs_common.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

using namespace iq4xs;

constexpr int kDepth = addr::kIq4GemvDepth;   // units of loads in flight per lane

constexpr int kStageSub = 2;   // sub-blocks per thread per staging round trip
static_assert(layout::kIq4xsTableBytes == (size_t)kTableEntries * 4, "the table's LDS bytes");

// Stage sub-block s of activation row r, pair-interleaved, at xs[r * rg + x_slot(s)].
__device__ __forceinline__ void stage_one(const uint4 *__restrict__ xg, uint4 *__restrict__ xs, const int t,
                                          const int nsub, const int k, const int rg) {
  const int r = t / nsub, s = t - r * nsub;
  const uint4 *src = xg + (size_t)r * (k >> 3) + 4 * s;
  uint4 o[4];
  interleave(src[0], src[1], src[2], src[3], o);
#pragma unroll
  for (int q = 0; q < 4; ++q) xs[r * rg + x_slot(s) + q] = o[q];
}

// All M * nsub sub-blocks of the activations, kStageSub per thread per round
// trip; only the last round is partial (each staged sub-block is read once).
template <int M, int T>
__device__ __forceinline__ void stage_activations(const uint4 *__restrict__ xg, uint4 *__restrict__ xs,
                                                  const int tid, const int nsub, const int k, const int rg) {
  const int total = M * nsub;
  int base = 0;
  for (; base + kStageSub * T <= total; base += kStageSub * T) {
    uint4 g[kStageSub][4];
#pragma unroll
    for (int i = 0; i < kStageSub; ++i) {
      const int t = base + tid + i * T, r = t / nsub, s = t - r * nsub;
#pragma unroll
      for (int q = 0; q < 4; ++q) g[i][q] = xg[(size_t)r * (k >> 3) + 4 * s + q];
    }
#pragma unroll
    for (int i = 0; i < kStageSub; ++i) {
      const int t = base + tid + i * T, r = t / nsub, s = t - r * nsub;
      uint4 o[4];
      interleave(g[i][0], g[i][1], g[i][2], g[i][3], o);
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[r * rg + x_slot(s) + q] = o[q];
    }
  }
  for (int t = base + tid; t < total; t += T) stage_one(xg, xs, t, nsub, k, rg);
}

template <int M, int G, int T>
__global__ __launch_bounds__(T) void iq4xs_gemv_kernel(const uint8_t *__restrict__ w,
                                                       const uint16_t *__restrict__ x,
                                                       float *__restrict__ y, const int n, const int k) {
  static_assert(G % 8 == 0, "a lane's sub-block index inside the super-block must stay fixed");
  // the table is static LDS, so its address is a compile-time constant and the
  // scaled index byte is the whole read address
  __shared__ uint32_t tbl[kTableEntries];
  extern __shared__ uint4 xs[];
  const uint8_t *tbl_bytes = reinterpret_cast<const uint8_t *>(tbl);
  const int tid = threadIdx.x;
  const int nblk = k >> 8, nsub = nblk * 8, rg = row_granules(nsub);
  const int row = addr::lane_row(blockIdx.x, tid, T, G);
  const int l = tid % G;
  // Lane l takes sub-blocks u = l + G t: super-block (l >> 3) + (G / 8) t, sub-block j = l & 7.
  const addr::Iq4Lane ln = addr::iq4_lane(G, nblk, (size_t)(row < n ? row : 0), l);
  const int j = l & 7, qoff = ln.qoff;
  const uint8_t *row_ptr = w + ln.row_base, *lane_ptr = w + ln.lane_base;
  const int nlive = ln.nlive;                                   // live units of this lane
  const int nslots = addr::iq4_slots(G, nblk, kDepth);
  auto unit_ptr = [&](const int t) -> const uint8_t * {
    return t < nlive ? lane_ptr + addr::iq4_unit_offset(t, ln.unit_bytes) : row_ptr;
  };
  // activation granule of unit t: x_slot(l + G t) = x_slot(l) + t * (4 G + G / 4)
  constexpr int kXStride = 4 * G + G / 4;
  const int x_l = x_slot(l < nsub ? l : 0);

  // the first weights are requested before anything else; a unit past the
  // lane's last re-reads sub-block j of the row's first super-block
  Unit ring[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    load_unit(unit_ptr(d), qoff, ring[d]);

  // table and activations
  if (tid < kTableEntries) tbl[tid] = grid_bf16((uint32_t)tid & 15u) | (grid_bf16((uint32_t)tid >> 4) << 16);
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  stage_activations<M, T>(xg, xs, tid, nsub, k, rg);
  __syncthreads();

  const int sh_lo = 4 * j, sh_hi = 16 + 2 * j;
  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;
  for (int t0 = 0; t0 < nslots; t0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int t = t0 + d;
      const bool live = t < nlive;
      const Unit &cur = ring[d];
      // the slot's data is consumed (scale decoded, table reads issued) before
      // the slot is refilled, so the refill can land in the same registers
      const float dl_raw = sub_scale(cur.hdr, sh_lo, sh_hi);
      const float dl = live ? dl_raw : 0.0f;
      const int xg0 = live ? x_l + t * kXStride : x_l;
      const Pairs p0 = word_pairs(tbl_bytes, cur.q0.x), p1 = word_pairs(tbl_bytes, cur.q0.y);
      const Pairs p2 = word_pairs(tbl_bytes, cur.q1.x), p3 = word_pairs(tbl_bytes, cur.q1.y);
      // refill the slot kDepth units ahead (clamped, never guarded)
      {
        const int tn = t + kDepth;
        load_unit(unit_ptr(tn), qoff, ring[d]);
      }
#pragma unroll
      for (int r = 0; r < M; ++r) {
        const uint4 *xp = xs + r * rg + xg0;
        float s0 = pairs_dot(p0, xp[0], 0.0f);
        float s1 = pairs_dot(p1, xp[1], 0.0f);
        s0 = pairs_dot(p2, xp[2], s0);
        s1 = pairs_dot(p3, xp[3], s1);
        acc[r] = __builtin_fmaf(dl, s0 + s1, acc[r]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float v = group_sum<G>(acc[r]);
    if (l == r && row < n) y[(size_t)r * n + row] = v;
  }
}

// Dequantization export: one thread per (row, sub-block), 32 fp32 weights, each
// d * (ls - 32) * grid[index] -- exact in fp32 (11 + 6 + 7 significant bits).
__global__ __launch_bounds__(256) void iq4xs_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                             const size_t nsub_total) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nsub_total) return;
  const size_t b = t >> 3;
  const int j = (int)(t & 7);
  const uint8_t *bp = w + b * kIQ4XSBlockBytes;
  const uint2 hdr = *reinterpret_cast<const uint2 *>(bp);
  const float dl = sub_scale(hdr, 4 * j, 16 + 2 * j);
  const uint2 q0 = *reinterpret_cast<const uint2 *>(bp + 8 + 16 * j);
  const uint2 q1 = *reinterpret_cast<const uint2 *>(bp + 16 + 16 * j);
  const uint32_t qw[4] = {q0.x, q0.y, q1.x, q1.y};
  float4 *o = reinterpret_cast<float4 *>(out + t * 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {      // h = 0: low nibbles (weights 0..15), 1: high (16..31)
#pragma unroll
    for (int wq = 0; wq < 4; ++wq) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t idx = (qw[wq] >> (8 * e + 4 * h)) & 15u;
        v[e] = dl * __builtin_bit_cast(float, grid_bf16(idx) << 16);
      }
      o[4 * h + wq] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}


template <int M, int G, int T>
int launch_mgt(const addr::Iq4Plan &p, const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t s) {
  static LdsGrant granted;
  const size_t lds = layout::iq4xs_gemv_dyn_lds(M, k);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&iq4xs_gemv_kernel<M, G, T>), lds, granted,
                        "iq4xs_gemv_kernel lds"))
    return QMV_ERR_HIP;
  return launch_kernel("iq4xs_gemv_kernel", iq4xs_gemv_kernel<M, G, T>, dim3(p.grid), dim3(T), lds, s,
                       static_cast<const uint8_t *>(w), x, y, n, k);
}

// The plan is addr::iq4_gemv_plan: long rows take 32 lanes (more independent
// loads per row, fewer rows per workgroup); once the staged activations leave
// room for a single workgroup per CU, that workgroup takes 512 threads, so a
// CU still holds 8 waves.
template <int M>
int launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t s) {
  const addr::Iq4Plan p = addr::iq4_gemv_plan(M, n, k);
  if (p.G == 16) return launch_mgt<M, 16, 256>(p, w, x, y, n, k, s);
  if (p.threads == 512) return launch_mgt<M, 32, 512>(p, w, x, y, n, k, s);
  return launch_mgt<M, 32, 256>(p, w, x, y, n, k, s);
}

}  // namespace

int launch_iq4_xs_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1>(w, x, y, n, k, s);
    case 2: return launch_m<2>(w, x, y, n, k, s);
    case 3: return launch_m<3>(w, x, y, n, k, s);
    case 4: return launch_m<4>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_dequant_iq4_xs(const void *w, float *out, int n, int k, void *stream) {
  const size_t nsub = (size_t)n * (size_t)(k >> 8) * 8;
  return launch_kernel("iq4xs_dequant_kernel", iq4xs_dequant_kernel, dim3((unsigned)((nsub + 255) / 256)), dim3(256),
                       0, static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(w), out, nsub);
}

}  // namespace qmv
