// Q6_K matrix x bf16 activation rows (decode M = 1, verify M = 2..4) and Q6_K
// dequantization, gfx950.
//
// Q6_K super-block (210 bytes, 256 weights; public GGUF layout): L[0..127] low
// four bits of the quants, H[0..63] their top two bits, S[0..15] int8 scales,
// fp16 d. Weight 128h + 32c + l (half h, quarter c, l < 32) takes its low bits
// from L[64h + 32(c & 1) + l] (low nibble for c < 2, high nibble for c >= 2),
// its top bits from bits 2c, 2c + 1 of H[32h + l] and its scale from
// S[8h + 2c + l / 16]; q = low + 16 high - 32 and w = d * sc * q.
//
// Work unit. A lane handles 64 weights per step: unit (h, p) of a block, the
// positions l in [16p, 16p + 16) of half h in all four quarters. Its quant bytes
// are three 16-byte runs, L[64h + 16p ..], L[64h + 32 + 16p ..] and
// H[32h + 16p ..], and its four scales are S[8h + 2c + p]. Four lanes cover a
// block; G lanes (16 up to K = 8192, 32 beyond) own one output row and step
// G/4 blocks at a time.
//
// Alignment. 210 = 2 mod 4, so a block starts 0 or 2 bytes into a dword. A
// step moves an even number of blocks, so the offset is fixed per lane: every
// run is read as the dword-aligned window around it (a 16-byte load plus one
// dword) and realigned by v_alignbit with a per-lane shift of 0 or 16 bits.
// Every address read lies inside the lane's own block (the window of a block
// that starts 2 bytes into its dword begins 2 bytes before it, inside the
// previous block), except that a block's last dword is read only when it starts
// mid-dword, and d is read as a 16-bit load.
//
// Arithmetic. q' = q + 32 in [0, 63] enters v_dot2 as the exact bf16 value
// 128 + q' (bits 0x43 | q', one byte permute per pair), so per 16-weight group
// S' = sum (q + 160) x, and the group adds (d sc) (S' - 160 X) with X the
// group's activation sum, staged once per workgroup. d sc is exact in fp32,
// the products inside dot2 are exact, and the sums are fp32.
//
// LDS. The activations sit in 16-byte granules with granule g of a row at slot
// g ^ (((g >> 4) & 1) | ((g >> 3) & 12)): the 16 lanes of a half-wave (four
// blocks x two halves x two p) then read 16 distinct bank groups for every
// (quarter, granule) they load, with no padding, so M = 4 still fits K = 17408.
// The K/16 group sums follow, the four sums of a unit stored next to each other.
//
// Batch invariance: row r of the output runs the same instruction sequence for
// every M and workgroup shape, so an M = 2..4 call is bit-identical per row to
// M = 1.
#include "qmv_addr.h"
#include "qmv_device.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

constexpr int kQ6KBlockBytes = addr::kQ6KBytes;
constexpr int kMaxThreads = addr::q6_max_threads(1);      // M = 1
constexpr int kMaxThreadsRows = addr::q6_max_threads(2);  // M = 2..4: 20 rows of 32 lanes, one workgroup per CU at K = 17408

// LDS slot of activation granule g of a staged row (see the header comment).
__host__ __device__ constexpr int q6_slot(int g) { return g ^ (((g >> 4) & 1) | ((g >> 3) & 12)); }

// Position of the sum of 16-weight group g (g = 16 b + 8 h + 2 c + p) in the
// row's sum table: 16 b + 8 h + 4 p + c, so a unit's four sums are adjacent.
__device__ __forceinline__ int q6_sum_pos(int g) { return (g & ~7) | ((g & 1) << 2) | ((g >> 1) & 3); }

template <int M>
__host__ __device__ constexpr size_t q6_lds_bytes(int k) {
  return (size_t)M * (size_t)k * 2 + (size_t)M * (size_t)(k >> 4) * 4;
}

// The raw words of one unit: three 20-byte windows (quant runs), the 12-byte
// window around the half's eight scales, and d.
struct Q6Raw {
  uint32_t a[5], b[5], c[5], s[3], d;
};

// bp: the block's first byte; sb: 0 or 2, the block's offset into its dword.
// The reads are the windows of addr::q6_window: the dword-aligned windows
// around the three quant runs and the scales, and d.
__device__ __forceinline__ void q6_load(const uint8_t *__restrict__ bp, const int sb, const int h, const int p,
                                        Q6Raw &r) {
  const uint8_t *a = bp - sb;
  const uint32_t *pa =
      reinterpret_cast<const uint32_t *>(a + addr::q6_run_base(0) + addr::q6_run_h(h, 0) + addr::q6_run_p(p, 0));
  const uint32_t *pc =
      reinterpret_cast<const uint32_t *>(a + addr::q6_run_base(2) + addr::q6_run_h(h, 2) + addr::q6_run_p(p, 2));
  const uint32_t *ps =
      reinterpret_cast<const uint32_t *>(a + addr::q6_run_base(3) + addr::q6_run_h(h, 3) + addr::q6_run_p(p, 3));
  const int b_dw = (addr::q6_run(sb, h, p, 1) - addr::q6_run(sb, h, p, 0)) / 4;   // 8
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    r.a[i] = pa[i];
    r.b[i] = pa[b_dw + i];
    r.c[i] = pc[i];
  }
  r.s[0] = ps[0];
  r.s[1] = ps[1];
  r.s[2] = ps[(addr::q6_run(sb, h, p, 4) - addr::q6_run(sb, h, p, 3)) / 4];
  r.d = *reinterpret_cast<const uint16_t *>(bp + addr::q6_window(sb, h, p, 5).off);
}

// The four 6-bit quants (as q' = q + 32, one per byte) of dword i of quarter c.
__device__ __forceinline__ void q6_quants(const uint32_t a, const uint32_t b, const uint32_t h, uint32_t (&q)[4]) {
  q[0] = (a & 0x0F0F0F0Fu) | ((h << 4) & 0x30303030u);
  q[1] = (b & 0x0F0F0F0Fu) | ((h << 2) & 0x30303030u);
  q[2] = ((a >> 4) & 0x0F0F0F0Fu) | (h & 0x30303030u);
  q[3] = ((b >> 4) & 0x0F0F0F0Fu) | ((h >> 2) & 0x30303030u);
}

// bf16 pairs 128 + q' of bytes 0, 1 (lo) or 2, 3 (hi) of a quant word.
__device__ __forceinline__ bf16x2 q6_pair_lo(const uint32_t q) {
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, q, 0x04010400u));
}
__device__ __forceinline__ bf16x2 q6_pair_hi(const uint32_t q) {
  return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(0x43434343u, q, 0x04030402u));
}

// d * sc for the unit's four quarters; ssel picks bytes p, 2 + p, 4 + p, 6 + p
// of the realigned scale window.
__device__ __forceinline__ void q6_scales(const Q6Raw &r, const int shift, const uint32_t ssel, float (&dsc)[4]) {
  const uint32_t lo = __builtin_amdgcn_alignbit(r.s[1], r.s[0], shift);
  const uint32_t hi = __builtin_amdgcn_alignbit(r.s[2], r.s[1], shift);
  const uint32_t sg = __builtin_amdgcn_perm(hi, lo, ssel);
  const float d = fp16_bits_to_f32(r.d);
#pragma unroll
  for (int c = 0; c < 4; ++c) dsc[c] = d * (float)(int32_t)(int8_t)(uint8_t)(sg >> (8 * c));
}

// One unit against M activation rows. xo[c][e]: LDS granule index (relative to
// the unit's row base xr) of granule e of quarter c; xr: the unit's base in
// row 0; xsum4: the unit's four group sums in row 0.
template <int M>
__device__ __forceinline__ void q6_unit(float (&acc)[M], const Q6Raw &r, const int shift, const uint32_t ssel,
                                        const uint4 *__restrict__ xr, const int (&xo)[4][2], const int row_gran,
                                        const float *__restrict__ xsum4, const int row_sums) {
  float dsc[4];
  q6_scales(r, shift, ssel, dsc);
  float s[M][4];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) s[m][c] = 0.0f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * e + ii;
      const uint32_t wa = __builtin_amdgcn_alignbit(r.a[i + 1], r.a[i], shift);
      const uint32_t wb = __builtin_amdgcn_alignbit(r.b[i + 1], r.b[i], shift);
      const uint32_t wh = __builtin_amdgcn_alignbit(r.c[i + 1], r.c[i], shift);
      uint32_t q[4];
      q6_quants(wa, wb, wh, q);
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 xv = xr[m * row_gran + xo[c][e]];
          const uint32_t x0 = ii ? xv.z : xv.x, x1 = ii ? xv.w : xv.y;
          s[m][c] = __builtin_amdgcn_fdot2_f32_bf16(q6_pair_lo(q[c]), __builtin_bit_cast(bf16x2, x0), s[m][c], false);
          s[m][c] = __builtin_amdgcn_fdot2_f32_bf16(q6_pair_hi(q[c]), __builtin_bit_cast(bf16x2, x1), s[m][c], false);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float4 xs = *reinterpret_cast<const float4 *>(xsum4 + m * row_sums);
    const float xv[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m] = __builtin_fmaf(dsc[c], __builtin_fmaf(-160.0f, xv[c], s[m][c]), acc[m]);
  }
}

// Activation staging: granule g of the M concatenated rows (row r = g / gpr)
// to its swizzled slot.
template <int M>
__device__ __forceinline__ void q6_store_x(uint4 *xs, const int g, const int gpr, const uint4 v) {
  int r = 0;
#pragma unroll
  for (int t = 1; t < M; ++t) r += g >= t * gpr;
  xs[r * gpr + q6_slot(g - r * gpr)] = v;
}

template <int M, int kHead>
__device__ __forceinline__ void q6_load_x_head(const uint4 *__restrict__ xg, const int total, const int nthreads,
                                               uint4 (&v)[kHead]) {
#pragma unroll
  for (int i = 0; i < kHead; ++i) {
    const int g = (int)threadIdx.x + i * nthreads;
    v[i] = xg[g < total ? g : 0];
  }
}

template <int M, int kHead>
__device__ __forceinline__ void q6_store_x_head(const uint4 (&v)[kHead], uint4 *xs, const int gpr,
                                                const int nthreads) {
#pragma unroll
  for (int i = 0; i < kHead; ++i) {
    const int g = (int)threadIdx.x + i * nthreads;
    if (g < M * gpr) q6_store_x<M>(xs, g, gpr, v[i]);
  }
}

template <int M, int kHead, int BATCH>
__device__ __forceinline__ void q6_stage_x_tail(const uint4 *__restrict__ xg, uint4 *xs, const int gpr,
                                                const int nthreads) {
  const int total = M * gpr;
  for (int base = kHead * nthreads; base < total; base += nthreads * BATCH) {
    uint4 t[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int g = base + (int)threadIdx.x + i * nthreads;
      t[i] = xg[g < total ? g : 0];
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int g = base + (int)threadIdx.x + i * nthreads;
      if (g < total) q6_store_x<M>(xs, g, gpr, t[i]);
    }
  }
}

// After a barrier: each row's K/16 group sums (16 activations each, summed in
// index order) into the sum table. Ends with a barrier.
template <int M>
__device__ __forceinline__ void q6_x_sums(const uint4 *xs, float *xsum, const int gpr, const int ngrp,
                                          const int nthreads) {
  __syncthreads();
  for (int t = threadIdx.x; t < M * ngrp; t += nthreads) {
    int r = 0;
#pragma unroll
    for (int u = 1; u < M; ++u) r += t >= u * ngrp;
    const int g = t - r * ngrp;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint4 v = xs[r * gpr + q6_slot(2 * g + e)];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += bf16_bits_to_f32(wv[u] & 0xFFFFu);
        s += bf16_bits_to_f32(wv[u] >> 16);
      }
    }
    xsum[r * ngrp + q6_sum_pos(g)] = s;
  }
  __syncthreads();
}

template <int M, int G>
constexpr int q6_x_head() { return (G == 16 ? 4 * M : 9 * M) < 9 ? (G == 16 ? 4 * M : 9 * M) : 9; }

// G lanes own one output row; lane j holds unit j % 4 of block j / 4 + s G/4 at
// step s. Every weight load is issued unconditionally: steps past the row,
// blocks past a partial last step and rows past the matrix read block 0 or 1
// of the matrix (the one with the lane's dword offset) and are never used, so
// the loads in flight are known at every point and each step waits only for
// its own ring slot. NS > 0: rows of exactly NS steps, loop unrolled; NS == 0:
// any length, runtime loop.
template <int M, int G, int D, int NS>
__global__ __launch_bounds__(M == 1 ? kMaxThreads : kMaxThreadsRows) void q6k_gemv_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, const int n, const int k) {
  constexpr int kBlocksPerStep = G / 4;
  constexpr int kStepGranules = kBlocksPerStep * 32;
  constexpr int kStepSums = kBlocksPerStep * 16;
  extern __shared__ uint4 lds[];
  const int nblk = k >> 8;
  const int gpr = k >> 3;
  const int ngrp = k >> 4;
  uint4 *xs = lds;
  float *xsum = reinterpret_cast<float *>(lds + (size_t)M * gpr);

  const int lane = threadIdx.x & 63;
  const int j = lane & (G - 1);
  const int nthreads = (int)blockDim.x;
  const int row = addr::lane_row(blockIdx.x, threadIdx.x, nthreads, G);
  // dword offset of the lane's blocks: 2 bytes when (row * nblk + block) is odd;
  // the same for every step. Fallback loads read block `par` of the matrix
  // (a one-block matrix has only block 0, whose offset is 0).
  const addr::Q6Lane ln = addr::q6_lane(G, NS, n, nblk, row, j);
  const int h = ln.h, p = ln.p, jb = ln.jb, sb = ln.sb;
  const bool active = ln.active, last_ok = ln.last_ok;
  const int nsteps = ln.nsteps;
  const int shift = 8 * sb;
  const uint8_t *wl = w + ln.base, *wfb = w + ln.fb;
  auto step_ptr = [&](const int t) -> const uint8_t * {
    return addr::q6_step_ok(ln, G, nblk, t) ? wl + addr::q6_step_offset(G, t) : wfb;
  };

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  constexpr int kHead = q6_x_head<M, G>();
  uint4 xv[kHead];
  q6_load_x_head<M, kHead>(xg, M * gpr, nthreads, xv);
  Q6Raw ring[D];
  if constexpr (M == 1) {
    q6_load(step_ptr(0), sb, h, p, ring[0]);
    q6_store_x_head<M, kHead>(xv, xs, gpr, nthreads);
#pragma unroll
    for (int t = 1; t < D; ++t) q6_load(step_ptr(t), sb, h, p, ring[t]);
    q6_stage_x_tail<M, kHead, 2>(xg, xs, gpr, nthreads);
  } else {
    q6_store_x_head<M, kHead>(xv, xs, gpr, nthreads);
    q6_stage_x_tail<M, kHead, 8>(xg, xs, gpr, nthreads);
#pragma unroll
    for (int t = 0; t < D; ++t) q6_load(step_ptr(t), sb, h, p, ring[t]);
  }
  q6_x_sums<M>(xs, xsum, gpr, ngrp, nthreads);
  if (!active) return;

  // per-lane LDS granule offsets of (quarter c, granule e) within the unit's
  // 16-granule half-block row: (4c + 2p + e) xor (h | (block & 3) << 2); the
  // block advances by a multiple of 4 per step, so these are fixed per lane
  const int f = h | ((jb & 3) << 2);
  int xo[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 2; ++e) xo[c][e] = (4 * c + 2 * p + e) ^ f;
  const uint4 *xr = xs + 32 * jb + 16 * h;
  const float *xsu = xsum + 16 * jb + 8 * h + 4 * p;
  const uint32_t ssel = p ? 0x07050301u : 0x06040200u;
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int t = s % D;
      if (s < NS - 1 || last_ok)
        q6_unit<M>(acc, ring[t], shift, ssel, xr + s * kStepGranules, xo, gpr, xsu + s * kStepSums, ngrp);
      if (s + D < NS) q6_load(step_ptr(s + D), sb, h, p, ring[t]);
    }
  } else {
    for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
      for (int t = 0; t < D; ++t) {
        const int s = s0 + t;
        if (s < nsteps && s * kBlocksPerStep + jb < nblk)
          q6_unit<M>(acc, ring[t], shift, ssel, xr + s * kStepGranules, xo, gpr, xsu + s * kStepSums, ngrp);
        q6_load(step_ptr(s + D), sb, h, p, ring[t]);
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float v = group_sum<G>(acc[m]);
    if (j == m) y[(size_t)m * n + row] = v;
  }
}

// One thread per unit: the unit's 64 weights rounded once to fp32 (d sc is
// exact, so (d sc) q is the single rounding of the exact weight).
__global__ __launch_bounds__(256) void q6k_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                          const size_t nunits) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nunits) return;
  const size_t blk = t >> 2;
  const int u = (int)(t & 3), h = u >> 1, p = u & 1;
  const int par = (int)(blk & 1);  // the matrix base is 16-byte aligned
  Q6Raw r;
  q6_load(w + blk * kQ6KBlockBytes, 2 * par, h, p, r);
  float dsc[4];
  q6_scales(r, 16 * par, p ? 0x07050301u : 0x06040200u, dsc);
  float *ob = out + blk * 256 + 128 * h + 16 * p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t q[4];
    q6_quants(__builtin_amdgcn_alignbit(r.a[i + 1], r.a[i], 16 * par),
              __builtin_amdgcn_alignbit(r.b[i + 1], r.b[i], 16 * par),
              __builtin_amdgcn_alignbit(r.c[i + 1], r.c[i], 16 * par), q);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float4 v;
      v.x = dsc[c] * (float)((int)(q[c] & 0xFFu) - 32);
      v.y = dsc[c] * (float)((int)((q[c] >> 8) & 0xFFu) - 32);
      v.z = dsc[c] * (float)((int)((q[c] >> 16) & 0xFFu) - 32);
      v.w = dsc[c] * (float)((int)(q[c] >> 24) - 32);
      *reinterpret_cast<float4 *>(ob + 32 * c + 4 * i) = v;
    }
  }
}

// The plan (lanes per row, steps, ring depth, rows per workgroup, grid) is
// addr::q6_gemv_plan. Ring depths (addr::q6_depth): at M = 1 a 5-step row of
// 16 lanes keeps every load in flight from the start, and the 9-step rows of
// 32 lanes run fastest with 2; at M = 2..4 (more registers per step, fewer
// waves) 3 is fastest for both. Each instantiation below is the one the plan
// names.
template <int M, int G, int NS>
int q6_launch(const addr::GemvPlan &pl, const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream) {
  constexpr int D = addr::q6_depth(M, G);
  const size_t lds = q6_lds_bytes<M>(k);
  auto *fn = q6k_gemv_kernel<M, G, D, NS>;
  static LdsGrant granted;
  if (allow_dynamic_lds(reinterpret_cast<const void *>(fn), lds, granted, "q6k_gemv_kernel")) return QMV_ERR_HIP;
  return launch_kernel("q6k_gemv_kernel", fn, dim3(pl.grid), dim3(pl.rows * G), lds, stream, w, x, y, n, k);
}

template <int M>
int q6_launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream) {
  const addr::GemvPlan p = addr::q6_gemv_plan(M, n, k);
  if (p.G == 16) {
    switch (p.ns) {
      case 1: return q6_launch<M, 16, 1>(p, w, x, y, n, k, stream);
      case 2: return q6_launch<M, 16, 2>(p, w, x, y, n, k, stream);
      case 3: return q6_launch<M, 16, 3>(p, w, x, y, n, k, stream);
      case 4: return q6_launch<M, 16, 4>(p, w, x, y, n, k, stream);
      case 5: return q6_launch<M, 16, 5>(p, w, x, y, n, k, stream);
      case 6: return q6_launch<M, 16, 6>(p, w, x, y, n, k, stream);
      case 7: return q6_launch<M, 16, 7>(p, w, x, y, n, k, stream);
      default: return q6_launch<M, 16, 8>(p, w, x, y, n, k, stream);
    }
  }
  switch (p.ns) {
    case 5: return q6_launch<M, 32, 5>(p, w, x, y, n, k, stream);
    case 6: return q6_launch<M, 32, 6>(p, w, x, y, n, k, stream);
    case 7: return q6_launch<M, 32, 7>(p, w, x, y, n, k, stream);
    case 8: return q6_launch<M, 32, 8>(p, w, x, y, n, k, stream);
    case 9: return q6_launch<M, 32, 9>(p, w, x, y, n, k, stream);
    default: return q6_launch<M, 32, 0>(p, w, x, y, n, k, stream);
  }
}

}  // namespace

int launch_q6_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return q6_launch_m<1>(w, x, y, n, k, s);
    case 2: return q6_launch_m<2>(w, x, y, n, k, s);
    case 3: return q6_launch_m<3>(w, x, y, n, k, s);
    case 4: return q6_launch_m<4>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_dequant_q6_k(const void *w, float *out, int n, int k, void *stream) {
  const size_t nunits = (size_t)n * (size_t)(k >> 8) * 4;
  const unsigned grid = (unsigned)((nunits + 255) / 256);
  return launch_kernel("q6k_dequant_kernel", q6k_dequant_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), w, out, nunits);
}

}  // namespace qmv
