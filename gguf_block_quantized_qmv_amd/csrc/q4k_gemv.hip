// Q4_K matrix x bf16 activation rows (decode M=1, speculative verify M=2..4), gfx950.
//
// Work mapping. A group of 16 lanes (one DPP row) owns one output row; a wave
// owns 4 rows and a 256-thread workgroup 16 rows. Lane j of a group reads, at
// step s, 64-weight chunk c = j % 4 of super-block b = 4s + j / 4 of its row:
// the 16-byte block header and the 32 quant bytes of that chunk, as 16-byte
// loads (the four lanes of a block cover its 144 bytes). Rows of 5120 and 17408
// weights are exactly 5 and 17 steps. The chunk fixes the lane's two sub-blocks
// (2c, 2c+1), so each lane unpacks two scales and two mins per step.
//
// Arithmetic per chunk and activation row r:
//   S_lo = sum q_i x_i over the 32 weights of sub-block 2c   (v_dot2 on exact bf16 q)
//   S_hi = the same over sub-block 2c+1
//   acc_r += (d sc_2c) S_lo - (dmin m_2c) X_2c + (d sc_2c+1) S_hi - (dmin m_2c+1) X_2c+1
// where X_j = sum of the 32 activations of sub-block j, precomputed once per
// workgroup. The quants are converted exactly (q is an e4m3 value q*2^-9 scaled
// by 2^9), products of q with bf16 x are exact in fp32, and accumulation is fp32.
//
// LDS holds only the activations: M rows of bf16 in swizzled 16-byte granules,
// then the M x K/32 sub-block sums. Each row is reduced inside its 16-lane DPP
// row; nothing crosses waves.
//
// Batch invariance: the instruction sequence applied to activation row r does
// not depend on M (every row runs the same unrolled body, explicit fma/dot
// builtins, no reassociation), so row r is bit-identical for M = 1..4.
#include "q4k_common.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {


template <int M>
__host__ __device__ constexpr size_t dense_lds_bytes(int k) {
  return (size_t)M * padded_row_granules(k) * 16 + (size_t)M * (size_t)(k >> 5) * 4;
}

// Stage M activation rows (row r at x + r*K) in the padded layout, then each
// row's K/32 sub-block sums from LDS (summed in index order). Ends with a barrier.
template <int M, int kThreads>
__device__ __forceinline__ void stage_dense(const uint16_t *__restrict__ x, uint4 *xs, float *xsum, const int gpr,
                                            const int gpp, const int nsub) {
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const int total = M * gpr;
  for (int base = 0; base < total; base += kThreads * 8) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = base + (int)threadIdx.x + i * kThreads;
      v[i] = xg[g < total ? g : 0];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = base + (int)threadIdx.x + i * kThreads;
      if (g < total) {
        int r = 0;
#pragma unroll
        for (int q = 1; q < M; ++q) r += g >= q * gpr;
        xs[r * gpp + padded_granule(g - r * gpr)] = v[i];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < M * nsub; t += kThreads) {
    int r = 0;
#pragma unroll
    for (int q = 1; q < M; ++q) r += t >= q * nsub;
    const int sb = t - r * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = xs[r * gpp + padded_granule(4 * sb + q)];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
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
template <int M>
__device__ __forceinline__ void dense_chunk(float (&acc)[M], const uint4 hdr, const uint4 qa, const uint4 qb,
                                            const ScaleSel &sel, const uint4 *__restrict__ xc, const int gpp,
                                            const float *__restrict__ xsc, const int nsub) {
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
  for (int r = 0; r < M; ++r) {
    const uint4 *xr = xc + r * gpp;
    // four independent dot2 chains (two per sub-block), joined in a fixed order
    float s_lo0 = 0.0f, s_lo1 = 0.0f, s_hi0 = 0.0f, s_hi1 = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint4 v = xr[g];
      const uint4 u = xr[4 + g];
      s_lo0 = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 0], __builtin_bit_cast(bf16x2, v.x), s_lo0, false);
      s_hi0 = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 0], __builtin_bit_cast(bf16x2, u.x), s_hi0, false);
      s_lo1 = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 1], __builtin_bit_cast(bf16x2, v.y), s_lo1, false);
      s_hi1 = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 1], __builtin_bit_cast(bf16x2, u.y), s_hi1, false);
      s_lo0 = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 2], __builtin_bit_cast(bf16x2, v.z), s_lo0, false);
      s_hi0 = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 2], __builtin_bit_cast(bf16x2, u.z), s_hi0, false);
      s_lo1 = __builtin_amdgcn_fdot2_f32_bf16(lo[4 * g + 3], __builtin_bit_cast(bf16x2, v.w), s_lo1, false);
      s_hi1 = __builtin_amdgcn_fdot2_f32_bf16(hi[4 * g + 3], __builtin_bit_cast(bf16x2, u.w), s_hi1, false);
    }
    const float s_lo = s_lo0 + s_lo1, s_hi = s_hi0 + s_hi1;
    const float2 xsm = *reinterpret_cast<const float2 *>(xsc + r * nsub);
    acc[r] = __builtin_fmaf(cs.a0, s_lo, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b0, xsm.x, acc[r]);
    acc[r] = __builtin_fmaf(cs.a1, s_hi, acc[r]);
    acc[r] = __builtin_fmaf(-cs.b1, xsm.y, acc[r]);
  }
}

// G lanes own one output row (G = 16, 32 or 64): a step covers G/4 super-blocks
// of the row, lane j holding chunk j % 4 of block j / 4. A wave owns 64/G rows.
// The first D steps of weight loads are issued before the activations are
// staged; afterwards a ring of D steps stays in flight. FULL: the row is a whole
// number of steps, so no lane needs a block-range test.
template <int M, int G, int D, bool FULL, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void q4k_gemv_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  constexpr int kRows = 64 / G;
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
  const int c = j & 3;
  const int jb = j >> 2;
  const int row = (blockIdx.x * kWaves + (threadIdx.x >> 6)) * kRows + lane / G;
  const bool active = row < n;
  const int nsteps = (nblk + kBlocksPerStep - 1) / kBlocksPerStep;
  const uint8_t *wl = w + (size_t)(active ? row : 0) * (size_t)nblk * kQ4KBlockBytes + (size_t)jb * kQ4KBlockBytes;

  uint4 hdr[D], qa[D], qb[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (active && u < nsteps && (FULL || u * kBlocksPerStep + jb < nblk)) {
      const uint8_t *bp = wl + (size_t)(u * kBlocksPerStep) * kQ4KBlockBytes;
      hdr[u] = *reinterpret_cast<const uint4 *>(bp);
      qa[u] = *reinterpret_cast<const uint4 *>(bp + 16 + 32 * c);
      qb[u] = *reinterpret_cast<const uint4 *>(bp + 32 + 32 * c);
    }
  }
  stage_dense<M, 64 * kWaves>(x, xs, xsum, gpr, gpp, nsub);
  if (!active) return;

  const ScaleSel sel = scale_selectors(c);
  const uint4 *xb = xs + (j >> 1) * 17 + (j & 1) * 8;
  const float *sb = xsum + 2 * j;
  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;

  for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int s = s0 + u;
      if (s < nsteps && (FULL || s * kBlocksPerStep + jb < nblk))
        dense_chunk<M>(acc, hdr[u], qa[u], qb[u], sel, xb + s * kStepGranules, gpp, sb + s * 2 * G, nsub);
      const int sn = s + D;
      if (sn < nsteps && (FULL || sn * kBlocksPerStep + jb < nblk)) {
        const uint8_t *bp = wl + (size_t)(sn * kBlocksPerStep) * kQ4KBlockBytes;
        hdr[u] = *reinterpret_cast<const uint4 *>(bp);
        qa[u] = *reinterpret_cast<const uint4 *>(bp + 16 + 32 * c);
        qb[u] = *reinterpret_cast<const uint4 *>(bp + 32 + 32 * c);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float v = group_sum<G>(acc[r]);
    if (j == r) y[(size_t)r * n + row] = v;
  }
}

template <int M, int G, int D, int W>
int launch_mgd(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream) {
  const size_t lds = dense_lds_bytes<M>(k);
  const bool full = ((k >> 8) % (G / 4)) == 0;
  const void *fn = full ? reinterpret_cast<const void *>(&q4k_gemv_kernel<M, G, D, true, W>)
                        : reinterpret_cast<const void *>(&q4k_gemv_kernel<M, G, D, false, W>);
  static std::atomic<size_t> granted_full{0}, granted_part{0};
  if (allow_dynamic_lds(fn, lds, full ? granted_full : granted_part, "q4k_gemv_kernel lds")) return QMV_ERR_HIP;
  const int rows_per_group = W * (64 / G);
  const unsigned grid = (unsigned)((n + rows_per_group - 1) / rows_per_group);
  if (full)
    return launch_kernel("q4k_gemv_kernel", q4k_gemv_kernel<M, G, D, true, W>, dim3(grid), dim3(64 * W), lds, stream,
                         w, x, y, n, k);
  return launch_kernel("q4k_gemv_kernel", q4k_gemv_kernel<M, G, D, false, W>, dim3(grid), dim3(64 * W), lds, stream,
                       w, x, y, n, k);
}

// Lanes per row and ring depth by row length.
template <int M>
int launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream) {
  if (k <= 8192) return launch_mgd<M, 16, 4, 4>(w, x, y, n, k, stream);
  return launch_mgd<M, 32, 4, 4>(w, x, y, n, k, stream);
}

}  // namespace

int launch_q4_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1>(w, x, y, n, k, s);
    case 2: return launch_m<2>(w, x, y, n, k, s);
    case 3: return launch_m<3>(w, x, y, n, k, s);
    case 4: return launch_m<4>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

}  // namespace qmv
