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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerWave = 64 / kLanesPerRow;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr int kStepsInFlight = 4;   // super-block steps whose loads are issued together

template <int M>
__global__ __launch_bounds__(kThreads) void q4k_gemv_kernel(const uint8_t *__restrict__ w,
                                                            const uint16_t *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  extern __shared__ uint4 lds[];
  const int nblk = k >> 8;   // super-blocks per row
  const int gpr = k >> 3;    // 16-byte granules per staged activation row
  const int nsub = k >> 5;   // 32-weight sub-blocks per row
  uint4 *xs = lds;
  float *xsum = reinterpret_cast<float *>(lds + M * gpr);
#pragma unroll
  for (int r = 0; r < M; ++r)
    stage_bf16_row(x + (size_t)r * k, xs + r * gpr, xsum + r * nsub, gpr, nsub, threadIdx.x, kThreads);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);
  const int row = (blockIdx.x * kWaves + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanesPerRow;
  if (row >= n) return;  // whole 16-lane groups leave together

  const int c = j & 3;
  const ScaleSel sel = scale_selectors(c);
  const uint8_t *wrow = w + (size_t)row * (size_t)nblk * kQ4KBlockBytes;
  const int nsteps = (nblk + 3) >> 2;

  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;

  for (int s0 = 0; s0 < nsteps; s0 += kStepsInFlight) {
    uint4 hdr[kStepsInFlight], qa[kStepsInFlight], qb[kStepsInFlight];
    bool ok[kStepsInFlight];
#pragma unroll
    for (int u = 0; u < kStepsInFlight; ++u) {
      const int b = (s0 + u) * 4 + (j >> 2);
      ok[u] = b < nblk;
      if (ok[u]) {
        const uint8_t *blk = wrow + (size_t)b * kQ4KBlockBytes;
        hdr[u] = *reinterpret_cast<const uint4 *>(blk);
        qa[u] = *reinterpret_cast<const uint4 *>(blk + 16 + 32 * c);
        qb[u] = *reinterpret_cast<const uint4 *>(blk + 32 + 32 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < kStepsInFlight; ++u)
      if (ok[u]) q4k_chunk_bf16<M>(acc, M, hdr[u], qa[u], qb[u], (s0 + u) * 16 + j, sel, xs, xsum, gpr, nsub);
  }

#pragma unroll
  for (int r = 0; r < M; ++r) {
    const float v = row16_sum(acc[r]);
    if (j == r) y[(size_t)r * n + row] = v;
  }
}

template <int M>
int launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t stream) {
  const size_t lds = (size_t)M * (size_t)(k >> 3) * 16 + (size_t)M * (size_t)(k >> 5) * 4;
  static std::atomic<size_t> granted{0};
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&q4k_gemv_kernel<M>), lds, granted, "q4k_gemv_kernel lds"))
    return QMV_ERR_HIP;
  const unsigned grid = (unsigned)((n + kRowsPerGroup - 1) / kRowsPerGroup);
  return launch_kernel("q4k_gemv_kernel", q4k_gemv_kernel<M>, dim3(grid), dim3(kThreads), lds, stream, w, x, y, n, k);
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
