// Prefill-sized Q4_K GEMM Y = X W^T on bf16 matrix cores, gfx950.
//
// Prompt processing ahead of decode (the time-to-first-token rows of the memra
// summary page's performance table) multiplies the same quantized weights by
// many activation rows at once, which makes it a dense contraction: the weights
// are dequantized into bf16 tiles in LDS and fed to v_mfma_f32_16x16x32_bf16
// with fp32 accumulation.
//
// Tiling. A 256-thread workgroup owns a 128 (rows of X) x 128 (rows of W) tile
// of Y; its four waves own 64x64 sub-tiles (4x4 MFMA tiles of 16x16, 64 fp32
// accumulators per lane). K advances 64 at a time -- one 64-weight chunk of each
// W row's super-block -- through two LDS stages of 32 KiB (X tile + W tile,
// 16-byte granules swizzled by row so fragment reads are conflict-free). While
// the matrix cores work on stage s, the next step's X granules and Q4_K bytes
// are already in flight from global memory; after the MFMAs they are written
// (W dequantized) into the other stage.
//
// Dequantization matches the bf16 dequant entry point bit for bit: each weight
// is fma(d*sc, q, -(dmin*m)) (one rounding of the exact value to fp32), then
// rounded to nearest-even bf16.
#include "q4k_common.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kGranPerRow = BK / 8;                 // 16-byte granules per tile row
constexpr int kTileGran = BM * kGranPerRow;         // granules per operand tile

__device__ __forceinline__ int tile_slot(int row, int g) { return row * kGranPerRow + (g ^ (row & 7)); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Issue the global loads of K-step s: four X granules and this thread's W header + 16 quant bytes.
__device__ __forceinline__ void prefill_load(const uint16_t *__restrict__ x, const uint8_t *__restrict__ w_rowp,
                                             const bool w_ok, const int w_half, const int m0, const int M,
                                             const int K, const int s, uint4 (&xr)[4], uint4 &whdr, uint4 &wq) {
  const int k0 = s * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = threadIdx.x + kThreads * i;
    const int row = m0 + (g >> 3);
    xr[i] = row < M ? *reinterpret_cast<const uint4 *>(x + (size_t)row * K + k0 + 8 * (g & 7))
                    : make_uint4(0u, 0u, 0u, 0u);
  }
  if (w_ok) {
    const uint8_t *bp = w_rowp + (size_t)(s >> 2) * kQ4KBlockBytes;
    whdr = *reinterpret_cast<const uint4 *>(bp);
    wq = *reinterpret_cast<const uint4 *>(bp + 16 + 32 * (s & 3) + 16 * w_half);
  } else {
    whdr = make_uint4(0u, 0u, 0u, 0u);  // d = dmin = 0: padding rows dequantize to zeros
    wq = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Write K-step s into an LDS stage: the X granules as loaded, the W chunk dequantized to bf16.
__device__ __forceinline__ void prefill_store(uint4 *__restrict__ xt, uint4 *__restrict__ wt, const int s,
                                              const int w_row, const int w_half, const uint4 (&xr)[4],
                                              const uint4 whdr, const uint4 wq) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = threadIdx.x + kThreads * i;
    xt[tile_slot(g >> 3, g & 7)] = xr[i];
  }
  const ChunkScales cs = chunk_scales(whdr, scale_selectors(s & 3));
  const uint32_t qw[4] = {wq.x, wq.y, wq.z, wq.w};
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b0 = (qw[i >> 1] >> (16 * (i & 1))) & 0xFFu;
    const uint32_t b1 = (qw[i >> 1] >> (16 * (i & 1) + 8)) & 0xFFu;
    lo[i] = pack_bf16(__builtin_fmaf(cs.a0, (float)(b0 & 0xFu), -cs.b0),
                      __builtin_fmaf(cs.a0, (float)(b1 & 0xFu), -cs.b0));
    hi[i] = pack_bf16(__builtin_fmaf(cs.a1, (float)(b0 >> 4), -cs.b1),
                      __builtin_fmaf(cs.a1, (float)(b1 >> 4), -cs.b1));
  }
  // local k of this thread's weights: 16h + 0..15 (sub-block 2c) and 32 + 16h + 0..15 (2c + 1)
  wt[tile_slot(w_row, 2 * w_half)] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  wt[tile_slot(w_row, 2 * w_half + 1)] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
  wt[tile_slot(w_row, 4 + 2 * w_half)] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  wt[tile_slot(w_row, 5 + 2 * w_half)] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
}

__global__ __launch_bounds__(kThreads) void q4k_prefill_kernel(const uint8_t *__restrict__ w,
                                                               const uint16_t *__restrict__ x,
                                                               float *__restrict__ y, const int M, const int N,
                                                               const int K) {
  __shared__ uint4 lds[2][2][kTileGran];  // [stage][0 = X, 1 = W]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nblk = K >> 8;
  const int nsteps = K / BK;

  // X tile loads: granule g = tid + 256 i covers tile row g / 8, granule g % 8.
  // W tile: thread t dequantizes 32 weights of W row n0 + t/2 (half t%2 of the chunk).
  const int w_row = tid >> 1, w_half = tid & 1;
  const bool w_ok = n0 + w_row < N;
  const uint8_t *w_rowp = w + (size_t)(w_ok ? n0 + w_row : 0) * (size_t)nblk * kQ4KBlockBytes;
  uint4 xr[4], whdr, wq;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  prefill_load(x, w_rowp, w_ok, w_half, m0, M, K, 0, xr, whdr, wq);
  prefill_store(lds[0][0], lds[0][1], 0, w_row, w_half, xr, whdr, wq);
  __syncthreads();

  const int frag_row = lane & 15, frag_g = lane >> 4;
  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    if (s + 1 < nsteps) prefill_load(x, w_rowp, w_ok, w_half, m0, M, K, s + 1, xr, whdr, wq);
    const uint4 *xt = lds[stage][0];
    const uint4 *wt = lds[stage][1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = __builtin_bit_cast(bf16x8, xt[tile_slot(wm + 16 * i + frag_row, 4 * kk + frag_g)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = __builtin_bit_cast(bf16x8, wt[tile_slot(wn + 16 * j + frag_row, 4 * kk + frag_g)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsteps) prefill_store(lds[stage ^ 1][0], lds[stage ^ 1][1], s + 1, w_row, w_half, xr, whdr, wq);
    __syncthreads();
  }

  // C fragment of a 16x16 MFMA tile: lane l holds rows 4*(l/16) + r, column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + 16 * j + frag_row;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm + 16 * i + 4 * frag_g + r;
        if (row < M) y[(size_t)row * N + col] = acc[i][j][r];
      }
    }
}

}  // namespace

int launch_q4_k_prefill(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  return launch_kernel("q4k_prefill_kernel", q4k_prefill_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), w, x, y, m, n,
                       k);
}

}  // namespace qmv
