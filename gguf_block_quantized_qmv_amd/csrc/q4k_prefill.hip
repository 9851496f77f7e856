// Prefill-sized Q4_K GEMM Y = X W^T on bf16 matrix cores, gfx950.
//
// Prompt processing ahead of decode (the time-to-first-token rows of the memra
// summary page's performance table) multiplies the same quantized weights by
// many activation rows at once, which makes it a dense contraction: the weights
// are dequantized into bf16 tiles in LDS and fed to v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.
//
// Tiling. A 256-thread workgroup owns a 128 (rows of X) x 128 (rows of W) tile
// of Y; each of its four waves owns a 64 x 64 quarter, four 32x32 MFMA tiles
// (64 fp32 accumulators per lane). K advances 64 at a time -- one 64-weight
// chunk of each W row's super-block -- through two LDS stages of 32 KiB (X tile
// + W tile, rows of eight 16-byte granules, swizzled so that the 16 lanes a
// 16-byte read serves per cycle hit 16 distinct bank groups). Global loads run
// kDepth steps ahead through a ring of registers: while the matrix cores work
// on stage s, step s + 1 (loaded kDepth - 1 steps earlier) is written into the
// other stage, W dequantized, and the loads for step s + 1 + kDepth go out.
// Every load is unconditional (steps past K reload the last step) and the step
// loop is unrolled by kDepth, which divides the step count because K is a
// multiple of 256, so each wait covers exactly the slot being consumed.
// Workgroups (n, m) and (n, m + 1) are n_tiles apart in launch order, so with
// n_tiles a multiple of 8 they run on the same XCD and share the W rows in its L2.
//
// Dequantization matches the bf16 dequant entry point bit for bit: each weight
// is fma(d*sc, q, -(dmin*m)) (one rounding of the exact value to fp32), then
// rounded to nearest-even bf16 by v_cvt_pk_bf16_f32.
#include "q4k_common.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kDepth = 4;                    // steps of global loads in flight
constexpr int kXGran = BM * 8;               // 16-byte granules of an X tile
constexpr int kWGran = BN * 8;               // and of a W tile
constexpr int kStageGran = kXGran + kWGran;
constexpr size_t kLdsBytes = 2 * (size_t)kStageGran * 16;
constexpr int kXPerThread = kXGran / kThreads;   // 4

// Granule g (8 bf16 of K) of tile row r. A 16-byte LDS read serves 16 lanes per
// cycle over 64 banks, i.e. 16 granule slots of a 256-byte line; 16 consecutive
// rows read at one g land on 16 distinct slots because rows of equal parity get
// distinct g ^ ((r >> 1) & 7).
__device__ __forceinline__ int tslot(int r, int g) { return r * 8 + (g ^ ((r >> 1) & 7)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// One step's global data for this thread: four X granules, and for W row
// n0 + tid / 2 the block header and quant bytes 16 * (tid % 2) .. + 15 of chunk s % 4.
struct StepRegs {
  uint4 x[kXPerThread];
  uint4 hdr, q;
};

// Rows past M read row 0 and rows past N row 0 of W (the caller zeroes their
// contribution); steps past K read the last step.
__device__ __forceinline__ void load_step(const uint16_t *__restrict__ x, const uint8_t *__restrict__ w_rowp,
                                          const int m0, const int M, const int K, const int nsteps, int s,
                                          StepRegs &r) {
  s = s < nsteps ? s : nsteps - 1;
  const int k0 = s * BK;
#pragma unroll
  for (int i = 0; i < kXPerThread; ++i) {
    const int g = (int)threadIdx.x + kThreads * i;
    const int row = m0 + (g >> 3);
    r.x[i] = reinterpret_cast<const uint4 *>(x + (size_t)(row < M ? row : 0) * K + k0)[g & 7];
  }
  const uint8_t *bp = w_rowp + (size_t)(s >> 2) * kQ4KBlockBytes;
  r.hdr = *reinterpret_cast<const uint4 *>(bp);
  r.q = *reinterpret_cast<const uint4 *>(bp + 16 + 32 * (s & 3) + 16 * (threadIdx.x & 1));
}

// Eight nibbles (the low or high nibbles of two quant words, already masked to
// one per byte) as exact fp32: a byte q <= 15 read as e4m3 is q * 2^-9.
__device__ __forceinline__ void nibbles_f32(uint32_t b0, uint32_t b1, float (&f)[8]) {
  const floatx2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b0, 512.0f, false);
  const floatx2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b0, 512.0f, true);
  const floatx2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b1, 512.0f, false);
  const floatx2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b1, 512.0f, true);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y; f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// Write a step into a stage: X granules as loaded (rows past M as zeros), the
// W half-chunk dequantized to bf16 (rows past N as zeros).
__device__ __forceinline__ void store_step(uint4 *__restrict__ xt, uint4 *__restrict__ wt, const int s,
                                           const StepRegs &r, const int m0, const int M, const bool w_ok) {
#pragma unroll
  for (int i = 0; i < kXPerThread; ++i) {
    const int g = (int)threadIdx.x + kThreads * i;
    xt[tslot(g >> 3, g & 7)] = m0 + (g >> 3) < M ? r.x[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  const uint4 hdr = w_ok ? r.hdr : make_uint4(0u, 0u, 0u, 0u);   // d = dmin = 0: zero weights
  const ChunkScales cs = chunk_scales(hdr, scale_selectors(s & 3));
  const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
  uint32_t pl[8], ph[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float lo[8], hi[8];
    nibbles_f32(qw[2 * h] & 0x0F0F0F0Fu, qw[2 * h + 1] & 0x0F0F0F0Fu, lo);
    nibbles_f32((qw[2 * h] >> 4) & 0x0F0F0F0Fu, (qw[2 * h + 1] >> 4) & 0x0F0F0F0Fu, hi);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pl[4 * h + e] = pack_bf16x2(__builtin_fmaf(cs.a0, lo[2 * e], -cs.b0), __builtin_fmaf(cs.a0, lo[2 * e + 1], -cs.b0));
      ph[4 * h + e] = pack_bf16x2(__builtin_fmaf(cs.a1, hi[2 * e], -cs.b1), __builtin_fmaf(cs.a1, hi[2 * e + 1], -cs.b1));
    }
  }
  // this thread's weights: local k 16 h2 .. +15 (sub-block 2c) and 32 + 16 h2 .. +15 (2c + 1)
  const int row = threadIdx.x >> 1, h2 = threadIdx.x & 1;
  wt[tslot(row, 2 * h2)] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  wt[tslot(row, 2 * h2 + 1)] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
  wt[tslot(row, 4 + 2 * h2)] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  wt[tslot(row, 5 + 2 * h2)] = make_uint4(ph[4], ph[5], ph[6], ph[7]);
}

__global__ __launch_bounds__(kThreads) void q4k_prefill_kernel(const uint8_t *__restrict__ w,
                                                               const uint16_t *__restrict__ x,
                                                               float *__restrict__ y, const int M, const int N,
                                                               const int K) {
  extern __shared__ uint4 lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nblk = K >> 8;
  const int nsteps = K / BK;   // a multiple of kDepth

  const bool w_ok = n0 + (tid >> 1) < N;
  const uint8_t *w_rowp = w + (size_t)(w_ok ? n0 + (tid >> 1) : 0) * (size_t)nblk * kQ4KBlockBytes;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  StepRegs ring[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) load_step(x, w_rowp, m0, M, K, nsteps, u, ring[u]);
  store_step(lds, lds + kXGran, 0, ring[0], m0, M, w_ok);
  load_step(x, w_rowp, m0, M, K, nsteps, kDepth, ring[0]);
  __syncthreads();

  // MFMA operands: lane l supplies row (l % 32) and K granule (l / 32) of a 32 x 16 slice
  const int frow = lane & 31, fg = lane >> 5;
  for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int s = s0 + u;
      const uint4 *xt = lds + (u & 1) * kStageGran;   // s & 1 == u & 1: kDepth is even
      const uint4 *wt = xt + kXGran;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = __builtin_bit_cast(bf16x8, xt[tslot(wm + 32 * i + frow, 2 * kk + fg)]);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = __builtin_bit_cast(bf16x8, wt[tslot(wn + 32 * j + frow, 2 * kk + fg)]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      // step s + 1 into the other stage (past the last step this writes a copy
      // of the last step, which nobody reads), then its ring slot is refilled
      constexpr int kD = kDepth;
      const int un = (u + 1) % kD;
      uint4 *nx = lds + ((u + 1) & 1) * kStageGran;
      store_step(nx, nx + kXGran, s + 1, ring[un], m0, M, w_ok);
      load_step(x, w_rowp, m0, M, K, nsteps, s + 1 + kDepth, ring[un]);
      __syncthreads();
    }
  }

  // 32x32 accumulator layout: lane l holds column l % 32 and, in register
  // 4 q + e, row 8 q + 4 (l / 32) + e
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + frow;
      if (col >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm + 32 * i + 8 * q + 4 * fg + e;
          if (row < M) y[(size_t)row * N + col] = acc[i][j][4 * q + e];
        }
    }
}

}  // namespace

int launch_q4_k_prefill(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream) {
  static std::atomic<size_t> granted{0};
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&q4k_prefill_kernel), kLdsBytes, granted,
                        "q4k_prefill_kernel lds"))
    return QMV_ERR_HIP;
  const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  return launch_kernel("q4k_prefill_kernel", q4k_prefill_kernel, grid, dim3(kThreads), kLdsBytes,
                       static_cast<hipStream_t>(stream), w, x, y, m, n, k);
}

}  // namespace qmv
