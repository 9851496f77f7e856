// Q8_0 matrix x fp32 activation rows, and Q8_0 dequantization, gfx950.
//
// Q8_0 block (34 bytes, 32 weights): fp16 d then int8 q[32]; w = d * q.
// Blocks are only 2-byte aligned (34 = 2 mod 4), so a lane reads the 36-byte
// dword-aligned window that holds its block: eight dwords plus a final dword
// (block at offset 2 mod 4, the window starting in the previous block's last
// two bytes) or 16-bit half (block at offset 0 mod 4), so every access stays
// inside the matrix, then realigns with v_alignbit. 32 lanes own one output row (one block per lane per step);
// activations are staged in LDS as fp32 in swizzled 16-byte granules.
#include "qmv_addr.h"
#include "qmv_device.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

constexpr int kQ80BlockBytes = 34;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 32;
constexpr int kRowsPerWave = 64 / kLanesPerRow;

// LDS slot of fp32 granule g (4 activations) of a staged row: a 32-weight block
// spans 8 granules, and granule i of block b sits at 8 b + (i ^ ((b >> 1) & 7)),
// so the lanes of a row, which read granule i of consecutive blocks, spread over
// eight slot positions (at most two lanes of a 16-lane read share a bank group).
__device__ __forceinline__ int swizzle_granule(int g) { return g ^ ((g >> 4) & 7); }

// Load Q8_0 block starting at byte offset `off` (even) from a dword-aligned base.
// Returns d and the 32 quants as 8 little-endian words (q[4i..4i+3] in word i).
// The reads are addr::q80_window(off): 36 bytes from 2 before the block when it
// starts mid-dword, else its 34 bytes.
__device__ __forceinline__ float load_q8_0_block(const uint8_t *__restrict__ base, size_t off, uint32_t (&q)[8]) {
  const size_t a = off - (size_t)(-addr::q80_window(off).off);
  const bool shifted = (off & 3) != 0;  // block starts 2 bytes into its first dword
  const uint32_t *p = reinterpret_cast<const uint32_t *>(base + a);
  uint32_t dw[9];
#pragma unroll
  for (int i = 0; i < 8; ++i) dw[i] = p[i];
  dw[8] = shifted ? p[8] : (uint32_t)(*reinterpret_cast<const uint16_t *>(base + a + 32));
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = shifted ? dw[i + 1] : __builtin_amdgcn_alignbit(dw[i + 1], dw[i], 16);
  return fp16_bits_to_f32(shifted ? (dw[0] >> 16) : (dw[0] & 0xFFFFu));
}

__device__ __forceinline__ float sbyte_to_f32(uint32_t word, int byte) {
  return (float)(int32_t)(int8_t)(uint8_t)(word >> (8 * byte));
}

template <int M>
__global__ __launch_bounds__(kThreads) void q80_gemv_kernel(const uint8_t *__restrict__ w, const float *__restrict__ x,
                                                            float *__restrict__ y, const int n, const int k) {
  extern __shared__ uint4 lds[];
  const int nblk = k >> 5;
  const int gpr = k >> 2;  // fp32 granules per row
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
#pragma unroll
  for (int r = 0; r < M; ++r)
    for (int g = threadIdx.x; g < gpr; g += kThreads) lds[r * gpr + swizzle_granule(g)] = xg[r * gpr + g];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int j = lane & (kLanesPerRow - 1);
  const int row = (blockIdx.x * kWaves + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanesPerRow;
  if (row >= n) return;  // whole 32-lane groups leave together

  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;

  for (int b = j; b < nblk; b += kLanesPerRow) {
    uint32_t q[8];
    const float d = load_q8_0_block(w, ((size_t)row * nblk + b) * kQ80BlockBytes, q);
#pragma unroll
    for (int r = 0; r < M; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint4 v = lds[r * gpr + swizzle_granule(b * 8 + g)];
        s = __builtin_fmaf(sbyte_to_f32(q[g], 0), __builtin_bit_cast(float, v.x), s);
        s = __builtin_fmaf(sbyte_to_f32(q[g], 1), __builtin_bit_cast(float, v.y), s);
        s = __builtin_fmaf(sbyte_to_f32(q[g], 2), __builtin_bit_cast(float, v.z), s);
        s = __builtin_fmaf(sbyte_to_f32(q[g], 3), __builtin_bit_cast(float, v.w), s);
      }
      acc[r] = __builtin_fmaf(d, s, acc[r]);
    }
  }

#pragma unroll
  for (int r = 0; r < M; ++r) {
    float v = row16_sum(acc[r]);
    v += __shfl_xor(v, 16);  // join the two 16-lane halves of the row's 32 lanes
    if (j == r) y[(size_t)r * n + row] = v;
  }
}

__global__ __launch_bounds__(256) void q80_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                          const size_t nblocks) {
  const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t q[8];
  const float d = load_q8_0_block(w, b * kQ80BlockBytes, q);
  float4 *o = reinterpret_cast<float4 *>(out + b * 32);
#pragma unroll
  for (int g = 0; g < 8; ++g)
    o[g] = make_float4(d * sbyte_to_f32(q[g], 0), d * sbyte_to_f32(q[g], 1), d * sbyte_to_f32(q[g], 2),
                       d * sbyte_to_f32(q[g], 3));
}

template <int M>
int launch_m(const void *w, const float *x, float *y, int n, int k, hipStream_t s) {
  const size_t lds = (size_t)M * (size_t)k * 4;
  static LdsGrant granted;
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&q80_gemv_kernel<M>), lds, granted, "q80_gemv_kernel lds"))
    return QMV_ERR_HIP;
  const int rows_per_group = kWaves * kRowsPerWave;
  const unsigned grid = (unsigned)((n + rows_per_group - 1) / rows_per_group);
  return launch_kernel("q80_gemv_kernel", q80_gemv_kernel<M>, dim3(grid), dim3(kThreads), lds, s, w, x, y, n, k);
}

}  // namespace

int launch_q8_0_gemv(const void *w, const float *x, float *y, int m, int n, int k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (m) {
    case 1: return launch_m<1>(w, x, y, n, k, s);
    case 2: return launch_m<2>(w, x, y, n, k, s);
    case 3: return launch_m<3>(w, x, y, n, k, s);
    case 4: return launch_m<4>(w, x, y, n, k, s);
    default: return QMV_ERR_RANGE;
  }
}

int launch_dequant_q8_0(const void *w, float *out, int n, int k, void *stream) {
  const size_t nblocks = (size_t)n * (size_t)(k >> 5);
  const unsigned grid = (unsigned)((nblocks + 255) / 256);
  return launch_kernel("q80_dequant_kernel", q80_dequant_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), w, out,
                       nblocks);
}

}  // namespace qmv
