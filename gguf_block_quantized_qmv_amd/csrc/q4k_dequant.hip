// Q4_K dequantization to dense fp32 or bf16, and Q5_K and Q4_0 to fp32, gfx950.
//
// One thread per 16-byte quant granule (32 weights): granule g of a block holds
// quant bytes 16g..16g+15, i.e. chunk c = g / 2, weights 64c + 16(g%2) + 0..15 in
// the low nibbles (sub-block 2c) and 64c + 32 + 16(g%2) + 0..15 in the high
// nibbles (sub-block 2c + 1). Each weight is computed as fma(d*sc, q, -(dmin*m)):
// d*sc and dmin*m are exact in fp32 (11 x 6 significant bits) and d*sc*q is
// exact inside the fma, so the single rounding gives RN_fp32 of the exact value.
// The bf16 output rounds that fp32 value to nearest even.
#include "q4k_common.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void q4k_dequant_kernel(const uint8_t *__restrict__ w, void *__restrict__ out,
                                                          const size_t ngran) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= ngran) return;
  const size_t blk = t >> 3;
  const int g = (int)(t & 7);
  const int c = g >> 1;
  const uint8_t *bp = w + blk * kQ4KBlockBytes;
  const uint4 hdr = *reinterpret_cast<const uint4 *>(bp);
  const uint4 qv = *reinterpret_cast<const uint4 *>(bp + 16 + 16 * g);
  const uint32_t scm = unpack_scale_mins(hdr.y, hdr.z, hdr.w, scale_selectors(c));
  const float d = fp16_bits_to_f32(hdr.x & 0xFFFFu);
  const float dmin = fp16_bits_to_f32(hdr.x >> 16);
  const float ds0 = d * (float)(scm & 0xFFu), ds1 = d * (float)((scm >> 8) & 0xFFu);
  const float dm0 = dmin * (float)((scm >> 16) & 0xFFu), dm1 = dmin * (float)(scm >> 24);

  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
  float lo[16], hi[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t byte = (qw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    lo[i] = __builtin_fmaf(ds0, (float)(byte & 0xFu), -dm0);
    hi[i] = __builtin_fmaf(ds1, (float)(byte >> 4), -dm1);
  }
  const size_t base = blk * kQ4KBlockWeights + 64 * c + 16 * (g & 1);
  if constexpr (!BF16) {
    float4 *o_lo = reinterpret_cast<float4 *>(static_cast<float *>(out) + base);
    float4 *o_hi = reinterpret_cast<float4 *>(static_cast<float *>(out) + base + 32);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      o_lo[v] = make_float4(lo[4 * v], lo[4 * v + 1], lo[4 * v + 2], lo[4 * v + 3]);
      o_hi[v] = make_float4(hi[4 * v], hi[4 * v + 1], hi[4 * v + 2], hi[4 * v + 3]);
    }
  } else {
    uint4 *o_lo = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + base);
    uint4 *o_hi = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + base + 32);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint32_t pl[4], ph[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pl[e] = f32_to_bf16_rne(lo[8 * v + 2 * e]) | (f32_to_bf16_rne(lo[8 * v + 2 * e + 1]) << 16);
        ph[e] = f32_to_bf16_rne(hi[8 * v + 2 * e]) | (f32_to_bf16_rne(hi[8 * v + 2 * e + 1]) << 16);
      }
      o_lo[v] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      o_hi[v] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    }
  }
}

// Q5_K to fp32: one thread per 16-byte nibble granule, as above, with the fifth
// bit of weight 64c + 16(g%2) + i from bit 2c of high-plane byte 16(g%2) + i
// and of weight 64c + 32 + 16(g%2) + i from bit 2c + 1. d*sc*q (q <= 31) is
// still exact inside the fma, so the result is RN_fp32 of the exact weight.
__global__ __launch_bounds__(256) void q5k_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                          const size_t ngran) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= ngran) return;
  const size_t blk = t >> 3;
  const int g = (int)(t & 7);
  const int c = g >> 1;
  const uint8_t *bp = w + blk * kQ5KBlockBytes;
  const uint4 hdr = *reinterpret_cast<const uint4 *>(bp);
  const uint4 hv = *reinterpret_cast<const uint4 *>(bp + 16 + 16 * (g & 1));
  const uint4 qv = *reinterpret_cast<const uint4 *>(bp + 48 + 16 * g);
  const uint32_t scm = unpack_scale_mins(hdr.y, hdr.z, hdr.w, scale_selectors(c));
  const float d = fp16_bits_to_f32(hdr.x & 0xFFFFu);
  const float dmin = fp16_bits_to_f32(hdr.x >> 16);
  const float ds0 = d * (float)(scm & 0xFFu), ds1 = d * (float)((scm >> 8) & 0xFFu);
  const float dm0 = dmin * (float)((scm >> 16) & 0xFFu), dm1 = dmin * (float)(scm >> 24);

  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
  const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
  float lo[16], hi[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t byte = (qw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    const uint32_t hbits = (hw[i >> 2] >> (8 * (i & 3) + 2 * c)) & 3u;
    lo[i] = __builtin_fmaf(ds0, (float)((byte & 0xFu) | ((hbits & 1u) << 4)), -dm0);
    hi[i] = __builtin_fmaf(ds1, (float)((byte >> 4) | ((hbits >> 1) << 4)), -dm1);
  }
  const size_t base = blk * kQ4KBlockWeights + 64 * c + 16 * (g & 1);
  float4 *o_lo = reinterpret_cast<float4 *>(out + base);
  float4 *o_hi = reinterpret_cast<float4 *>(out + base + 32);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    o_lo[v] = make_float4(lo[4 * v], lo[4 * v + 1], lo[4 * v + 2], lo[4 * v + 3]);
    o_hi[v] = make_float4(hi[4 * v], hi[4 * v + 1], hi[4 * v + 2], hi[4 * v + 3]);
  }
}

// Q4_0 to fp32: one thread per 18-byte block, read as nine 16-bit halves (the
// blocks are only 2-byte aligned). Byte i holds weight i (low nibble) and
// weight 16 + i (high nibble); d (q - 8) is exact in fp32.
__global__ __launch_bounds__(256) void q40_dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                          const size_t nblocks) {
  const size_t b = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const uint16_t *p = reinterpret_cast<const uint16_t *>(w + b * 18);
  const float d = fp16_bits_to_f32(p[0]);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = p[1 + i];  // quant bytes 2i (low half) and 2i + 1
    v[2 * i] = d * (float)((int)(h & 0xFu) - 8);
    v[2 * i + 1] = d * (float)((int)((h >> 8) & 0xFu) - 8);
    v[16 + 2 * i] = d * (float)((int)((h >> 4) & 0xFu) - 8);
    v[16 + 2 * i + 1] = d * (float)((int)((h >> 12) & 0xFu) - 8);
  }
  float4 *o = reinterpret_cast<float4 *>(out + b * 32);
#pragma unroll
  for (int g = 0; g < 8; ++g) o[g] = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
}

}  // namespace

int launch_dequant_q5_k(const void *w, float *out, int n, int k, void *stream) {
  const size_t ngran = (size_t)n * (size_t)(k >> 8) * 8;
  const unsigned grid = (unsigned)((ngran + 255) / 256);
  return launch_kernel("q5k_dequant_kernel", q5k_dequant_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(w), out, ngran);
}

int launch_dequant_q4_k(const void *w, void *out, bool bf16, int n, int k, void *stream) {
  const size_t ngran = (size_t)n * (size_t)(k >> 8) * 8;
  const unsigned grid = (unsigned)((ngran + 255) / 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return bf16 ? launch_kernel("q4k_dequant_kernel", q4k_dequant_kernel<true>, dim3(grid), dim3(256), 0, s, w, out, ngran)
              : launch_kernel("q4k_dequant_kernel", q4k_dequant_kernel<false>, dim3(grid), dim3(256), 0, s, w, out, ngran);
}

int launch_dequant_q4_0(const void *w, float *out, int n, int k, void *stream) {
  const size_t nblocks = (size_t)n * (size_t)(k >> 5);
  const unsigned grid = (unsigned)((nblocks + 255) / 256);
  return launch_kernel("q40_dequant_kernel", q40_dequant_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(w), out, nblocks);
}

}  // namespace qmv
