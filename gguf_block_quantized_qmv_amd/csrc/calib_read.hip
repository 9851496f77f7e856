// Streaming-read calibration: the HBM read rate a plain kernel reaches on the
// same buffers the GEMVs stream, measured beside them. It is the achievable
// ceiling the GEMV rates are read against (the roofline itself stays the
// 8 TB/s nominal peak).
//
// Thread t of the grid reads granules t, t + S, t + 2S, ... (S = the grid's
// thread count), so a wave's loads are 1 KiB coalesced runs, and keeps D of
// them in flight through a ring of registers: every load is unconditional (an
// index past the end re-reads the last granule, whose value is not used), so
// each step waits for exactly its own ring slot. NT: non-temporal loads (the
// lines are not kept for reuse). The granules are folded with
// XOR and each workgroup writes the XOR of its threads to sink[blockIdx.x], so
// the result is checkable against a host XOR of the same bytes.
#include "qmv_device.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

constexpr int kReadThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 read16(const uint4 *p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  return *p;
}

template <int D, bool NT>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *__restrict__ p, const size_t n16,
                                                                   uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  const size_t i0 = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  const size_t its = i0 < n16 ? (n16 - 1 - i0) / stride + 1 : 0;   // granules of this thread
  const size_t last = n16 - 1;
  uint4 v[D];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    const size_t j = i0 + (size_t)u * stride;
    v[u] = read16<NT>(p + (j < last ? j : last));
  }
  uint32_t acc = 0;
  for (size_t it = 0; it < its; it += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (it + u < its) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      const size_t j = i0 + (it + u + D) * stride;
      v[u] = read16<NT>(p + (j < last ? j : last));
    }
  }
  // workgroup XOR: within the wave, then the four waves through LDS
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

template <bool NT>
int launch_nt(const uint4 *q, size_t n16, uint32_t *sink, int grid, int depth, hipStream_t s) {
  switch (depth) {
    case 1: return launch_kernel("stream_read_kernel", stream_read_kernel<1, NT>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, q, n16, sink);
    case 2: return launch_kernel("stream_read_kernel", stream_read_kernel<2, NT>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, q, n16, sink);
    case 4: return launch_kernel("stream_read_kernel", stream_read_kernel<4, NT>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, q, n16, sink);
    default: return launch_kernel("stream_read_kernel", stream_read_kernel<8, NT>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, q, n16, sink);
  }
}

}  // namespace

int launch_stream_read(const void *p, size_t bytes, uint32_t *sink, int grid, int depth, int nontemporal, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint4 *q = static_cast<const uint4 *>(p);
  const size_t n16 = bytes / 16;
  return nontemporal ? launch_nt<true>(q, n16, sink, grid, depth, s) : launch_nt<false>(q, n16, sink, grid, depth, s);
}

}  // namespace qmv
