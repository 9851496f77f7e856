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
// Work mapping: G lanes per W row (16, or 32 for long rows), 256 / G rows per
// workgroup; lane l of a row takes the row's sub-blocks l, l + G, ... Loads
// run kDepth units ahead through a register ring; they are unconditional
// (units past the row re-read the row's first sub-block with a zero scale) and
// the unit loop is unrolled by kDepth, so every wait is exact. Row r of the
// output is computed by the same instruction sequence for every M.
#include "qmv_device.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

constexpr int kIQ4XSBlockBytes = 136;
constexpr int kThreads = 256;
constexpr int kDepth = 4;          // units of loads in flight per lane
constexpr int kTableEntries = 256;  // LDS table: one bf16 pair per index byte

// The format's 16 grid values, packed as signed bytes (index 4w + b in byte b of word w).
constexpr uint32_t kGrid0 = 0xBFAD9881u;  // -127, -104,  -83,  -65
constexpr uint32_t kGrid1 = 0xF6EADDCFu;  //  -49,  -35,  -22,  -10
constexpr uint32_t kGrid2 = 0x26190D01u;  //    1,   13,   25,   38
constexpr uint32_t kGrid3 = 0x71594535u;  //   53,   69,   89,  113

__device__ __forceinline__ uint32_t grid_bf16(uint32_t idx) {
  const uint32_t w = idx < 4 ? kGrid0 : idx < 8 ? kGrid1 : idx < 12 ? kGrid2 : kGrid3;
  const int v = (int)(int8_t)(uint8_t)(w >> (8 * (idx & 3)));
  return __builtin_bit_cast(uint32_t, (float)v) >> 16;   // exact: |v| < 2^8
}

// x staging: row r's sub-block s lives at granule r * row_gran + 4 s + (s >> 2)
// (one pad granule after every 4 sub-blocks: the 16 lanes of a row reading
// granule q of 16 consecutive sub-blocks hit 16 distinct bank groups).
__device__ __forceinline__ int x_slot(int s) { return 4 * s + (s >> 2); }
__host__ __device__ constexpr int row_granules(int nsub) { return 4 * nsub + nsub / 4; }

// Pair-interleave one 32-value sub-block: in granules g0..g3 hold x[0..31]; out
// granule t holds the pairs (x[4t + e], x[16 + 4t + e]) for e < 4.
__device__ __forceinline__ void interleave(const uint4 g0, const uint4 g1, const uint4 g2, const uint4 g3,
                                           uint4 (&o)[4]) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;   // (b.lo16, a.lo16), (b.hi16, a.hi16)
  o[0] = make_uint4(__builtin_amdgcn_perm(g2.x, g0.x, kLo), __builtin_amdgcn_perm(g2.x, g0.x, kHi),
                    __builtin_amdgcn_perm(g2.y, g0.y, kLo), __builtin_amdgcn_perm(g2.y, g0.y, kHi));
  o[1] = make_uint4(__builtin_amdgcn_perm(g2.z, g0.z, kLo), __builtin_amdgcn_perm(g2.z, g0.z, kHi),
                    __builtin_amdgcn_perm(g2.w, g0.w, kLo), __builtin_amdgcn_perm(g2.w, g0.w, kHi));
  o[2] = make_uint4(__builtin_amdgcn_perm(g3.x, g1.x, kLo), __builtin_amdgcn_perm(g3.x, g1.x, kHi),
                    __builtin_amdgcn_perm(g3.y, g1.y, kLo), __builtin_amdgcn_perm(g3.y, g1.y, kHi));
  o[3] = make_uint4(__builtin_amdgcn_perm(g3.z, g1.z, kLo), __builtin_amdgcn_perm(g3.z, g1.z, kHi),
                    __builtin_amdgcn_perm(g3.w, g1.w, kLo), __builtin_amdgcn_perm(g3.w, g1.w, kHi));
}

constexpr int kStageSub = 2;   // sub-blocks per thread per staging round trip

// One unit's global data for a lane: the block's 8 header bytes and the
// sub-block's 16 index bytes (blocks are only 8-byte aligned: 8-byte loads).
struct Unit {
  uint2 hdr, q0, q1;
};

__device__ __forceinline__ void load_unit(const uint8_t *__restrict__ row_ptr, const int u, Unit &r) {
  const uint8_t *bp = row_ptr + (size_t)(u >> 3) * kIQ4XSBlockBytes;
  const uint8_t *qp = bp + 8 + 16 * (u & 7);
  r.hdr = *reinterpret_cast<const uint2 *>(bp);
  r.q0 = *reinterpret_cast<const uint2 *>(qp);
  r.q1 = *reinterpret_cast<const uint2 *>(qp + 8);
}

// dot2 of the four table entries of index word w with four activation pairs.
__device__ __forceinline__ float word_dot(const uint32_t *__restrict__ tbl, const uint32_t w, const uint4 xp,
                                          float s) {
  const bf16x2 e0 = __builtin_bit_cast(bf16x2, tbl[w & 0xFF]);
  const bf16x2 e1 = __builtin_bit_cast(bf16x2, tbl[(w >> 8) & 0xFF]);
  const bf16x2 e2 = __builtin_bit_cast(bf16x2, tbl[(w >> 16) & 0xFF]);
  const bf16x2 e3 = __builtin_bit_cast(bf16x2, tbl[w >> 24]);
  s = __builtin_amdgcn_fdot2_f32_bf16(e0, __builtin_bit_cast(bf16x2, xp.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(e1, __builtin_bit_cast(bf16x2, xp.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(e2, __builtin_bit_cast(bf16x2, xp.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(e3, __builtin_bit_cast(bf16x2, xp.w), s, false);
  return s;
}

template <int M, int G>
__global__ __launch_bounds__(kThreads) void iq4xs_gemv_kernel(const uint8_t *__restrict__ w,
                                                              const uint16_t *__restrict__ x,
                                                              float *__restrict__ y, const int n, const int k) {
  extern __shared__ uint4 lds[];
  uint32_t *tbl = reinterpret_cast<uint32_t *>(lds);
  uint4 *xs = lds + kTableEntries / 4;
  const int tid = threadIdx.x;
  const int nblk = k >> 8, nsub = nblk * 8, rg = row_granules(nsub);
  const int row = blockIdx.x * (kThreads / G) + tid / G;
  const int l = tid % G;
  const uint8_t *row_ptr = w + (size_t)(row < n ? row : 0) * (size_t)nblk * kIQ4XSBlockBytes;
  const int nunits = (nsub + G - 1) / G;              // units of this lane, the last may be past the row
  const int nslots = (nunits + kDepth - 1) / kDepth * kDepth;

  // the first weights are requested before anything else
  Unit ring[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    const int u = l + G * d;
    load_unit(row_ptr, u < nsub && d < nunits ? u : 0, ring[d]);
  }

  // table and activations
  tbl[tid] = grid_bf16((uint32_t)tid & 15u) | (grid_bf16((uint32_t)tid >> 4) << 16);
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const int total = M * nsub;   // sub-blocks to stage
  for (int base = 0; base < total; base += kStageSub * kThreads) {
    uint4 g[kStageSub][4];
#pragma unroll
    for (int i = 0; i < kStageSub; ++i) {
      const int t0 = base + tid + i * kThreads, t = t0 < total ? t0 : 0;   // a clamped lane rewrites sub-block 0
      const int r = t / nsub, s = t - r * nsub;
#pragma unroll
      for (int q = 0; q < 4; ++q) g[i][q] = xg[(size_t)r * (k >> 3) + 4 * s + q];
    }
#pragma unroll
    for (int i = 0; i < kStageSub; ++i) {
      const int t0 = base + tid + i * kThreads, t = t0 < total ? t0 : 0;
      const int r = t / nsub, s = t - r * nsub;
      uint4 o[4];
      interleave(g[i][0], g[i][1], g[i][2], g[i][3], o);
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[r * rg + x_slot(s) + q] = o[q];
    }
  }
  __syncthreads();

  float acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = 0.0f;
  for (int t0 = 0; t0 < nslots; t0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int t = t0 + d, u = l + G * t;
      const bool live = u < nsub;
      const Unit cur = ring[d];
      // refill the slot kDepth units ahead (clamped, never guarded)
      {
        const int un = u + G * kDepth;
        load_unit(row_ptr, un < nsub ? un : 0, ring[d]);
      }
      const int j = u & 7;
      const uint32_t ls = ((cur.hdr.y >> (4 * j)) & 15u) | (((cur.hdr.x >> (16 + 2 * j)) & 3u) << 4);
      const float dl = live ? fp16_bits_to_f32(cur.hdr.x & 0xFFFFu) * (float)((int)ls - 32) : 0.0f;
      const int s = live ? u : 0;
#pragma unroll
      for (int r = 0; r < M; ++r) {
        const uint4 *xp = xs + r * rg + x_slot(s);
        float s0 = 0.0f, s1 = 0.0f;
        s0 = word_dot(tbl, cur.q0.x, xp[0], s0);
        s1 = word_dot(tbl, cur.q0.y, xp[1], s1);
        s0 = word_dot(tbl, cur.q1.x, xp[2], s0);
        s1 = word_dot(tbl, cur.q1.y, xp[3], s1);
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
  const uint32_t ls = ((hdr.y >> (4 * j)) & 15u) | (((hdr.x >> (16 + 2 * j)) & 3u) << 4);
  const float dl = fp16_bits_to_f32(hdr.x & 0xFFFFu) * (float)((int)ls - 32);
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

size_t gemv_lds(int m, int k) {
  return (size_t)kTableEntries * 4 + (size_t)m * row_granules((k >> 8) * 8) * 16;
}

template <int M, int G>
int launch_mg(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t s) {
  static std::atomic<size_t> granted{0};
  const size_t lds = gemv_lds(M, k);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&iq4xs_gemv_kernel<M, G>), lds, granted,
                        "iq4xs_gemv_kernel lds"))
    return QMV_ERR_HIP;
  const int rows = kThreads / G;
  return launch_kernel("iq4xs_gemv_kernel", iq4xs_gemv_kernel<M, G>, dim3((unsigned)((n + rows - 1) / rows)),
                       dim3(kThreads), lds, s, static_cast<const uint8_t *>(w), x, y, n, k);
}

template <int M>
int launch_m(const void *w, const uint16_t *x, float *y, int n, int k, hipStream_t s) {
  // long rows take 32 lanes (more independent loads per row, fewer rows per workgroup)
  return k > 8192 ? launch_mg<M, 32>(w, x, y, n, k, s) : launch_mg<M, 16>(w, x, y, n, k, s);
}

}  // namespace

bool iq4xs_fits_lds(int m, int k) { return gemv_lds(m, k) <= (size_t)QMV_LDS_X_BYTES; }

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
