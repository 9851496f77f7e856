// Prefill-sized Q4_K GEMM Y = X W^T on bf16 matrix cores, gfx950.
//
// Prompt processing ahead of decode (the time-to-first-token rows of the memra
// summary page's performance table) multiplies the same quantized weights by
// many activation rows at once, which makes it a dense contraction: the weights
// are dequantized into bf16 tiles in LDS and fed to v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.
//
// Tiling. A 1024-thread workgroup owns a 256 (rows of X) x 128 (rows of W) tile
// of Y. K advances 64 at a time -- one 64-weight chunk of each W row's
// super-block -- through two LDS stages of 48 KiB (X tile + W tile, rows of
// eight 16-byte granules, swizzled so that no 16-byte access conflicts on the
// LDS banks). The waves split into two kinds. Eight consumers each own a 64 x 64
// part, four 32x32 MFMA tiles (64 fp32 accumulators per lane), and only read
// fragments and issue matrix instructions. Eight producers run kDepth steps of
// global loads ahead through a ring of registers: while the consumers work on
// stage s, the producers write step s + 1 (loaded kDepth - 1 steps earlier) into
// the other stage, dequantizing W, and send the loads of step s + 1 + kDepth.
// Each SIMD runs two waves of each kind, so the dequantization issues while the
// other waves' matrix instructions execute. The 256-row tile writes a quarter
// fewer LDS bytes per flop than 128 x 128 (16-byte LDS writes run at about a
// third of the read rate) and dequantizes each W chunk once per 256 rows of X. Every load is unconditional (steps
// past K reload the last step) and the step loop is unrolled by kDepth, which
// divides the step count because K is a multiple of 256, so each wait covers
// exactly the slot being consumed.
//
// Dequantization matches the bf16 dequant entry point bit for bit: each weight
// is fma(d*sc, q, -(dmin*m)) (one rounding of the exact value to fp32), then
// rounded to nearest-even bf16 by v_cvt_pk_bf16_f32.
#include "q4k_common.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int BK = addr::kPrefillBK;
constexpr int kThreads = addr::kPrefillHalf;

// Tile shape: BM rows of X x BN rows of W per workgroup, four consumer waves of
// (BM / WM_WAVES) x (BN / WN_WAVES), DEPTH steps of global loads in flight;
// kThreads is the size of each kind's half of the workgroup.
template <int BM_, int BN_, int DEPTH_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, kDepth = DEPTH_;
  static constexpr int kWaves = kThreads / 64;                      // consumer (and producer) waves
  static constexpr int WN_WAVES = BN / 64, WM_WAVES = kWaves / WN_WAVES;   // wave tile 64 x 64
  static constexpr int kXGran = BM * 8, kWGran = BN * 8, kStageGran = kXGran + kWGran;
  static constexpr size_t kLdsBytes = 2 * (size_t)kStageGran * 16;
  static constexpr int kXPerThread = kXGran / kThreads;
  static constexpr int kWThreadsPerRow = kThreads / BN;          // 2 or 4
  static constexpr int kQBytes = 32 / kWThreadsPerRow;            // quant bytes per thread: 16 or 8
  static_assert(WM_WAVES * 64 == BM && WN_WAVES * 64 == BN, "one 64x64 wave tile per consumer wave");
};

// Granule g (8 bf16 of K) of tile row r sits at slot (g + f(r)) & 7 of the
// row, with f(r) = 2 ((r >> 2) & 3) + 4 (r & 1) + ((r >> 1) & 1) mod 8.
// Measured on gfx950 (ds_read_b128 / ds_write_b128 with a bank-conflict
// counter): a 16-byte read serves 16 lanes per cycle from 16 groups of 16 B
// (group = slot mod 16), a 16-byte write 8 lanes per cycle from 8 groups
// (slot mod 8). A row is 8 slots, so for reads rows of one parity share
// their 8 groups. The layout keeps every access of the kernel conflict-free:
//  * MFMA fragment reads (16 consecutive rows from a multiple of 16, one
//    granule): the 8 even rows take f = 2q + {0, 1} (q = 0..3), all 8
//    values, and the odd rows the same plus 4;
//  * X tile writes (one row per 8 lanes, all 8 granules): distinct within a
//    row;
//  * W tile writes (8 lanes: rows 4k .. 4k + 3, granules g and g + 2): the
//    four rows take f in {2q, 2q + 4, 2q + 1, 2q + 5}, and f and f + 2 cover
//    all 8 slots.
// (The layout before this one paired rows 2i and 2i + 1 on the same f, a
// 2-way conflict on every W write.)
__device__ __forceinline__ int tslot(int r, int g) {
  const int f = 2 * ((r >> 2) & 3) + 4 * (r & 1) + ((r >> 1) & 1);
  return r * 8 + ((g + f) & 7);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// One step's global data for this thread: its X granules, and for W row
// n0 + tid / kWThreadsPerRow the block header and kQBytes quant bytes of chunk s % 4.
template <class C>
struct StepRegs {
  uint4 x[C::kXPerThread];
  uint4 hdr;
  uint32_t q[C::kQBytes / 4];
};

// Rows past M read row 0 of X and rows past N row 0 of W: they only feed
// outputs that are never stored. Steps past K read the last step. X granules
// are addressed by a 32-bit granule index: the argument checks bound the
// M * K / 8 granules of X to 2^32 - 1.
template <class C>
__device__ __forceinline__ void load_step(const int pt, const uint4 *__restrict__ xg, const int m0, const int M,
                                          const int gpr, const uint8_t *__restrict__ w_rowp, const int nsteps, int s,
                                          StepRegs<C> &r) {
  s = addr::prefill_clamp(s, nsteps);
#pragma unroll
  for (int i = 0; i < C::kXPerThread; ++i) r.x[i] = xg[addr::prefill_x_granule(pt, i, m0, M, gpr, s)];
  const uint8_t *bp = w_rowp + addr::prefill_w_step(s);
  r.hdr = *reinterpret_cast<const uint4 *>(bp + addr::prefill_w_window(s, pt, C::kWThreadsPerRow, 0).off);
  const uint8_t *qp = bp + addr::prefill_w_window(s, pt, C::kWThreadsPerRow, 1).off;   // C::kQBytes long
  if constexpr (C::kQBytes == 16) {
    const uint4 v = *reinterpret_cast<const uint4 *>(qp);
    r.q[0] = v.x; r.q[1] = v.y; r.q[2] = v.z; r.q[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(qp);
    r.q[0] = v.x; r.q[1] = v.y;
  }
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

// Write a step into a stage: X granules as loaded, the W part-chunk dequantized to bf16.
template <class C>
__device__ __forceinline__ void store_step(const int pt, uint4 *__restrict__ xt, uint4 *__restrict__ wt, const int s,
                                           const StepRegs<C> &r) {
#pragma unroll
  for (int i = 0; i < C::kXPerThread; ++i) {
    const int g = pt + kThreads * i;
    const uint4 v = r.x[i];
    xt[tslot(g >> 3, g & 7)] = make_uint4(v.x, v.y, v.z, v.w);   // element-wise: keeps the ring in registers
  }
  const ChunkScales cs = chunk_scales(r.hdr, scale_selectors(s & 3));
  constexpr int kPairs = C::kQBytes / 8;   // word pairs: 8 low and 8 high weights each
  uint32_t pl[4 * kPairs], ph[4 * kPairs];
#pragma unroll
  for (int h = 0; h < kPairs; ++h) {
    float lo[8], hi[8];
    nibbles_f32(r.q[2 * h] & 0x0F0F0F0Fu, r.q[2 * h + 1] & 0x0F0F0F0Fu, lo);
    nibbles_f32((r.q[2 * h] >> 4) & 0x0F0F0F0Fu, (r.q[2 * h + 1] >> 4) & 0x0F0F0F0Fu, hi);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pl[4 * h + e] = pack_bf16x2(__builtin_fmaf(cs.a0, lo[2 * e], -cs.b0), __builtin_fmaf(cs.a0, lo[2 * e + 1], -cs.b0));
      ph[4 * h + e] = pack_bf16x2(__builtin_fmaf(cs.a1, hi[2 * e], -cs.b1), __builtin_fmaf(cs.a1, hi[2 * e + 1], -cs.b1));
    }
  }
  // this thread's weights: local k p*kQBytes .. + kQBytes - 1 (sub-block 2c) and 32 + the same (2c + 1)
  const int row = pt / C::kWThreadsPerRow, p = pt % C::kWThreadsPerRow;
  constexpr int kG = C::kQBytes / 8;   // granules per sub-block part
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    wt[tslot(row, kG * p + h)] = make_uint4(pl[4 * h], pl[4 * h + 1], pl[4 * h + 2], pl[4 * h + 3]);
    wt[tslot(row, 4 + kG * p + h)] = make_uint4(ph[4 * h], ph[4 * h + 1], ph[4 * h + 2], ph[4 * h + 3]);
  }
}

// MFMA fragments of K slice kk (16 values) for a wave's 64 x 64 tile: lane l
// supplies row l % 32 and K granule l / 32 of each 32 x 16 operand.
__device__ __forceinline__ void read_frags(const uint4 *__restrict__ xt, const uint4 *__restrict__ wt, const int wm,
                                           const int wn, const int kk, bf16x8 (&fa)[2], bf16x8 (&fb)[2]) {
  const int lane = threadIdx.x & 63, frow = lane & 31, fg = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) fa[i] = __builtin_bit_cast(bf16x8, xt[tslot(wm + 32 * i + frow, 2 * kk + fg)]);
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[j] = __builtin_bit_cast(bf16x8, wt[tslot(wn + 32 * j + frow, 2 * kk + fg)]);
}

// Tile t as (mt, nt): addr::tile_of.

// Wave-specialised form: 2 kWaves waves per workgroup. Waves kWaves.. produce --
// they load X and the Q4_K blocks kDepth steps ahead, dequantize W and write the
// next LDS stage -- while waves 0 .. kWaves - 1 consume the current stage with
// MFMAs (a 64 x 64 part each). Each SIMD runs waves of both kinds, so the
// dequantization VALU work issues while the other waves' matrix instructions
// execute. One barrier per step hands a stage from the producers to the
// consumers and back; both kinds pass the same number of barriers.
//
// Blocks below t_main each compute a whole tile (tile = block) into Y. The
// r_tiles tiles after them, when the tile count does not divide over the
// workgroups the device holds at once, are split along K: block t_main + s *
// r_tiles + r computes part s of tile t_main + r -- a run of whole 256-value
// K blocks -- and stores its BM x BN sums to that part's slot of `part`;
// q4k_prefill_reduce_kernel adds the parts in order afterwards.
// One workgroup (four waves per SIMD) per CU: at most 128 VGPRs per lane.
template <class C>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(4))) void q4k_prefill_ws_kernel(
    const uint8_t *__restrict__ w, const uint16_t *__restrict__ x, float *__restrict__ y, float *__restrict__ part,
    const int M, const int N, const int K, const int t_main, const int r_tiles, const int splits) {
  constexpr int BM = C::BM, BN = C::BN, kDepth = C::kDepth;
  extern __shared__ uint4 lds[];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int m_tiles = (M + BM - 1) / BM, n_tiles = (N + BN - 1) / BN;
  const int blk = (int)blockIdx.x;
  // this block's tile and its K steps [s_begin, s_begin + nsteps), both
  // multiples of 4 (whole K blocks), so of kDepth in {2, 4}
  const addr::PrefillWork wk = addr::prefill_work(blk, K, t_main, r_tiles, splits);
  const int tile = wk.tile, s_begin = wk.s_begin, nsteps = wk.nsteps, slot = wk.slot;
  int mt, nt;
  addr::tile_of(tile, m_tiles, n_tiles, mt, nt);
  const int n0 = nt * BN, m0 = mt * BM;

  if (wave >= C::kWaves) {
    const int pt = tid - kThreads;
    const int nblk = K >> 8;
    const uint8_t *w_rowp = w + addr::prefill_w_row(n0, N, K, s_begin, pt, C::kWThreadsPerRow);
    const uint4 *xg = reinterpret_cast<const uint4 *>(x) + s_begin * 8;   // step s_begin of row 0
    const int gpr = K >> 3;
    StepRegs<C> ring[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) load_step<C>(pt, xg, m0, M, gpr, w_rowp, nsteps, u, ring[u]);
    store_step<C>(pt, lds, lds + C::kXGran, 0, ring[0]);
    load_step<C>(pt, xg, m0, M, gpr, w_rowp, nsteps, kDepth, ring[0]);
    __syncthreads();
    for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        // step s + 1 into the stage the consumers are not reading (past the last
        // step a copy of the last step, which nobody reads), then refill its slot
        const int s = s0 + u, un = (u + 1) % kDepth;
        uint4 *nx = lds + ((u + 1) & 1) * C::kStageGran;
        store_step<C>(pt, nx, nx + C::kXGran, s + 1, ring[un]);
        load_step<C>(pt, xg, m0, M, gpr, w_rowp, nsteps, s + 1 + kDepth, ring[un]);
        __syncthreads();
      }
    }
    return;
  }

  const int lane = tid & 63;
  const int wm = (wave / C::WN_WAVES) * 64, wn = (wave % C::WN_WAVES) * 64;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  __syncthreads();
  const int frow = lane & 31, fg = lane >> 5;
  bf16x8 a[2][2], b[2][2];
  read_frags(lds, lds + C::kXGran, wm, wn, 0, a[0], b[0]);
  for (int s0 = 0; s0 < nsteps; s0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const uint4 *xt = lds + (u & 1) * C::kStageGran;
      const uint4 *wt = xt + C::kXGran;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) read_frags(xt, wt, wm, wn, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
      const uint4 *nx = lds + ((u + 1) & 1) * C::kStageGran;
      read_frags(nx, nx + C::kXGran, wm, wn, 0, a[0], b[0]);
    }
  }
  // 32x32 accumulator layout: lane l holds column l % 32 and, in register
  // 4 q + e, row 8 q + 4 (l / 32) + e
  if (slot >= 0) {
    float *pt = part + (size_t)slot * BM * BN;   // the part's 128 x 128 sums, row-major
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pt[(size_t)(wm + 32 * i + 8 * q + 4 * fg + e) * BN + wn + 32 * j + frow] = acc[i][j][4 * q + e];
    return;
  }
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

// Y of the K-split tiles: each thread sums four adjacent values of one tile
// row over the parts, in part order (so in K order), and stores those inside Y.
template <class C>
__global__ __launch_bounds__(256) void q4k_prefill_reduce_kernel(const float *__restrict__ part, float *__restrict__ y,
                                                                 const int M, const int N, const int t_main,
                                                                 const int r_tiles, const int splits) {
  constexpr int BM = C::BM, BN = C::BN, kQuads = BM * BN / 4;
  const int idx = (int)(blockIdx.x * 256 + threadIdx.x);
  const int r = idx / kQuads, within = idx % kQuads;
  if (r >= r_tiles) return;
  const int row = within / (BN / 4), c4 = within % (BN / 4);
  int mt, nt;
  addr::tile_of(t_main + r, (M + BM - 1) / BM, (N + BN - 1) / BN, mt, nt);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int sp = 0; sp < splits; ++sp) {
    const float4 v = reinterpret_cast<const float4 *>(part + (size_t)(sp * r_tiles + r) * BM * BN)[within];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const int grow = mt * BM + row, gcol = nt * BN + 4 * c4;
  if (grow >= M) return;
  float *yr = y + (size_t)grow * N;
  if (gcol < N) yr[gcol] = acc.x;
  if (gcol + 1 < N) yr[gcol + 1] = acc.y;
  if (gcol + 2 < N) yr[gcol + 2] = acc.z;
  if (gcol + 3 < N) yr[gcol + 3] = acc.w;
}

using PrefillCfg = Cfg<layout::kPrefillTileM, layout::kPrefillTileN, 2>;

}  // namespace

int launch_q4_k_prefill(const void *w, const uint16_t *x, float *y, void *ws, int m, int n, int k, void *stream) {
  using C = PrefillCfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  static LdsGrant granted;
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&q4k_prefill_ws_kernel<C>), C::kLdsBytes, granted,
                        "q4k_prefill_ws_kernel lds"))
    return QMV_ERR_HIP;
  // the checks have bounded the tiles and required the plan's workspace
  const layout::PrefillPlan p = layout::prefill_plan(m, n, k);
  float *part = static_cast<float *>(ws);
  const int blocks = p.t_main + p.r_tiles * p.splits;
  int rc = launch_kernel("q4k_prefill_ws_kernel", q4k_prefill_ws_kernel<C>, dim3((unsigned)blocks),
                         dim3(2 * kThreads), C::kLdsBytes, s, w, x, y, part, m, n, k, p.t_main, p.r_tiles, p.splits);
  if (rc || p.splits == 0) return rc;
  const int threads = p.r_tiles * (C::BM * C::BN / 4);
  return launch_kernel("q4k_prefill_reduce_kernel", q4k_prefill_reduce_kernel<C>, dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, static_cast<const float *>(part), y, m, n, p.t_main, p.r_tiles, p.splits);
}

}  // namespace qmv
