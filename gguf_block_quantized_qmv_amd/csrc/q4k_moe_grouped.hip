// Routed-expert MoE over a prompt's tokens as grouped products on the matrix
// cores (Q4_K experts), gfx950.
//
// Launches, in order on one stream:
//  1. route:   per token, the top-k logits (ties to the lower id) and the
//              softmax over them (the decode form's routing, one wave a token);
//  2. group:   per expert, how many (token, rank) pairs chose it, how many
//              chose a lower expert, and its pairs in token order: the pair
//              list, sorted by expert then token;
//  3. chunks:  each expert's pairs cut into chunks of 16; the (expert, chunk)
//              list (and a list of chunks of 32 for the wide gate/up form);
//  4. gate/up: per (64 TPW rows of W_gate and W_up, chunk), each wave owning
//              TPW tiles of 16 rows over all of K: the 16 gathered
//              tokens' activations times each tile with one
//              v_mfma_f32_16x16x32_bf16 per 32-weight sub-block and matrix
//              (A = the tokens' activations, B = the quants as exact bf16
//              integers), per sub-block acc += (d sc) D - (dmin m) X; then
//              h = silu(g) u in fp32 per pair. From 2048 pairs, with 32
//              rows of x fitting in LDS, chunks of 32 pairs instead: eight
//              waves, two MFMA row blocks per converted weight fragment;
//  5. down:    per (64 TPW rows of W_down, chunk): the same with A = h split
//              into three bf16 parts (h_hi = bf16(h), h_mi = bf16(h - h_hi),
//              h_lo = bf16(h - h_hi - h_mi), about 24 bits of h), three
//              MFMAs per sub-block, z per pair;
//  6. combine: y_t = sum over ranks j of w_tj z_tj, in rank order.
// Each expert's weights are read once per chunk of 16 of its tokens. Every
// step has a fixed order, so results are bitwise reproducible.
//
// MFMA lane layout (16x16x32 bf16): lane l supplies A row l % 16 and B column
// l % 16 with k = 8 (l / 16) .. + 7, and holds D[4 (l / 16) + e][l % 16] in
// register e. Lane group g = l / 16 takes positions 8g .. 8g + 7 of every
// sub-block: the low and high nibbles of quant bytes 32c + 8g .. + 7 of chunk c.
#include "moe_routing.h"
#include "q4k_common.h"
#include "qmv_addr.h"
#include "qmv_internal.h"
#include "../../include/qmv.h"

namespace qmv {
namespace {

using moe::kTopK;
using moe::Logits;
using moe::load_logits;
using moe::route_token;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = layout::kGroupChunk;   // pairs per chunk (the MFMA's M)
constexpr int kTile = addr::kGroupTile;    // weight rows per tile (the MFMA's N)
constexpr int kWv = 4;       // waves per workgroup; they split the super-blocks
constexpr int kThr = 64 * kWv;


// Eight nibbles (bytes 0..3 of lo, then of hi) as eight exact bf16 integers.
__device__ __forceinline__ bf16x8 nibbles8(const uint32_t lo, const uint32_t hi) {
  const bf16x2 a = nibbles_to_bf16x2<false>(lo), b = nibbles_to_bf16x2<true>(lo);
  const bf16x2 c = nibbles_to_bf16x2<false>(hi), d = nibbles_to_bf16x2<true>(hi);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---------------------------------------------------------------- 1. route

__global__ __launch_bounds__(kThr) void g_route_kernel(const float *__restrict__ logits, int *__restrict__ ids,
                                                        float *__restrict__ wts, int32_t *__restrict__ topk_ids,
                                                        float *__restrict__ topk_w, const int T, const int E,
                                                        const int K) {
  __shared__ int sid[kWv][kTopK];
  __shared__ float swt[kWv][kTopK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * kWv + wave;
  const Logits lg = load_logits(logits, t < T ? t : T - 1, E);
  route_token(lg, wave, t < T, E, K, sid, swt);
  __syncthreads();
  if (t < T && lane < K) {
    ids[(size_t)t * K + lane] = sid[wave][lane];
    wts[(size_t)t * K + lane] = swt[wave][lane];
    if (topk_ids) topk_ids[(size_t)t * K + lane] = sid[wave][lane];
    if (topk_w) topk_w[(size_t)t * K + lane] = swt[wave][lane];
  }
}

// ---------------------------------------------------------------- 2. group

// Workgroup e: counts, then the pairs p (= t K + j) with ids[p] == e in
// increasing p, written at off[e] .. off[e] + cnt[e]. Wave w owns the
// contiguous run [w R, (w + 1) R) of pairs (R a multiple of 64), so after one
// exchange of the waves' counts each wave writes its pairs at its own running
// offset, in order, with no further barrier.
__global__ __launch_bounds__(kThr) void g_group_kernel(const int *__restrict__ ids, int *__restrict__ cnt,
                                                        int *__restrict__ off, int *__restrict__ plist, const int P) {
  __shared__ int red[2][kWv];
  const int e = (int)blockIdx.x;
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = ((P + kWv - 1) / kWv + 63) / 64 * 64;
  const int p0 = wave * R, p1 = p0 + R < P ? p0 + R : P;
  // kBatch loads in flight per lane per round trip (ids past p1 read as -1)
  constexpr int kBatch = 8;
  int lt = 0, eq = 0;
  for (int base = p0; base < p1; base += 64 * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = base + 64 * i + lane;
      v[i] = p < p1 ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      lt += v[i] >= 0 && v[i] < e;
      eq += v[i] == e;
    }
  }
  for (int s = 32; s >= 1; s >>= 1) {
    lt += __shfl_xor(lt, s);
    eq += __shfl_xor(eq, s);
  }
  if (lane == 0) red[0][wave] = lt, red[1][wave] = eq;
  __syncthreads();
  int o = 0, n = 0, run = 0;
#pragma unroll
  for (int w = 0; w < kWv; ++w) {
    o += red[0][w], n += red[1][w];
    run += w < wave ? red[1][w] : 0;
  }
  if (tid == 0) cnt[e] = n, off[e] = o;
  run += o;
  for (int base = p0; base < p1; base += 64 * kBatch) {
    int v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = base + 64 * i + lane;
      v[i] = p < p1 ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const bool f = v[i] == e;
      const unsigned long long bal = __ballot(f);
      if (f) plist[run + __popcll(bal & ((1ull << lane) - 1ull))] = base + 64 * i + lane;
      run += __popcll(bal);
    }
  }
}

// ---------------------------------------------------------------- 3. chunks

// One workgroup: chunk offsets per expert (an exclusive scan in expert order)
// and the (expert, chunk) list, for chunks of CH pairs; when choff32 is not
// null, the same for chunks of 32 pairs (the wide gate/up form) as well.
template <int CH>
__device__ __forceinline__ void chunk_list(const int *__restrict__ cnt, int *__restrict__ choff,
                                           int2 *__restrict__ chunks, const int E, int *nch) {
  // E <= 256 = kThr: thread e holds expert e's chunk count; an inclusive scan
  // over the threads (in-wave shuffles, then the waves' totals), written
  // shifted by one as the exclusive offsets
  static_assert(QMV_MOE_MAX_EXPERTS <= kThr, "one thread per expert");
  __shared__ int wsum[kWv];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid < E ? (cnt[tid] + CH - 1) / CH : 0;
  int v = c;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWv; ++w) v += w < wave ? wsum[w] : 0;
  if (tid < E) nch[tid + 1] = v;
  if (tid == 0) nch[0] = 0;
  __syncthreads();
  for (int e = tid; e <= E; e += kThr) choff[e] = nch[e];
  for (int e = tid; e < E; e += kThr)
    for (int c = 0; c < nch[e + 1] - nch[e]; ++c) chunks[nch[e] + c] = make_int2(e, c);
}

__global__ __launch_bounds__(kThr) void g_chunks_kernel(const int *__restrict__ cnt, int *__restrict__ choff,
                                                         int2 *__restrict__ chunks, int *__restrict__ choff32,
                                                         int2 *__restrict__ chunks32, const int E) {
  __shared__ int nch[2][QMV_MOE_MAX_EXPERTS + 1];
  chunk_list<kChunk>(cnt, choff, chunks, E, nch[0]);
  if (choff32) chunk_list<layout::kGroupChunk32>(cnt, choff32, chunks32, E, nch[1]);
}

// ---------------------------------------------------------------- 4. gate/up

// Super-block b of one W row for lane group kg: the 16-byte header and the
// lane's 8 quant bytes of each 64-weight chunk.
struct SbLoad {
  uint4 hdr;
  uint2 q[4];
};
// (The windows of addr::group_window.)
__device__ __forceinline__ SbLoad load_sb(const uint8_t *__restrict__ bp, const int kg) {
  SbLoad r;
  r.hdr = *reinterpret_cast<const uint4 *>(bp + addr::group_window(kg, 0).off);
#pragma unroll
  for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const uint2 *>(bp + addr::group_window(kg, 1 + c).off);
  return r;
}

// Chunk y's pairs: expert e, the list positions pos0 .. pos0 + n - 1 (n <= 16).
struct ChunkInfo {
  int e, pos0, n;
};
template <int CH = kChunk>
__device__ __forceinline__ ChunkInfo chunk_info(const int2 *__restrict__ chunks, const int *__restrict__ cnt,
                                                const int *__restrict__ off, const int y) {
  const int2 ec = chunks[y];
  ChunkInfo ci;
  ci.e = ec.x;
  const int first = ec.y * CH;
  ci.pos0 = off[ec.x] + first;
  const int left = cnt[ec.x] - first;
  ci.n = left < CH ? left : CH;
  return ci;
}

// Each wave owns TPW tiles of 16 weight rows over the whole of K; the
// workgroup's four waves cover 64 TPW consecutive rows and share the chunk's
// staged activations. The next super-block's weights are loaded while the
// current one is multiplied.
template <int TPW>
__global__ __launch_bounds__(kThr) void g_gate_up_kernel(const uint8_t *__restrict__ w_gate,
                                                          const uint8_t *__restrict__ w_up,
                                                          const uint16_t *__restrict__ x,
                                                          const int *__restrict__ cnt, const int *__restrict__ off,
                                                          const int *__restrict__ choff,
                                                          const int2 *__restrict__ chunks,
                                                          const int *__restrict__ plist, float *__restrict__ h,
                                                          const int hidden, const int ffn, const int E, const int K) {
  extern __shared__ uint4 lds[];
  const int y = (int)blockIdx.y;
  if (y >= choff[E]) return;   // uniform over the workgroup
  const ChunkInfo ci = chunk_info(chunks, cnt, off, y);
  const int gpr = hidden >> 3, rs = gpr + layout::kGroupRowPad, nsub = hidden >> 5, nblk = hidden >> 8;
  const int ss = nsub + layout::kGroupSumPad;
  uint4 *xs = lds;                                                    // [16][rs]
  float *xsum = reinterpret_cast<float *>(lds + (size_t)kChunk * rs); // [16][ss]
  const int tid = (int)threadIdx.x, wv = tid >> 6, l = tid & 63, nl = l & 15, kg = l >> 4;

  // stage the chunk's activation rows (zeros past its pairs)
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  for (int g = tid; g < kChunk * gpr; g += kThr) {
    const int i = g / gpr, gg = g - i * gpr;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < ci.n) v = xg[(size_t)(plist[ci.pos0 + i] / K) * gpr + gg];
    xs[i * rs + gg] = v;
  }
  __syncthreads();
  for (int t = tid; t < kChunk * nsub; t += kThr) {
    const int i = t / nsub, sb = t - i * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 g = xs[i * rs + 4 * sb + q];
      const uint32_t v4[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += bf16_bits_to_f32(v4[u] & 0xFFFFu);
        s += bf16_bits_to_f32(v4[u] >> 16);
      }
    }
    xsum[i * ss + sb] = s;
  }
  __syncthreads();

  // rows rb .. rb + 16 TPW - 1 (the grid covers ffn exactly)
  const int rb = ((int)blockIdx.x * kWv + wv) * (TPW * kTile);
  const size_t row_bytes = (size_t)nblk * kQ4KBlockBytes;
  const uint8_t *gr[TPW], *ur[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    gr[tt] = w_gate + addr::group_row(ci.e, ffn, blockIdx.x, kWv, wv, TPW, tt, l) * row_bytes;
    ur[tt] = w_up + addr::group_row(ci.e, ffn, blockIdx.x, kWv, wv, TPW, tt, l) * row_bytes;
  }
  float ag[TPW][4], au[TPW][4];
  SbLoad lg[TPW], lu[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) ag[tt][r] = 0.0f, au[tt][r] = 0.0f;
    lg[tt] = load_sb(gr[tt], kg);
    lu[tt] = load_sb(ur[tt], kg);
  }
  const uint4 *xa = xs + nl * rs + kg;
  for (int b = 0; b < nblk; ++b) {
    const size_t nb = addr::group_block(b + 1, nblk);   // last block re-read at the end
    SbLoad ng[TPW], nu[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      ng[tt] = load_sb(gr[tt] + nb, kg);
      nu[tt] = load_sb(ur[tt] + nb, kg);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const ScaleSel sel = scale_selectors(c);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jg = 8 * b + 2 * c + hh;
        const bf16x8 av = __builtin_bit_cast(bf16x8, xa[4 * jg]);
        float xsr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xsr[r] = xsum[(4 * kg + r) * ss + jg];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const ChunkScales cg = chunk_scales(lg[tt].hdr, sel), cu = chunk_scales(lu[tt].hdr, sel);
          const uint2 qg = lg[tt].q[c], qu = lu[tt].q[c];
          const bf16x8 bg = hh ? nibbles8((qg.x >> 4) & 0x0F0F0F0Fu, (qg.y >> 4) & 0x0F0F0F0Fu)
                               : nibbles8(qg.x & 0x0F0F0F0Fu, qg.y & 0x0F0F0F0Fu);
          const bf16x8 bu = hh ? nibbles8((qu.x >> 4) & 0x0F0F0F0Fu, (qu.y >> 4) & 0x0F0F0F0Fu)
                               : nibbles8(qu.x & 0x0F0F0F0Fu, qu.y & 0x0F0F0F0Fu);
          f32x4 dg = {0.0f, 0.0f, 0.0f, 0.0f}, du = {0.0f, 0.0f, 0.0f, 0.0f};
          dg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bg, dg, 0, 0, 0);
          du = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bu, du, 0, 0, 0);
          const float sag = hh ? cg.a1 : cg.a0, sbg = hh ? cg.b1 : cg.b0;
          const float sau = hh ? cu.a1 : cu.a0, sbu = hh ? cu.b1 : cu.b0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ag[tt][r] = __builtin_fmaf(sag, dg[r], ag[tt][r]);
            ag[tt][r] = __builtin_fmaf(-sbg, xsr[r], ag[tt][r]);
            au[tt][r] = __builtin_fmaf(sau, du[r], au[tt][r]);
            au[tt][r] = __builtin_fmaf(-sbu, xsr[r], au[tt][r]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) lg[tt] = ng[tt], lu[tt] = nu[tt];
  }
  // lane l holds pairs 4 kg .. 4 kg + 3 of row rb + 16 tt + nl
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * kg + r;
      const float g = ag[tt][r], u = au[tt][r];
      if (i < ci.n) h[(size_t)(ci.pos0 + i) * ffn + rb + kTile * tt + nl] = g / (1.0f + expf(-g)) * u;
    }
}

// The same product for chunks of 32 pairs: eight waves, each owning TPW tiles
// over all of K, and two MFMA row blocks (pairs 0..15 and 16..31) per
// converted weight fragment, so each expert's weights are read once per 32 of
// its pairs and each conversion feeds two products. One tile per wave (128 rows
// per workgroup) measured about 1% faster than two at 512 tokens: twice the
// workgroups, each staging the chunk's activations, but shorter ones.
constexpr int kChunk32 = layout::kGroupChunk32;
constexpr int kWv32 = addr::kGroupWideWaves;
constexpr int kThr32 = 64 * kWv32;

template <int TPW>
__global__ __launch_bounds__(kThr32) void g_gate_up32_kernel(const uint8_t *__restrict__ w_gate,
                                                              const uint8_t *__restrict__ w_up,
                                                              const uint16_t *__restrict__ x,
                                                              const int *__restrict__ cnt, const int *__restrict__ off,
                                                              const int *__restrict__ choff,
                                                              const int2 *__restrict__ chunks,
                                                              const int *__restrict__ plist, float *__restrict__ h,
                                                              const int hidden, const int ffn, const int E,
                                                              const int K) {
  extern __shared__ uint4 lds[];
  const int y = (int)blockIdx.y;
  if (y >= choff[E]) return;   // uniform over the workgroup
  const ChunkInfo ci = chunk_info<kChunk32>(chunks, cnt, off, y);
  const int gpr = hidden >> 3, rs = gpr + layout::kGroupRowPad, nsub = hidden >> 5, nblk = hidden >> 8;
  const int ss = nsub + layout::kGroupSumPad;
  uint4 *xs = lds;                                                      // [32][rs]
  float *xsum = reinterpret_cast<float *>(lds + (size_t)kChunk32 * rs); // [32][ss]
  const int tid = (int)threadIdx.x, wv = tid >> 6, l = tid & 63, nl = l & 15, kg = l >> 4;

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  for (int g = tid; g < kChunk32 * gpr; g += kThr32) {
    const int i = g / gpr, gg = g - i * gpr;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < ci.n) v = xg[(size_t)(plist[ci.pos0 + i] / K) * gpr + gg];
    xs[i * rs + gg] = v;
  }
  __syncthreads();
  for (int t = tid; t < kChunk32 * nsub; t += kThr32) {
    const int i = t / nsub, sb = t - i * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 g = xs[i * rs + 4 * sb + q];
      const uint32_t v4[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += bf16_bits_to_f32(v4[u] & 0xFFFFu);
        s += bf16_bits_to_f32(v4[u] >> 16);
      }
    }
    xsum[i * ss + sb] = s;
  }
  __syncthreads();

  // rows rb .. rb + 16 TPW - 1 (the grid covers ffn exactly)
  const int rb = ((int)blockIdx.x * kWv32 + wv) * (TPW * kTile);
  const size_t row_bytes = (size_t)nblk * kQ4KBlockBytes;
  const uint8_t *gr[TPW], *ur[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    gr[tt] = w_gate + addr::group_row(ci.e, ffn, blockIdx.x, kWv32, wv, TPW, tt, l) * row_bytes;
    ur[tt] = w_up + addr::group_row(ci.e, ffn, blockIdx.x, kWv32, wv, TPW, tt, l) * row_bytes;
  }
  float ag[TPW][2][4], au[TPW][2][4];
  SbLoad lg[TPW], lu[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ag[tt][hb][r] = 0.0f, au[tt][hb][r] = 0.0f;
    lg[tt] = load_sb(gr[tt], kg);
    lu[tt] = load_sb(ur[tt], kg);
  }
  const uint4 *xa0 = xs + nl * rs + kg, *xa1 = xs + (kTile + nl) * rs + kg;
  for (int b = 0; b < nblk; ++b) {
    const size_t nb = addr::group_block(b + 1, nblk);   // last block re-read at the end
    SbLoad ng[TPW], nu[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      ng[tt] = load_sb(gr[tt] + nb, kg);
      nu[tt] = load_sb(ur[tt] + nb, kg);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const ScaleSel sel = scale_selectors(c);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jg = 8 * b + 2 * c + hh;
        const bf16x8 av0 = __builtin_bit_cast(bf16x8, xa0[4 * jg]);
        const bf16x8 av1 = __builtin_bit_cast(bf16x8, xa1[4 * jg]);
        float xs0[4], xs1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xs0[r] = xsum[(4 * kg + r) * ss + jg];
          xs1[r] = xsum[(kTile + 4 * kg + r) * ss + jg];
        }
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const ChunkScales cg = chunk_scales(lg[tt].hdr, sel), cu = chunk_scales(lu[tt].hdr, sel);
          const uint2 qg = lg[tt].q[c], qu = lu[tt].q[c];
          const bf16x8 bg = hh ? nibbles8((qg.x >> 4) & 0x0F0F0F0Fu, (qg.y >> 4) & 0x0F0F0F0Fu)
                               : nibbles8(qg.x & 0x0F0F0F0Fu, qg.y & 0x0F0F0F0Fu);
          const bf16x8 bu = hh ? nibbles8((qu.x >> 4) & 0x0F0F0F0Fu, (qu.y >> 4) & 0x0F0F0F0Fu)
                               : nibbles8(qu.x & 0x0F0F0F0Fu, qu.y & 0x0F0F0F0Fu);
          const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
          const f32x4 dg0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av0, bg, z4, 0, 0, 0);
          const f32x4 dg1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av1, bg, z4, 0, 0, 0);
          const f32x4 du0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av0, bu, z4, 0, 0, 0);
          const f32x4 du1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av1, bu, z4, 0, 0, 0);
          const float sag = hh ? cg.a1 : cg.a0, sbg = hh ? cg.b1 : cg.b0;
          const float sau = hh ? cu.a1 : cu.a0, sbu = hh ? cu.b1 : cu.b0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ag[tt][0][r] = __builtin_fmaf(sag, dg0[r], ag[tt][0][r]);
            ag[tt][0][r] = __builtin_fmaf(-sbg, xs0[r], ag[tt][0][r]);
            ag[tt][1][r] = __builtin_fmaf(sag, dg1[r], ag[tt][1][r]);
            ag[tt][1][r] = __builtin_fmaf(-sbg, xs1[r], ag[tt][1][r]);
            au[tt][0][r] = __builtin_fmaf(sau, du0[r], au[tt][0][r]);
            au[tt][0][r] = __builtin_fmaf(-sbu, xs0[r], au[tt][0][r]);
            au[tt][1][r] = __builtin_fmaf(sau, du1[r], au[tt][1][r]);
            au[tt][1][r] = __builtin_fmaf(-sbu, xs1[r], au[tt][1][r]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) lg[tt] = ng[tt], lu[tt] = nu[tt];
  }
  // lane l holds pairs 16 hb + 4 kg .. + 3 of row rb + 16 tt + nl
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = kTile * hb + 4 * kg + r;
        const float g = ag[tt][hb][r], u = au[tt][hb][r];
        if (i < ci.n) h[(size_t)(ci.pos0 + i) * ffn + rb + kTile * tt + nl] = g / (1.0f + expf(-g)) * u;
      }
}

// ---------------------------------------------------------------- 5. down

template <int TPW>
__global__ __launch_bounds__(kThr) void g_down_kernel(const uint8_t *__restrict__ w_down,
                                                       const int *__restrict__ cnt, const int *__restrict__ off,
                                                       const int *__restrict__ choff, const int2 *__restrict__ chunks,
                                                       const int *__restrict__ plist, const float *__restrict__ h,
                                                       float *__restrict__ z, const int hidden, const int ffn,
                                                       const int E) {
  extern __shared__ uint4 lds[];
  const int y = (int)blockIdx.y;
  if (y >= choff[E]) return;
  const ChunkInfo ci = chunk_info(chunks, cnt, off, y);
  const int gpr = ffn >> 3, rs = gpr + layout::kGroupRowPad, nsub = ffn >> 5, nblk = ffn >> 8;
  const int ss = nsub + layout::kGroupSumPad;
  uint4 *hs_hi = lds;                                                     // [16][rs]
  uint4 *hs_mi = lds + (size_t)kChunk * rs;                               // [16][rs]
  uint4 *hs_lo = lds + (size_t)2 * kChunk * rs;                           // [16][rs]
  float *hsum = reinterpret_cast<float *>(lds + (size_t)3 * kChunk * rs); // [16][ss]
  const int tid = (int)threadIdx.x, wv = tid >> 6, l = tid & 63, nl = l & 15, kg = l >> 4;

  // stage h of the chunk's pairs as three bf16 parts (zeros past its pairs):
  // h_hi = bf16(h), h_mi = bf16(h - h_hi), h_lo = bf16(h - h_hi - h_mi); each
  // difference is exact in fp32, so the parts keep about 24 bits of h
  for (int g = tid; g < kChunk * gpr; g += kThr) {
    const int i = g / gpr, gg = g - i * gpr;
    uint32_t hi[4] = {0u, 0u, 0u, 0u}, mi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
    if (i < ci.n) {
      const float4 *hp = reinterpret_cast<const float4 *>(h + (size_t)(ci.pos0 + i) * ffn + 8 * gg);
      const float4 a = hp[0], b = hp[1];
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t p[2][3];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float v0 = v[2 * q + e];
          p[e][0] = f32_to_bf16_rne(v0);
          const float r1 = v0 - bf16_bits_to_f32(p[e][0]);
          p[e][1] = f32_to_bf16_rne(r1);
          p[e][2] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(p[e][1]));
        }
        hi[q] = p[0][0] | (p[1][0] << 16);
        mi[q] = p[0][1] | (p[1][1] << 16);
        lo[q] = p[0][2] | (p[1][2] << 16);
      }
    }
    hs_hi[i * rs + gg] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    hs_mi[i * rs + gg] = make_uint4(mi[0], mi[1], mi[2], mi[3]);
    hs_lo[i * rs + gg] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  __syncthreads();
  // per-sub-block sums of the values the products see (h_hi + h_mi + h_lo), in index order
  for (int t = tid; t < kChunk * nsub; t += kThr) {
    const int i = t / nsub, sb = t - i * nsub;
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 gh = hs_hi[i * rs + 4 * sb + q], gm = hs_mi[i * rs + 4 * sb + q], gl = hs_lo[i * rs + 4 * sb + q];
      const uint32_t vh[4] = {gh.x, gh.y, gh.z, gh.w}, vm[4] = {gm.x, gm.y, gm.z, gm.w};
      const uint32_t vl[4] = {gl.x, gl.y, gl.z, gl.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s += bf16_bits_to_f32(vh[u] & 0xFFFFu) + (bf16_bits_to_f32(vm[u] & 0xFFFFu) + bf16_bits_to_f32(vl[u] & 0xFFFFu));
        s += bf16_bits_to_f32(vh[u] >> 16) + (bf16_bits_to_f32(vm[u] >> 16) + bf16_bits_to_f32(vl[u] >> 16));
      }
    }
    hsum[i * ss + sb] = s;
  }
  __syncthreads();

  // W_down rows rb .. rb + 16 TPW - 1 (the grid covers hidden exactly)
  const int rb = ((int)blockIdx.x * kWv + wv) * (TPW * kTile);
  const size_t row_bytes = (size_t)nblk * kQ4KBlockBytes;
  const uint8_t *dr[TPW];
  float acc[TPW][4];
  SbLoad ld[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    dr[tt] = w_down + addr::group_row(ci.e, hidden, blockIdx.x, kWv, wv, TPW, tt, l) * row_bytes;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tt][r] = 0.0f;
    ld[tt] = load_sb(dr[tt], kg);
  }
  const uint4 *ha = hs_hi + nl * rs + kg, *ma = hs_mi + nl * rs + kg, *la = hs_lo + nl * rs + kg;
  for (int b = 0; b < nblk; ++b) {
    const size_t nb = addr::group_block(b + 1, nblk);
    SbLoad nx[TPW];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) nx[tt] = load_sb(dr[tt] + nb, kg);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const ScaleSel sel = scale_selectors(c);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jg = 8 * b + 2 * c + hh;
        const bf16x8 ahi = __builtin_bit_cast(bf16x8, ha[4 * jg]), ami = __builtin_bit_cast(bf16x8, ma[4 * jg]);
        const bf16x8 alo = __builtin_bit_cast(bf16x8, la[4 * jg]);
        float hsr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hsr[r] = hsum[(4 * kg + r) * ss + jg];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const ChunkScales cs = chunk_scales(ld[tt].hdr, sel);
          const uint2 qd = ld[tt].q[c];
          const bf16x8 bq = hh ? nibbles8((qd.x >> 4) & 0x0F0F0F0Fu, (qd.y >> 4) & 0x0F0F0F0Fu)
                               : nibbles8(qd.x & 0x0F0F0F0Fu, qd.y & 0x0F0F0F0Fu);
          f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bq, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ami, bq, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bq, d, 0, 0, 0);
          const float sa = hh ? cs.a1 : cs.a0, sb = hh ? cs.b1 : cs.b0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[tt][r] = __builtin_fmaf(sa, d[r], acc[tt][r]);
            acc[tt][r] = __builtin_fmaf(-sb, hsr[r], acc[tt][r]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) ld[tt] = nx[tt];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * kg + r;
    if (i < ci.n) {
      float *zr = z + (size_t)plist[ci.pos0 + i] * hidden + rb + nl;
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) zr[kTile * tt] = acc[tt][r];
    }
  }
}

// ---------------------------------------------------------------- 6. combine

__global__ __launch_bounds__(kThr) void g_combine_kernel(const float *__restrict__ z, const float *__restrict__ wts,
                                                          float *__restrict__ y, const int hidden, const int K) {
  const int t = (int)blockIdx.x;
  const int nn = (int)blockIdx.y * kThr + (int)threadIdx.x;
  if (nn >= hidden) return;
  float acc = 0.0f;
  for (int j = 0; j < K; ++j) acc = __builtin_fmaf(wts[(size_t)t * K + j], z[((size_t)t * K + j) * hidden + nn], acc);
  y[(size_t)t * hidden + nn] = acc;
}

}  // namespace

namespace {

// Tiles per wave from the number of pairs P. Measured on the 35B-A3B layer
// (hidden 2048, ffn 768, 128 experts, top-8): four tiles per wave is fastest
// from 512 tokens (P = 4096) up, two at 64 tokens (P = 512).
int tiles_per_wave(int P) { return addr::group_tiles_per_wave(P); }

template <int TPW>
int launch_gate_up(const uint8_t *w_gate, const uint8_t *w_up, const uint16_t *x, const int *cnt, const int *off,
                   const int *choff, const int2 *chunks, const int *plist, float *h, int hidden, int ffn, int E,
                   int K, unsigned maxch, hipStream_t s) {
  static LdsGrant granted;
  const size_t lds = layout::group_gate_up_lds(kChunk, hidden);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&g_gate_up_kernel<TPW>), lds, granted, "g_gate_up_kernel lds"))
    return QMV_ERR_HIP;
  return launch_kernel("g_gate_up_kernel", g_gate_up_kernel<TPW>,
                       dim3((unsigned)(ffn / (kWv * kTile * TPW)), maxch), dim3(kThr), lds, s, w_gate, w_up, x, cnt,
                       off, choff, chunks, plist, h, hidden, ffn, E, K);
}

template <int TPW>
int launch_gate_up32(const uint8_t *w_gate, const uint8_t *w_up, const uint16_t *x, const int *cnt, const int *off,
                     const int *choff, const int2 *chunks, const int *plist, float *h, int hidden, int ffn, int E,
                     int K, unsigned maxch, hipStream_t s) {
  static LdsGrant granted;
  const size_t lds = layout::group_gate_up_lds(kChunk32, hidden);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&g_gate_up32_kernel<TPW>), lds, granted,
                        "g_gate_up32_kernel lds"))
    return QMV_ERR_HIP;
  return launch_kernel("g_gate_up32_kernel", g_gate_up32_kernel<TPW>,
                       dim3((unsigned)(ffn / (kWv32 * kTile * TPW)), maxch), dim3(kThr32), lds, s, w_gate, w_up, x,
                       cnt, off, choff, chunks, plist, h, hidden, ffn, E, K);
}

template <int TPW>
int launch_down(const uint8_t *w_down, const int *cnt, const int *off, const int *choff, const int2 *chunks,
                const int *plist, const float *h, float *z, int hidden, int ffn, int E, unsigned maxch,
                hipStream_t s) {
  static LdsGrant granted;
  const size_t lds = layout::group_down_lds(ffn);
  if (allow_dynamic_lds(reinterpret_cast<const void *>(&g_down_kernel<TPW>), lds, granted, "g_down_kernel lds"))
    return QMV_ERR_HIP;
  return launch_kernel("g_down_kernel", g_down_kernel<TPW>, dim3((unsigned)(hidden / (kWv * kTile * TPW)), maxch),
                       dim3(kThr), lds, s, w_down, cnt, off, choff, chunks, plist, h, z, hidden, ffn, E);
}

}  // namespace

int launch_q4_k_moe_grouped(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                            const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, void *ws, int t,
                            int hidden, int ffn, int n_experts, int top_k, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const layout::GroupLayout L = layout::group_layout(t, hidden, ffn, n_experts, top_k);
  uint8_t *wb = static_cast<uint8_t *>(ws);
  int *ids = reinterpret_cast<int *>(wb + L.ids);
  float *wts = reinterpret_cast<float *>(wb + L.wts);
  int *cnt = reinterpret_cast<int *>(wb + L.cnt);
  int *off = reinterpret_cast<int *>(wb + L.off);
  int *choff = reinterpret_cast<int *>(wb + L.choff);
  int2 *chunks = reinterpret_cast<int2 *>(wb + L.chunks);
  int *choff32 = reinterpret_cast<int *>(wb + L.choff32);
  int2 *chunks32 = reinterpret_cast<int2 *>(wb + L.chunks32);
  int *plist = reinterpret_cast<int *>(wb + L.plist);
  float *h = reinterpret_cast<float *>(wb + L.h);
  float *z = reinterpret_cast<float *>(wb + L.z);
  const int P = t * top_k;
  const unsigned maxch = (unsigned)((P + kChunk - 1) / kChunk + n_experts);
  const uint8_t *wg = static_cast<const uint8_t *>(w_gate), *wu = static_cast<const uint8_t *>(w_up);
  const uint8_t *wd = static_cast<const uint8_t *>(w_down);
  int rc = launch_kernel("g_route_kernel", g_route_kernel, dim3((unsigned)((t + kWv - 1) / kWv)), dim3(kThr), 0, s,
                         logits, ids, wts, topk_ids, topk_w, t, n_experts, top_k);
  if (!rc) rc = launch_kernel("g_group_kernel", g_group_kernel, dim3((unsigned)n_experts), dim3(kThr), 0, s, ids,
                              cnt, off, plist, P);
  // gate/up in chunks of 32 where there are enough pairs and 32 rows of x fit in LDS
  const bool wide = P >= 2048 && layout::group_gate_up_lds(kChunk32, hidden) <= layout::kLdsBudget;
  if (!rc) rc = launch_kernel("g_chunks_kernel", g_chunks_kernel, dim3(1), dim3(kThr), 0, s, cnt, choff, chunks,
                              wide ? choff32 : nullptr, wide ? chunks32 : nullptr, n_experts);
  if (!rc && wide) {
    const unsigned maxch32 = (unsigned)((P + kChunk32 - 1) / kChunk32 + n_experts);
    rc = launch_gate_up32<addr::kGroupWideTiles>(wg, wu, x, cnt, off, choff32, chunks32, plist, h, hidden, ffn, n_experts, top_k, maxch32,
                             s);
  } else if (!rc) {
    switch (tiles_per_wave(P)) {
      case 4: rc = launch_gate_up<4>(wg, wu, x, cnt, off, choff, chunks, plist, h, hidden, ffn, n_experts, top_k,
                                     maxch, s); break;
      case 2: rc = launch_gate_up<2>(wg, wu, x, cnt, off, choff, chunks, plist, h, hidden, ffn, n_experts, top_k,
                                     maxch, s); break;
      default: rc = launch_gate_up<1>(wg, wu, x, cnt, off, choff, chunks, plist, h, hidden, ffn, n_experts, top_k,
                                      maxch, s); break;
    }
  }
  if (!rc) {
    switch (tiles_per_wave(P)) {
      case 4: rc = launch_down<4>(wd, cnt, off, choff, chunks, plist, h, z, hidden, ffn, n_experts, maxch, s); break;
      case 2: rc = launch_down<2>(wd, cnt, off, choff, chunks, plist, h, z, hidden, ffn, n_experts, maxch, s); break;
      default: rc = launch_down<1>(wd, cnt, off, choff, chunks, plist, h, z, hidden, ffn, n_experts, maxch, s); break;
    }
  }
  if (!rc) rc = launch_kernel("g_combine_kernel", g_combine_kernel, dim3((unsigned)t,
                              (unsigned)((hidden + kThr - 1) / kThr)), dim3(kThr), 0, s, z, wts, y, hidden, top_k);
  return rc;
}

}  // namespace qmv
