// Drives every entry point's argument checks in a host-only build (qmv_api.cpp
// + stand-in launchers, no HIP runtime), compiled with the address and
// undefined-behaviour sanitizers. Pointers are fake, aligned device-like
// addresses that nothing dereferences: a call either fails a check or reaches
// a stand-in launcher. Exit status 0 means every expectation held and the
// sanitizers found nothing.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/qmv.h"
#include "stub_launchers.h"

namespace {

int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

// Fake device addresses, 4 GiB apart, 256-byte aligned.
const uintptr_t kBase = (uintptr_t)0x7F0000000000ull;
void *at(int region, uintptr_t off = 0) { return reinterpret_cast<void *>(kBase + ((uintptr_t)region << 32) + off); }
const void *W = at(0), *X = at(1);
float *Y = static_cast<float *>(at(2));
void *WS = at(3);

const int kInts[] = {INT_MIN, -257, -1, 0, 1, 2, 3, 4, 5, 31, 32, 33, 255, 256, 257, 512, 4096, 17408,
                     65536, 65537, 1 << 24, INT_MAX / 256 * 256, INT_MAX - 1, INT_MAX};

bool is_code(int rc) { return rc <= 0 && rc >= QMV_ERR_HIP; }

// Exact byte size of an n x k matrix of (bw weights, bb bytes) blocks, or 0.
size_t mbytes(int n, int k, int bw, int bb) {
  if (n <= 0 || k <= 0 || k % bw) return 0;
  return (size_t)n * (size_t)(k / bw) * (size_t)bb;
}

typedef int (*GemvBf16)(const void *, size_t, const uint16_t *, float *, int, int, int, void *);
typedef int (*Dequant)(const void *, size_t, float *, int, int, void *);

struct DenseFormat {
  const char *name;
  GemvBf16 fn;
  int block_weights, block_bytes, k_step;
};

void dense_formats() {
  const uint16_t *xb = static_cast<const uint16_t *>(X);
  const DenseFormat fmts[] = {{"q4_k", qmv_q4_k, 256, 144, 256},
                              {"q5_k", qmv_q5_k, 256, 176, 256},
                              {"q6_k", qmv_q6_k, 256, 210, 256},
                              {"q4_0", qmv_q4_0, 32, 18, 256},
                              {"iq4_xs", qmv_iq4_xs, 256, 136, 256}};
  for (const DenseFormat &f : fmts) {
    // a valid call reaches the launcher with its shape
    for (int m = 1; m <= 4; ++m) {
      const int n = 3, k = 2 * f.k_step;
      const int before = stub::launches;
      EXPECT(f.fn(W, mbytes(n, k, f.block_weights, f.block_bytes), xb, Y, m, n, k, nullptr) == QMV_OK);
      EXPECT(stub::launches == before + 1 && stub::last_m == m && stub::last_n == n && stub::last_k == k);
    }
    // every prefix and a few oversizes of a valid buffer are QMV_ERR_SIZE
    const int n = 2, k = 2 * f.k_step;
    const size_t full = mbytes(n, k, f.block_weights, f.block_bytes);
    for (size_t b = 0; b < full + 2 * (size_t)f.block_bytes; ++b)
      if (b != full) EXPECT(f.fn(W, b, xb, Y, 1, n, k, nullptr) == QMV_ERR_SIZE);
    // every extreme (m, n, k) returns a status code and launches only what fits
    for (int m : kInts)
      for (int nn : kInts)
        for (int kk : kInts) {
          const size_t wb = mbytes(nn, kk, f.block_weights, f.block_bytes);
          const int before = stub::launches;
          const int rc = f.fn(W, wb ? wb : 1, xb, Y, m, nn, kk, nullptr);
          EXPECT(is_code(rc));
          EXPECT((rc == QMV_OK) == (stub::launches == before + 1));
          if (rc == QMV_OK) EXPECT(m >= 1 && m <= 4 && nn >= 1 && kk >= 256 && kk % 256 == 0);
        }
    EXPECT(f.fn(nullptr, full, xb, Y, 1, n, k, nullptr) == QMV_ERR_NULL);
    EXPECT(f.fn(W, full, xb, static_cast<float *>(at(0, 64)), 1, n, k, nullptr) == QMV_ERR_ALIAS);
  }
}

void pair() {
  const uint16_t *xb = static_cast<const uint16_t *>(X);
  const void *W1 = at(4);
  float *Y1 = static_cast<float *>(at(5));
  for (int m = 1; m <= 4; ++m) {
    const int before = stub::launches;
    EXPECT(qmv_q4_k_pair(W, W1, mbytes(3, 512, 256, 144), xb, Y, Y1, m, 3, 512, nullptr) == QMV_OK);
    EXPECT(stub::launches == before + 1 && stub::last_m == m && stub::last_n == 3 && stub::last_k == 512);
  }
  const size_t full = mbytes(2, 512, 256, 144);
  for (size_t b = 0; b < full + 288; ++b)
    if (b != full) EXPECT(qmv_q4_k_pair(W, W1, b, xb, Y, Y1, 1, 2, 512, nullptr) == QMV_ERR_SIZE);
  EXPECT(qmv_q4_k_pair(W, nullptr, full, xb, Y, Y1, 1, 2, 512, nullptr) == QMV_ERR_NULL);
  EXPECT(qmv_q4_k_pair(W, W1, full, xb, Y, nullptr, 1, 2, 512, nullptr) == QMV_ERR_NULL);
  EXPECT(qmv_q4_k_pair(W, W1, full, xb, Y, static_cast<float *>(at(4, 64)), 1, 2, 512, nullptr) == QMV_ERR_ALIAS);
  EXPECT(qmv_q4_k_pair(W, W1, full, xb, Y, Y + 1, 1, 2, 512, nullptr) == QMV_ERR_ALIAS);
  EXPECT(qmv_q4_k_pair(W, W1, full, xb, Y, Y + 2, 1, 2, 512, nullptr) == QMV_OK);
  EXPECT(qmv_q4_k_pair(W, W1, full, xb, Y, Y, 1, 2, 512, nullptr) == QMV_ERR_ALIAS);
  // one grid covers 2n rows: n may be at most half the one-matrix row limit
  for (int m : kInts)
    for (int nn : kInts)
      for (int kk : kInts) {
        const size_t wb = mbytes(nn, kk, 256, 144);
        const int before = stub::launches;
        const int rc = qmv_q4_k_pair(W, W1, wb ? wb : 1, xb, Y, Y1, m, nn, kk, nullptr);
        EXPECT(is_code(rc));
        EXPECT((rc == QMV_OK) == (stub::launches == before + 1));
        if (rc == QMV_OK) EXPECT(m >= 1 && m <= 4 && nn >= 1 && nn <= QMV_MAX_MATRIX_ROWS / 2 && kk % 256 == 0);
      }
}

void q8_0() {
  const float *xf = static_cast<const float *>(X);
  EXPECT(qmv_q8_0(W, mbytes(4, 64, 32, 34), xf, Y, 1, 4, 64, nullptr) == QMV_OK);
  for (size_t b = 0; b < 3 * 34; ++b)
    if (b != 2 * 34) EXPECT(qmv_q8_0(W, b, xf, Y, 1, 1, 64, nullptr) == QMV_ERR_SIZE);
  for (int m : kInts)
    for (int k : kInts) {
      const size_t wb = mbytes(7, k, 32, 34);
      const int rc = qmv_q8_0(W, wb ? wb : 1, xf, Y, m, 7, k, nullptr);
      EXPECT(is_code(rc));
      if (rc == QMV_OK) EXPECT(m >= 1 && m <= 4 && (size_t)m * (size_t)k * 4 <= QMV_LDS_X_BYTES);
    }
}

void dequant() {
  const struct {
    Dequant fn;
    int bw, bb;
  } d[] = {{qmv_dequant_q4_k_f32, 256, 144}, {qmv_dequant_q8_0_f32, 32, 34}, {qmv_dequant_iq4_xs_f32, 256, 136},
           {qmv_dequant_q5_k_f32, 256, 176}, {qmv_dequant_q6_k_f32, 256, 210}, {qmv_dequant_q4_0_f32, 32, 18}};
  for (const auto &e : d) {
    EXPECT(e.fn(W, mbytes(3, 512, e.bw, e.bb), Y, 3, 512, nullptr) == QMV_OK);
    for (int n : kInts)
      for (int k : kInts) {
        const size_t wb = mbytes(n, k, e.bw, e.bb);
        EXPECT(is_code(e.fn(W, wb ? wb : 1, Y, n, k, nullptr)));
      }
  }
  EXPECT(qmv_dequant_q4_k_bf16(W, mbytes(3, 512, 256, 144), static_cast<uint16_t *>(at(2)), 3, 512, nullptr) ==
         QMV_OK);
}

typedef int (*MoeFn)(const void *, const void *, const void *, size_t, const float *, const uint16_t *, float *,
                     int32_t *, float *, int32_t *, void *, size_t, int, int, int, int, int, void *);
typedef size_t (*MoeWs)(int, int, int, int, int);

void moe(MoeFn fn, MoeWs wsfn, int block_bytes) {
  const void *wg = at(0), *wu = at(4), *wd = at(5);
  const float *lg = static_cast<const float *>(at(1));
  const uint16_t *xb = static_cast<const uint16_t *>(at(1, 1 << 20));
  int32_t *ids = static_cast<int32_t *>(at(2, 1 << 20));
  float *tw = static_cast<float *>(at(2, 2 << 20));
  int32_t *pairs = static_cast<int32_t *>(at(2, 3 << 20));
  for (int t = 1; t <= 4; ++t) {
    const int h = 2048, f = 768, e = 128, k = 8;
    const size_t bank = (size_t)e * f * (h / 256) * block_bytes;
    const size_t need = wsfn(t, h, f, e, k);
    EXPECT(need > 0);
    EXPECT(fn(wg, wu, wd, bank, lg, xb, Y, ids, tw, pairs, WS, need, t, h, f, e, k, nullptr) == QMV_OK);
    EXPECT(stub::last_ws == WS);
    EXPECT(fn(wg, wu, wd, bank, lg, xb, Y, ids, tw, pairs, WS, need - 1, t, h, f, e, k, nullptr) ==
           QMV_ERR_WORKSPACE);
    EXPECT(fn(wg, wu, wd, bank - 1, lg, xb, Y, ids, tw, pairs, WS, need, t, h, f, e, k, nullptr) == QMV_ERR_SIZE);
    EXPECT(fn(wg, wu, wd, bank, lg, xb, Y, ids, tw, pairs, at(3, 128), need, t, h, f, e, k, nullptr) ==
           QMV_ERR_ALIGN);
    EXPECT(fn(wg, wu, wd, bank, lg, xb, static_cast<float *>(at(4, 256)), ids, tw, pairs, WS, need, t, h, f, e, k,
              nullptr) == QMV_ERR_ALIAS);
  }
  // extremes of every count: a status code, never undefined behaviour
  for (int t : kInts)
    for (int e : {-1, 0, 1, 8, 128, 256, 257, INT_MAX})
      for (int k : {-1, 0, 1, 8, 9, INT_MAX})
        for (int h : {-256, 0, 256, 2048, 4096, INT_MAX / 256 * 256})
          for (int f : {0, 256, 768, INT_MAX / 256 * 256}) {
            (void)wsfn(t, h, f, e, k);
            EXPECT(is_code(fn(wg, wu, wd, 1, lg, xb, Y, ids, tw, pairs, WS, 1, t, h, f, e, k, nullptr)));
          }
}

void moe_noalloc() {
  const void *wg = at(0), *wu = at(4), *wd = at(5);
  const float *lg = static_cast<const float *>(at(1));
  const uint16_t *xb = static_cast<const uint16_t *>(at(1, 1 << 20));
  int32_t *ids = static_cast<int32_t *>(at(2, 1 << 20));
  for (int t = 1; t <= 4; ++t) {
    const int h = 2048, f = 768, e = 128, k = 8;
    const size_t bank = (size_t)e * f * (h / 256) * 144;
    const int before = stub::launches;
    EXPECT(qmv_q4_k_moe_noalloc(wg, wu, wd, bank, lg, xb, Y, ids, nullptr, nullptr, t, h, f, e, k, nullptr) == QMV_OK);
    EXPECT(stub::launches == before + 1 && stub::last_m == t);
    EXPECT(qmv_q4_k_moe_noalloc(wg, wu, wd, bank - 1, lg, xb, Y, ids, nullptr, nullptr, t, h, f, e, k, nullptr) ==
           QMV_ERR_SIZE);
    EXPECT(qmv_q4_k_moe_noalloc(wg, wu, wd, bank, lg, xb, static_cast<float *>(at(4, 256)), ids, nullptr, nullptr, t,
                                h, f, e, k, nullptr) == QMV_ERR_ALIAS);
  }
  // every call within the decode limits fits the fixed scratch: sweep the LDS-limited (pairs, ffn) corner
  for (int t = 1; t <= 4; ++t)
    for (int k = 1; k <= 8; ++k)
      for (int f = 256; f <= 65536; f += 256) {
        const int h = 256, e = 8;
        const size_t bank = (size_t)e * f * (h / 256) * 144;
        const size_t need = qmv_q4_k_moe_workspace(t, h, f, e, k);
        const int rc = qmv_q4_k_moe_noalloc(wg, wu, wd, bank, lg, xb, Y, ids, nullptr, nullptr, t, h, f, e, k, nullptr);
        EXPECT(need == 0 ? rc == QMV_ERR_RANGE : rc == QMV_OK);
        EXPECT(need <= QMV_MOE_NOALLOC_BYTES);
      }
  for (int t : kInts)
    for (int f : {0, 256, 768, 1024, 4096, INT_MAX / 256 * 256})
      EXPECT(is_code(qmv_q4_k_moe_noalloc(wg, wu, wd, 1, lg, xb, Y, ids, nullptr, nullptr, t, 2048, f, 128, 8, nullptr)));
}

void moe_prefill() {
  const void *wg = at(0), *wu = at(4), *wd = at(5);
  const float *lg = static_cast<const float *>(at(1));
  const uint16_t *xb = static_cast<const uint16_t *>(at(6));
  const int h = 2048, f = 768, e = 128, k = 8;
  const size_t bank = (size_t)e * f * (h / 256) * 144;
  for (int t : {1, 3, 17, 512, 4096, QMV_MOE_PREFILL_MAX_TOKENS}) {
    const size_t need = qmv_q4_k_moe_prefill_workspace(t, h, f, e, k);
    EXPECT(need > 0);
    EXPECT(qmv_q4_k_moe_prefill(wg, wu, wd, bank, lg, xb, Y, nullptr, nullptr, at(7), need, t, h, f, e, k,
                                nullptr) == QMV_OK);
    EXPECT(qmv_q4_k_moe_prefill(wg, wu, wd, bank, lg, xb, Y, nullptr, nullptr, at(7), need - 1, t, h, f, e, k,
                                nullptr) == QMV_ERR_WORKSPACE);
  }
  for (int t : kInts)
    for (int hh : {-256, 0, 256, 2048, 4608, 4864, INT_MAX / 256 * 256})
      for (int ff : {0, 256, 768, 1536, 1792, INT_MAX / 256 * 256}) {
        (void)qmv_q4_k_moe_prefill_workspace(t, hh, ff, e, k);
        EXPECT(is_code(qmv_q4_k_moe_prefill(wg, wu, wd, 1, lg, xb, Y, nullptr, nullptr, at(7), 1, t, hh, ff, e, k,
                                            nullptr)));
      }
}

void prefill() {
  const uint16_t *xb = static_cast<const uint16_t *>(X);
  struct Case {
    int m, n, k;
    size_t ws;
  } cases[] = {
      {512, 17408, 5120, (size_t)10 * 16 * 256 * 128 * 4},   // 272 tiles: 16 split in 10 parts of 2 K blocks
      {512, 5120, 17408, (size_t)3 * 80 * 256 * 128 * 4},    // 80 tiles in 3 parts of 23 K blocks
      {256, 32768, 5120, 0},                                   // 256 whole tiles
      {1, 16, 256, 0},                                         // one K block cannot split
      {64, 128, 1024, (size_t)4 * 256 * 128 * 4},            // one tile in 4 parts
  };
  for (const Case &c : cases) {
    EXPECT(qmm_q4_k_prefill_workspace(c.m, c.n, c.k) == c.ws);
    const size_t wb = mbytes(c.n, c.k, 256, 144);
    const int before = stub::launches;
    EXPECT(qmm_q4_k_prefill(W, wb, xb, Y, c.m, c.n, c.k, c.ws ? WS : nullptr, c.ws, nullptr) == QMV_OK);
    EXPECT(stub::launches == before + 1 && stub::last_ws == (c.ws ? WS : nullptr));
    if (c.ws) {
      EXPECT(qmm_q4_k_prefill(W, wb, xb, Y, c.m, c.n, c.k, nullptr, 0, nullptr) == QMV_ERR_WORKSPACE);
      EXPECT(qmm_q4_k_prefill(W, wb, xb, Y, c.m, c.n, c.k, WS, c.ws - 1, nullptr) == QMV_ERR_WORKSPACE);
    }
    // a workspace passed where none is needed is ignored
    EXPECT(qmm_q4_k_prefill(W, wb, xb, Y, c.m, c.n, c.k, WS, c.ws + 4096, nullptr) == QMV_OK);
  }
  // the 32-bit activation granule index bounds m * k / 8
  const int big_k = 1 << 20;
  const size_t wb = mbytes(4, big_k, 256, 144);
  const uint16_t *xbig = static_cast<const uint16_t *>(at(16));   // 64 GiB of activations, clear of the rest
  EXPECT(qmm_q4_k_prefill(W, wb, xbig, Y, 1 << 15, 4, big_k, WS, (size_t)1 << 40, nullptr) == QMV_OK);
  EXPECT(qmm_q4_k_prefill(W, wb, xbig, Y, (1 << 15) + 1, 4, big_k, WS, (size_t)1 << 40, nullptr) == QMV_ERR_RANGE);
  for (int m : kInts)
    for (int n : kInts)
      for (int k : kInts) {
        (void)qmm_q4_k_prefill_workspace(m, n, k);
        const size_t b = mbytes(n, k, 256, 144);
        EXPECT(is_code(qmm_q4_k_prefill(W, b ? b : 1, xb, Y, m, n, k, WS, (size_t)1 << 40, nullptr)));
      }
}

void stream_read() {
  uint32_t *sink = static_cast<uint32_t *>(at(2));
  EXPECT(qmv_stream_read(W, 1 << 20, sink, 2048, 4, 1, nullptr) == QMV_OK);
  EXPECT(stub::last_m == 2048 && stub::last_n == 4 && stub::last_k == 1);
  EXPECT(qmv_stream_read(W, 16, sink, 1, 1, 2, nullptr) == QMV_ERR_RANGE);
  EXPECT(qmv_stream_read(nullptr, 16, sink, 1, 1, 0, nullptr) == QMV_ERR_NULL);
  EXPECT(qmv_stream_read(W, 0, sink, 1, 1, 0, nullptr) == QMV_ERR_SIZE);
  EXPECT(qmv_stream_read(W, 24, sink, 1, 1, 0, nullptr) == QMV_ERR_SIZE);
  EXPECT(qmv_stream_read(W, 16, sink, 1, 3, 0, nullptr) == QMV_ERR_RANGE);
  EXPECT(qmv_stream_read(W, 16, sink, 65537, 1, 0, nullptr) == QMV_ERR_RANGE);
  EXPECT(qmv_stream_read(at(0, 8), 16, sink, 1, 1, 0, nullptr) == QMV_ERR_ALIGN);
  EXPECT(qmv_stream_read(W, 1 << 20, static_cast<uint32_t *>(at(0, 1024)), 4, 1, 0, nullptr) == QMV_ERR_ALIAS);
  for (int g : kInts)
    for (int u : kInts) EXPECT(is_code(qmv_stream_read(W, 4096, sink, g, u, u & 3, nullptr)));
}

}  // namespace

int main() {
  EXPECT(qmv_version() > 0);
  for (int c = -20; c <= 20; ++c) EXPECT(qmv_strerror(c) != nullptr && qmv_strerror(c)[0] != '\0');
  EXPECT(qmv_last_error() != nullptr);
  dense_formats();
  pair();
  q8_0();
  dequant();
  moe(qmv_q4_k_moe, qmv_q4_k_moe_workspace, 144);
  moe(qmv_iq4_xs_moe, qmv_iq4_xs_moe_workspace, 136);
  moe_noalloc();
  moe_prefill();
  prefill();
  stream_read();
  printf("validation driver: %d launches reached, %d failures\n", stub::launches, failures);
  return failures ? 1 : 0;
}
