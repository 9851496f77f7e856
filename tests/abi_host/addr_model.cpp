// Host model of every weight load the kernels issue. It runs the kernels' own
// address functions (qmv_addr.h: the launch plans, the per-lane bases, step
// and unit offsets and read windows the kernels form their pointers with) over
// every lane of the workgroups a launch runs, every step and unit it issues,
// for the instantiations the entry points pick over a sweep of shapes, and
// checks that
//   * every read [off, off + len) lies inside the weight array, and
//   * every read whose data is used lies in the lane's own row (own expert
//     matrix, own K range) -- loads with no data of their own may read any
//     block inside the array.
// Built with g++ (and the sanitizers) by tests/test_addr_model.py; no GPU.
//
//   addr_model            run the sweep; exit 0 when every read is in bounds
//   addr_model --prefix   the dense GEMV with its earlier step rule (every
//                         step below the row's step count counted as its own,
//                         the partial last step included): must report reads
//                         past the weights at K = 17408
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../gguf_block_quantized_qmv_amd/csrc/qmv_addr.h"

using namespace qmv;
using addr::Window;

namespace {

bool g_prefix = false;
long long g_reads = 0, g_bad = 0, g_outside = 0, g_foreign = 0;
long long g_max_over = 0;   // furthest any read ends past the array
int g_reported = 0;

void fail(const std::string &what) {
  ++g_bad;
  if (g_reported++ < 12) std::printf("VIOLATION %s\n", what.c_str());
}

// One read of `len` bytes at byte `base + w.off` of a `total`-byte array; when
// `own_lo < own_hi` the read is used and must also lie in [own_lo, own_hi).
void check(const char *what, size_t base, Window w, size_t total, size_t own_lo = 0, size_t own_hi = 0) {
  if (w.len == 0) return;
  ++g_reads;
  const long long lo = (long long)base + w.off, hi = lo + w.len;
  if (lo < 0 || (unsigned long long)hi > total) {
    ++g_outside;
    if (hi - (long long)total > g_max_over) g_max_over = hi - (long long)total;
    char b[256];
    std::snprintf(b, sizeof b, "%s: read [%lld, %lld) outside the %zu-byte weights", what, lo, hi, total);
    fail(b);
  } else if (own_lo < own_hi && ((size_t)lo < own_lo || (size_t)hi > own_hi)) {
    ++g_foreign;
    char b[256];
    std::snprintf(b, sizeof b, "%s: used read [%lld, %lld) outside its own range [%zu, %zu)", what, lo, hi, own_lo,
                  own_hi);
    fail(b);
  }
}

// Workgroups whose lanes are enumerated: all of them up to 8, else the first
// and last three (rows differ only in their index, and in being past the matrix).
std::vector<unsigned> groups_of(unsigned grid) {
  std::vector<unsigned> g;
  if (grid <= 8) {
    for (unsigned i = 0; i < grid; ++i) g.push_back(i);
  } else {
    for (unsigned i = 0; i < 3; ++i) g.push_back(i);
    for (unsigned i = grid - 3; i < grid; ++i) g.push_back(i);
  }
  return g;
}

// ---- dense GEMV (Q4_K, Q5_K, Q4_0) ------------------------------------------

// Steps the kernel issues loads for, in order: the ring's first D, then (NS > 0)
// step s + D after each step s with s + D < NS, or (NS == 0) step s + D after
// every step s of the runtime loop, which runs whole rounds of D.
std::vector<int> ring_steps(int ns, int nsteps, int depth) {
  std::vector<int> t;
  for (int u = 0; u < depth; ++u) t.push_back(u);
  if (ns > 0) {
    for (int s = 0; s < ns; ++s)
      if (s + depth < ns) t.push_back(s + depth);
  } else {
    for (int s0 = 0; s0 < nsteps; s0 += depth)
      for (int u = 0; u < depth; ++u) t.push_back(s0 + u + depth);
  }
  return t;
}

void dense_case(int fmt, int m, int n, int k) {
  const addr::GemvPlan p = addr::dense_gemv_plan(fmt, m, n, k);
  const int nblk = k >> 8, bb = addr::dense_block_bytes(fmt);
  const size_t total = (size_t)n * nblk * bb, row_bytes = (size_t)nblk * bb;
  const int threads = p.rows * p.G;
  char what[160];
  std::snprintf(what, sizeof what, "dense fmt %d m %d n %d k %d (G %d NS %d D %d rows %d)", fmt, m, n, k, p.G, p.ns,
                p.depth, p.rows);
  if (threads < 64 || threads % 64 || threads > addr::dense_max_threads(m)) fail(std::string(what) + ": workgroup");
  if ((size_t)p.grid * p.rows < (size_t)n) fail(std::string(what) + ": grid does not cover the rows");
  for (unsigned bid : groups_of(p.grid)) {
    for (int tid = 0; tid < threads; ++tid) {
      const int j = (tid & 63) & (p.G - 1);
      const int row = addr::lane_row((int)bid, tid, threads, p.G);
      const addr::DenseLane l = addr::dense_lane(p.G, p.ns, fmt, n, nblk, row, j);
      for (int t : ring_steps(p.ns, l.nsteps, p.depth)) {
        bool ok = addr::dense_step_ok(l.active, l.last_ok, l.nsteps, l.jb, p.ns, p.full, p.G, nblk, t);
        if (g_prefix) ok = l.active && t < l.nsteps;   // the earlier rule
        const size_t b = ok ? l.row_base + l.blk_off + addr::dense_step_offset(p.G, fmt, t) : l.fb;
        const size_t lo = ok ? (size_t)row * row_bytes : 0, hi = ok ? lo + row_bytes : 0;
        for (int i = 0; i < 2; ++i) check(what, b, addr::dense_window(fmt, l.c, i), total, lo, hi);
      }
    }
  }
}

// Two matrices on one activation (qmv_q4_k_pair): one grid over 2n rows, each
// lane reading its own matrix (addr::pair_row); both matrices are `total` bytes.
void pair_case(int m, int n, int k) {
  const int fmt = addr::kFmtQ4K;
  const addr::GemvPlan p = addr::dense_gemv_plan(fmt, m, 2 * n, k);
  const int nblk = k >> 8, bb = addr::dense_block_bytes(fmt);
  const size_t total = (size_t)n * nblk * bb, row_bytes = (size_t)nblk * bb;
  const int threads = p.rows * p.G;
  char what[160];
  std::snprintf(what, sizeof what, "pair m %d n %d k %d (G %d NS %d D %d rows %d)", m, n, k, p.G, p.ns, p.depth,
                p.rows);
  if ((size_t)p.grid * p.rows < 2 * (size_t)n) fail(std::string(what) + ": grid does not cover the rows");
  for (unsigned bid : groups_of(p.grid)) {
    for (int tid = 0; tid < threads; ++tid) {
      const int j = (tid & 63) & (p.G - 1);
      const addr::PairRow pr = addr::pair_row(addr::lane_row((int)bid, tid, threads, p.G), n);
      const addr::DenseLane l = addr::dense_lane(p.G, p.ns, fmt, n, nblk, pr.row, j);
      for (int t : ring_steps(p.ns, l.nsteps, p.depth)) {
        const bool ok = addr::dense_step_ok(l.active, l.last_ok, l.nsteps, l.jb, p.ns, p.full, p.G, nblk, t);
        const size_t b = ok ? l.row_base + l.blk_off + addr::dense_step_offset(p.G, fmt, t) : l.fb;
        const size_t lo = ok ? (size_t)pr.row * row_bytes : 0, hi = ok ? lo + row_bytes : 0;
        for (int i = 0; i < 2; ++i) check(what, b, addr::dense_window(fmt, l.c, i), total, lo, hi);
      }
    }
  }
}

// ---- Q6_K GEMV --------------------------------------------------------------

void q6_case(int m, int n, int k) {
  const addr::GemvPlan p = addr::q6_gemv_plan(m, n, k);
  const int nblk = k >> 8;
  const size_t total = (size_t)n * nblk * addr::kQ6KBytes, row_bytes = (size_t)nblk * addr::kQ6KBytes;
  const int threads = p.rows * p.G;
  char what[160];
  std::snprintf(what, sizeof what, "q6_k m %d n %d k %d (G %d NS %d D %d rows %d)", m, n, k, p.G, p.ns, p.depth,
                p.rows);
  if (threads < 64 || threads % 64 || threads > addr::q6_max_threads(m)) fail(std::string(what) + ": workgroup");
  for (unsigned bid : groups_of(p.grid)) {
    for (int tid = 0; tid < threads; ++tid) {
      const int j = (tid & 63) & (p.G - 1);
      const int row = addr::lane_row((int)bid, tid, threads, p.G);
      const addr::Q6Lane l = addr::q6_lane(p.G, p.ns, n, nblk, row, j);
      for (int t : ring_steps(p.ns, l.nsteps, p.depth)) {
        const bool ok = addr::q6_step_ok(l, p.G, nblk, t);
        const size_t b = ok ? l.base + addr::q6_step_offset(p.G, t) : l.fb;
        // the block's dword offset must be the lane's sb (a step moves an even number of blocks)
        if (b % 4 != (size_t)l.sb) fail(std::string(what) + ": block offset is not sb");
        // a used read may start in the last 2 bytes of the previous block
        const size_t lo = ok ? (size_t)row * row_bytes : 0, hi = ok ? lo + row_bytes : 0;
        for (int i = 0; i < addr::kQ6Windows; ++i) {
          const Window w = addr::q6_window(l.sb, l.h, l.p, i);
          check(what, b, w, total, ok ? (lo >= 2 ? lo - 2 : 0) : 0, hi);
        }
      }
    }
  }
}

// ---- IQ4_XS GEMV --------------------------------------------------------------

// Units the kernel issues, in order: the ring's first `depth`, then unit
// t + depth after each unit t of the nslots.
std::vector<int> unit_steps(int nslots, int depth) {
  std::vector<int> t;
  for (int d = 0; d < depth; ++d) t.push_back(d);
  for (int s = 0; s < nslots; ++s) t.push_back(s + depth);
  return t;
}

void iq4_case(int m, int n, int k) {
  const addr::Iq4Plan p = addr::iq4_gemv_plan(m, n, k);
  const int nblk = k >> 8;
  const size_t row_bytes = (size_t)nblk * addr::kIQ4XSBytes, total = (size_t)n * row_bytes;
  char what[160];
  std::snprintf(what, sizeof what, "iq4_xs m %d n %d k %d (G %d T %d)", m, n, k, p.G, p.threads);
  if ((size_t)p.grid * (p.threads / p.G) < (size_t)n) fail(std::string(what) + ": grid does not cover the rows");
  const int nslots = addr::iq4_slots(p.G, nblk, p.depth);
  for (unsigned bid : groups_of(p.grid)) {
    for (int tid = 0; tid < p.threads; ++tid) {
      const int row = addr::lane_row((int)bid, tid, p.threads, p.G), l = tid % p.G;
      const addr::Iq4Lane ln = addr::iq4_lane(p.G, nblk, (size_t)(row < n ? row : 0), l);
      for (int t : unit_steps(nslots, p.depth)) {
        const bool live = t < ln.nlive;
        const size_t b = live ? ln.lane_base + addr::iq4_unit_offset(t, ln.unit_bytes) : ln.row_base;
        const bool used = live && row < n;
        const size_t lo = used ? (size_t)row * row_bytes : 0, hi = used ? lo + row_bytes : 0;
        for (int i = 0; i < 2; ++i) check(what, b, addr::iq4_window(ln.qoff, i), total, lo, hi);
      }
    }
  }
}

// ---- routed-expert decode ------------------------------------------------------

void moe_q4k_case(int T, int hidden, int ffn, int E, int K) {
  const int nblk_up = hidden >> 8, nblk_dn = ffn >> 8;
  const size_t up_row = (size_t)nblk_up * addr::kQ4KBytes, up_total = (size_t)E * ffn * up_row;
  const size_t dn_row = (size_t)nblk_dn * addr::kQ4KBytes, dn_total = (size_t)E * hidden * dn_row;
  const size_t expert_bytes = (size_t)hidden * dn_row;
  const int max_slots = E < T * K ? E : T * K;
  char what[160];
  std::snprintf(what, sizeof what, "q4_k moe T %d hidden %d ffn %d E %d K %d", T, hidden, ffn, E, K);
  const int up_rows = addr::moe_up_rows(T), up_lanes = addr::moe_up_lanes(T);
  const unsigned gx = (unsigned)((ffn + up_rows - 1) / up_rows);
  for (int e : {0, E - 1}) {
    for (unsigned bx : groups_of(gx)) {
      for (int tid = 0; tid < addr::kMoeThreads; ++tid) {
        const addr::MoeUpLane l = addr::moe_up_lane(up_lanes, e, ffn, hidden, (int)bx, tid);
        for (int s = 0; s < l.nsteps + addr::kMoeUpDepth; ++s) {
          if (!addr::moe_up_step_ok(l, nblk_up, s)) continue;
          const size_t b = addr::moe_up_step_at(l.base, l.bps, s);
          const size_t lo = ((size_t)e * ffn + l.f) * up_row, hi = lo + up_row;
          for (int i = 0; i < 2; ++i) check(what, b, addr::dense_window(addr::kFmtQ4K, l.c, i), up_total, lo, hi);
        }
      }
    }
  }
  const unsigned gd = (unsigned)((hidden + addr::kMoeDnRows - 1) / addr::kMoeDnRows);
  for (int n_slots = 1; n_slots <= max_slots; ++n_slots) {
    for (int e : {0, E - 1}) {
      for (unsigned bx : groups_of(gd)) {
        for (int tid = 0; tid < addr::kMoeThreads; ++tid) {
          const addr::MoeDnLane l = addr::moe_dn_lane(hidden, ffn, n_slots, (int)bx, tid);
          int ls = l.grp, lb = 0;
          for (int u = 0; u < l.units; ++u) {   // the kernel loads exactly units 0 .. U - 1
            if (ls >= n_slots) fail(std::string(what) + ": slot index past the table");
            const size_t b = addr::moe_dn_unit_at(l.row, e, expert_bytes, lb);
            const int row = l.n < hidden ? l.n : 0;
            const size_t lo = (size_t)e * expert_bytes + (size_t)row * dn_row, hi = lo + dn_row;
            for (int i = 0; i < 2; ++i) check(what, b, addr::moe_dn_window(l.c, i), dn_total, lo, hi);
            addr::moe_dn_next(ls, lb, nblk_dn, addr::kMoeDnGroups);
          }
        }
      }
    }
  }
}

void moe_iq4_case(int T, int hidden, int ffn, int E, int K) {
  const int nblk_up = hidden >> 8, nblk_dn = ffn >> 8;
  const size_t up_row = (size_t)nblk_up * addr::kIQ4XSBytes, up_total = (size_t)E * ffn * up_row;
  const size_t dn_row = (size_t)nblk_dn * addr::kIQ4XSBytes, dn_total = (size_t)E * hidden * dn_row;
  const size_t expert_bytes = (size_t)hidden * dn_row;
  const int max_slots = E < T * K ? E : T * K;
  char what[160];
  std::snprintf(what, sizeof what, "iq4_xs moe T %d hidden %d ffn %d E %d K %d", T, hidden, ffn, E, K);
  const int up_lanes = addr::iq4_moe_up_lanes(T), up_rows = addr::iq4_moe_up_rows(T);
  const unsigned gx = (unsigned)((ffn + up_rows - 1) / up_rows);
  const int nslots = addr::iq4_slots(up_lanes, nblk_up, addr::kIq4MoeUpDepth);
  for (int e : {0, E - 1}) {
    for (unsigned bx : groups_of(gx)) {
      for (int tid = 0; tid < 64 * addr::kIq4MoeDnWaves; ++tid) {
        const int f = (int)bx * up_rows + tid / up_lanes;
        const addr::Iq4Lane ln = addr::iq4_moe_up_lane(up_lanes, e, ffn, hidden, (int)bx, tid);
        for (int t : unit_steps(nslots, addr::kIq4MoeUpDepth)) {
          const bool live = t < ln.nlive;
          const size_t b = live ? ln.lane_base + addr::iq4_unit_offset(t, ln.unit_bytes) : ln.row_base;
          const bool used = live && f < ffn;
          const size_t lo = used ? ((size_t)e * ffn + f) * up_row : 0, hi = used ? lo + up_row : 0;
          for (int i = 0; i < 2; ++i) check(what, b, addr::iq4_window(ln.qoff, i), up_total, lo, hi);
        }
      }
    }
  }
  const unsigned gd = (unsigned)((hidden + addr::kIq4MoeDnRows - 1) / addr::kIq4MoeDnRows);
  const int D = addr::kIq4MoeDnDepth;
  for (int n_slots = 1; n_slots <= max_slots; ++n_slots) {
    for (int e : {0, E - 1}) {
      for (unsigned bx : groups_of(gd)) {
        for (int tid = 0; tid < 64 * addr::kIq4MoeDnWaves; ++tid) {
          const addr::Iq4DnLane l = addr::iq4_moe_dn_lane(hidden, ffn, n_slots, (int)bx, tid);
          const int n = (int)bx * addr::kIq4MoeDnRows + (tid & 63) / addr::kIq4MoeDnLanes;
          int ls = l.wave, lb = 0;
          // one load per ring slot: unit (ls, lb) while units remain, else
          // slot 0, block 0 (any expert the table holds)
          auto load = [&](bool ok) {
            if (ok && ls >= n_slots) fail(std::string(what) + ": slot index past the table");
            const size_t b = addr::iq4_moe_dn_unit_at(l.row, e, expert_bytes, ok ? lb : 0);
            const size_t lo = ok && n < hidden ? (size_t)e * expert_bytes + (size_t)n * dn_row : 0;
            const size_t hi = ok && n < hidden ? lo + dn_row : 0;
            for (int i = 0; i < 2; ++i) check(what, b, addr::iq4_window(l.qoff, i), dn_total, lo, hi);
            if (ok) addr::moe_dn_next(ls, lb, nblk_dn, addr::kIq4MoeDnWaves);
          };
          for (int u = 0; u < D; ++u) load(u < l.units);
          for (int u0 = 0; u0 < l.units; u0 += D)
            for (int u = 0; u < D; ++u)
              if (u0 + u < l.units) load(u0 + u + D < l.units);
        }
      }
    }
  }
}

// ---- prefill GEMM --------------------------------------------------------------

void prefill_case(int m, int n, int k) {
  const layout::PrefillPlan p = layout::prefill_plan(m, n, k);
  const int BM = layout::kPrefillTileM, BN = layout::kPrefillTileN;
  const int m_tiles = (m + BM - 1) / BM, n_tiles = (n + BN - 1) / BN, tiles = m_tiles * n_tiles;
  const int blocks = p.t_main + p.r_tiles * p.splits;
  const int nblk = k >> 8, gpr = k >> 3, kDepth = 4, tpr = addr::kPrefillHalf / BN, x_per_thread = BM * 8 / addr::kPrefillHalf;
  const size_t row_bytes = (size_t)nblk * addr::kQ4KBytes, total = (size_t)n * row_bytes;
  const size_t x_total = (size_t)m * gpr;
  char what[160];
  std::snprintf(what, sizeof what, "prefill m %d n %d k %d (t_main %d r_tiles %d splits %d)", m, n, k, p.t_main,
                p.r_tiles, p.splits);
  // every tile once, every split tile's K blocks once, in part order
  std::vector<int> seen(tiles, 0);
  std::vector<int> kcover((size_t)tiles, 0);
  for (int blk = 0; blk < blocks; ++blk) {
    const addr::PrefillWork wk = addr::prefill_work(blk, k, p.t_main, p.r_tiles, p.splits);
    if (wk.tile < 0 || wk.tile >= tiles) { fail(std::string(what) + ": tile index"); continue; }
    int mt, nt;
    addr::tile_of(wk.tile, m_tiles, n_tiles, mt, nt);
    if (mt < 0 || mt >= m_tiles || nt < 0 || nt >= n_tiles) fail(std::string(what) + ": tile position");
    if (wk.slot < 0) {
      seen[(size_t)mt * n_tiles + nt] += 1;
      kcover[(size_t)mt * n_tiles + nt] += wk.nsteps;
    } else {
      if (kcover[(size_t)mt * n_tiles + nt] != wk.s_begin) fail(std::string(what) + ": split parts out of K order");
      kcover[(size_t)mt * n_tiles + nt] += wk.nsteps;
      if (wk.s_begin + wk.nsteps == k / addr::kPrefillBK) seen[(size_t)mt * n_tiles + nt] += 1;
    }
    if (wk.nsteps <= 0 || wk.nsteps % kDepth) fail(std::string(what) + ": step count");
    // producer loads of the blocks near the ends of the launch and of every
    // part of the first and last split tile
    const int rb = blk - p.t_main;
    const bool split_edge = wk.slot >= 0 && (rb % p.r_tiles == 0 || rb % p.r_tiles == p.r_tiles - 1);
    if (!(blk < 4 || (blk >= p.t_main - 4 && blk < p.t_main) || blk >= blocks - 4 || split_edge)) continue;
    const int n0 = nt * BN, m0 = mt * BM;
    std::vector<int> steps;
    for (int u = 0; u < kDepth; ++u) steps.push_back(u);
    steps.push_back(kDepth);
    for (int s0 = 0; s0 < wk.nsteps; s0 += kDepth)
      for (int u = 0; u < kDepth; ++u) steps.push_back(s0 + u + 1 + kDepth);
    for (int pt = 0; pt < addr::kPrefillHalf; ++pt) {
      const size_t wr = addr::prefill_w_row(n0, n, k, wk.s_begin, pt, tpr);
      const int w_row = n0 + pt / tpr;
      for (int s_issued : steps) {
        const int s = addr::prefill_clamp(s_issued, wk.nsteps);
        const size_t b = wr + addr::prefill_w_step(s);
        const bool used = w_row < n;
        const size_t lo = used ? (size_t)w_row * row_bytes : 0, hi = used ? lo + row_bytes : 0;
        for (int i = 0; i < 2; ++i) check(what, b, addr::prefill_w_window(s, pt, tpr, i), total, lo, hi);
        for (int i = 0; i < x_per_thread; ++i) {
          // granules from step s_begin of row 0, as the kernel's base pointer does
          const size_t g = (size_t)wk.s_begin * 8 + addr::prefill_x_granule(pt, i, m0, m, gpr, s);
          const int row = m0 + ((pt + addr::kPrefillHalf * i) >> 3);
          const size_t lo2 = row < m ? (size_t)row * gpr : 0, hi2 = row < m ? lo2 + gpr : 0;
          check(what, g * 16, Window{0, 16}, x_total * 16, lo2 * 16, hi2 * 16);
        }
      }
    }
  }
  for (int t = 0; t < tiles; ++t)
    if (seen[t] != 1 || kcover[t] != k / addr::kPrefillBK) fail(std::string(what) + ": tile coverage");
}

// ---- routed-expert prefill (grouped) ---------------------------------------------

void group_matrix(const char *what, int E, int rows, int kdim, int nwaves, int tpw) {
  const int nblk = kdim >> 8;
  const size_t row_bytes = (size_t)nblk * addr::kQ4KBytes, total = (size_t)E * rows * row_bytes;
  const int per_group = nwaves * addr::kGroupTile * tpw;
  if (rows % per_group) {
    fail(std::string(what) + ": the grid does not cover the rows exactly");
    return;
  }
  const unsigned gx = (unsigned)(rows / per_group);
  for (int e : {0, E - 1}) {
    for (unsigned bx : groups_of(gx)) {
      for (int wv = 0; wv < nwaves; ++wv) {
        for (int l = 0; l < 64; ++l) {
          const int kg = l >> 4;
          for (int tt = 0; tt < tpw; ++tt) {
            const size_t r = addr::group_row(e, rows, (int)bx, nwaves, wv, tpw, tt, l);
            if (r < (size_t)e * rows || r >= (size_t)(e + 1) * rows) fail(std::string(what) + ": row past the expert");
            // block 0, then block b + 1 (clamped) while block b is multiplied
            std::vector<int> blocks_read = {0};
            for (int b = 0; b < nblk; ++b) blocks_read.push_back(b + 1);
            for (int b : blocks_read) {
              const size_t base = r * row_bytes + addr::group_block(b, nblk);
              for (int i = 0; i < addr::kGroupWindows; ++i)
                check(what, base, addr::group_window(kg, i), total, r * row_bytes, (r + 1) * row_bytes);
            }
          }
        }
      }
    }
  }
}

void grouped_case(int T, int hidden, int ffn, int E, int K) {
  const int P = T * K, tpw = addr::group_tiles_per_wave(P);
  const bool wide = P >= 2048 && layout::group_gate_up_lds(layout::kGroupChunk32, hidden) <= layout::kLdsBudget;
  char what[160];
  std::snprintf(what, sizeof what, "grouped T %d hidden %d ffn %d E %d K %d", T, hidden, ffn, E, K);
  if (wide) group_matrix(what, E, ffn, hidden, addr::kGroupWideWaves, addr::kGroupWideTiles);
  else group_matrix(what, E, ffn, hidden, 4, tpw);
  group_matrix(what, E, hidden, ffn, 4, tpw);
}

// ---- Q8_0 GEMV ----------------------------------------------------------------------

void q80_case(int m, int n, int k) {
  (void)m;
  const int nblk = k >> 5;
  const size_t row_bytes = (size_t)nblk * addr::kQ80Bytes, total = (size_t)n * row_bytes;
  char what[96];
  std::snprintf(what, sizeof what, "q8_0 n %d k %d", n, k);
  const unsigned grid = (unsigned)((n + 7) / 8);   // 4 waves of two 32-lane rows
  for (unsigned bid : groups_of(grid)) {
    for (int tid = 0; tid < 256; ++tid) {
      const int lane = tid & 63, j = lane & 31;
      const int row = ((int)bid * 4 + (tid >> 6)) * 2 + lane / 32;
      if (row >= n) continue;
      for (int b = j; b < nblk; b += 32) {
        const size_t off = ((size_t)row * nblk + b) * addr::kQ80Bytes;
        const size_t lo = (size_t)row * row_bytes;
        check(what, off, addr::q80_window(off), total, lo >= 2 ? lo - 2 : 0, lo + row_bytes);
      }
    }
  }
}

}  // namespace

int main(int argc, char **argv) {
  for (int i = 1; i < argc; ++i)
    if (!std::strcmp(argv[i], "--prefix")) g_prefix = true;

  if (g_prefix) {
    // the down-projection shape of the memra README's 8B decode rows
    for (int m = 1; m <= 4; ++m)
      if (layout::q4k_x_lds(m, 17408) <= layout::kLdsBudget) dense_case(addr::kFmtQ4K, m, 5120, 17408);
    std::printf("prefix rule: %lld reads, %lld past the weights (up to %lld bytes past the end), %lld used reads "
                "outside their row\n", g_reads, g_outside, g_max_over, g_foreign);
    return g_outside ? 3 : 0;
  }

  auto t0 = std::chrono::steady_clock::now();
  auto lap = [&](const char *name) {
    const auto t1 = std::chrono::steady_clock::now();
    std::printf("%-28s %8.2f s  %lld reads so far\n", name, std::chrono::duration<double>(t1 - t0).count(), g_reads);
    t0 = t1;
  };
  // dense GEMV: every row length up to the unrolled limit, the runtime loop
  // beyond, and row counts that take each workgroup shape
  const int ns_[] = {1, 3, 255, 256, 768, 2048, 5120, 17408};
  std::vector<int> ks;
  for (int k = 256; k <= 18432; k += 256) ks.push_back(k);
  for (int k : {18688, 20480, 24576, 32768, 40960}) ks.push_back(k);
  for (int fmt : {addr::kFmtQ4K, addr::kFmtQ5K, addr::kFmtQ40})
    for (int m = 1; m <= 4; ++m)
      for (int k : ks) {
        if (layout::q4k_x_lds(m, k) > layout::kLdsBudget) continue;
        for (int n : ns_) dense_case(fmt, m, n, k);
      }
  lap("dense GEMV");
  for (int m = 1; m <= 4; ++m)
    for (int k : {256, 1024, 5120, 8448, 17408, 18432, 20480})
      if (layout::q4k_x_lds(m, k) <= layout::kLdsBudget)
        for (int n : {1, 3, 255, 256, 2560, 17408}) pair_case(m, n, k);
  lap("Q4_K pair GEMV");
  for (int m = 1; m <= 4; ++m)
    for (int k : ks) {
      if (layout::q6k_x_lds(m, k) > layout::kLdsBudget) continue;
      for (int n : ns_) q6_case(m, n, k);
    }
  lap("Q6_K GEMV");
  for (int m = 1; m <= 4; ++m)
    for (int k : ks) {
      if (layout::iq4xs_gemv_lds(m, k) > layout::kLdsBudget) continue;
      for (int n : ns_) iq4_case(m, n, k);
    }
  lap("IQ4_XS GEMV");
  for (int m = 1; m <= 4; ++m)
    for (int k : {32, 64, 96, 1024, 4096, 5120, 5152, 8192}) {
      if (layout::q80_x_lds(m, k) > layout::kLdsBudget) continue;
      for (int n : {1, 3, 17, 256, 5120}) q80_case(m, n, k);
    }
  lap("Q8_0 GEMV");
  // the largest matrices the entry points take (2^40 weights): first and last workgroups
  dense_case(addr::kFmtQ4K, 1, 1 << 24, 1 << 16);
  dense_case(addr::kFmtQ4K, 1, 1 << 30, 1 << 10);
  q6_case(1, 1 << 24, 1 << 16);
  iq4_case(1, 1 << 24, 1 << 16);

  lap("largest matrices");
  // routed-expert decode: the 35B-A3B layer (hidden 2048, ffn 768, 128
  // experts, top-8), ragged and one-expert cases, and rows whose last pass is
  // partial at both lane widths (5 and 18 blocks)
  for (int T = 1; T <= 4; ++T) {
    for (auto c : {std::vector<int>{2048, 768, 128, 8}, {256, 256, 1, 1}, {512, 1280, 16, 3}, {4096, 512, 64, 8},
                   {1280, 256, 16, 4}, {4608, 256, 16, 4}}) {
      if (layout::q4k_moe_fits_lds(T, c[0], c[1], c[3])) moe_q4k_case(T, c[0], c[1], c[2], c[3]);
      if (layout::iq4xs_moe_fits_lds(T, c[0], c[1], c[3])) moe_iq4_case(T, c[0], c[1], c[2], c[3]);
    }
  }
  lap("routed-expert decode");
  // routed-expert prefill: pair counts that take each tile count and the wide gate/up
  for (int T : {1, 16, 64, 255, 256, 512})
    for (auto c : {std::vector<int>{2048, 768, 128, 8}, {256, 256, 1, 1}, {512, 1280, 16, 3}})
      if (layout::group_fits_lds(c[0], c[1])) grouped_case(T, c[0], c[1], c[2], c[3]);

  lap("routed-expert prefill");
  // prefill GEMM: whole-tile and K-split launches, ragged M and N
  for (int m : {1, 64, 128, 200, 512, 1000})
    for (int n : {128, 300, 5120, 17408})
      for (int k : {256, 1024, 5120, 17408}) prefill_case(m, n, k);

  lap("prefill GEMM");
  std::printf("%lld reads checked: %lld past the weights, %lld used reads outside their row, %lld other "
              "violations\n", g_reads, g_outside, g_foreign, g_bad - g_outside - g_foreign);
  return g_bad ? 1 : 0;
}
