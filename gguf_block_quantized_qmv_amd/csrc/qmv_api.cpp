// C ABI of the block-quantized matrix-vector library: argument validation and
// dispatch. Pure host code: it calls no HIP function and reads no device
// property, so a call's checks -- and the sizes and plans they take from
// qmv_layout.h -- depend on its arguments alone. The CPU tests link this file
// with stand-in launchers and no HIP runtime at all, under the address and
// undefined-behaviour sanitizers. See include/qmv.h for the contract of each
// entry point.
#include "../../include/qmv.h"

#include <stdint.h>
#include <stdio.h>

#include "qmv_internal.h"
#include "qmv_layout.h"

namespace qmv {

// Text of the last HIP failure seen by this thread (qmv_last_error).
thread_local char g_error_detail[256] = "";

void set_error_detail(const char *what, int hip_code, const char *hip_text) {
  snprintf(g_error_detail, sizeof(g_error_detail), "%s: hip error %d (%s)", what ? what : "?", hip_code,
           hip_text ? hip_text : "?");
}

}  // namespace qmv

namespace {

constexpr int kVersion = 10000 * 0 + 100 * 3 + 0;  // 0.3.0

// a*b*c with overflow detection.
bool mul_size(size_t a, size_t b, size_t *out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p+pb) and [q, q+qb) share a byte.
bool overlap(const void *p, size_t pb, const void *q, size_t qb) {
  if (pb == 0 || qb == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qb && b < a + pb;
}

// Byte size of a row-major block-quantized matrix, 0 on overflow.
size_t matrix_bytes(int n, int k, int block_weights, int block_bytes) {
  size_t blocks = 0, bytes = 0;
  if (!mul_size((size_t)n, (size_t)(k / block_weights), &blocks)) return 0;
  if (!mul_size(blocks, (size_t)block_bytes, &bytes)) return 0;
  return bytes;
}

// Common checks of a row-major quantized matrix argument.
int check_matrix(const void *w, size_t w_bytes, int n, int k, int block_weights, int block_bytes,
                 uintptr_t w_align) {
  if (!w) return QMV_ERR_NULL;
  if (n <= 0 || k <= 0 || k % block_weights != 0) return QMV_ERR_SHAPE;
  if (!qmv::layout::matrix_in_range(n, k)) return QMV_ERR_RANGE;
  const size_t expect = matrix_bytes(n, k, block_weights, block_bytes);
  if (expect == 0 || w_bytes != expect) return QMV_ERR_SIZE;
  if (!aligned(w, w_align)) return QMV_ERR_ALIGN;
  return QMV_OK;
}

}  // namespace

namespace {

enum class MoeFormat { kQ4K, kIQ4XS };

bool moe_args_ok(MoeFormat f, int t, int hidden, int ffn, int n_experts, int top_k) {
  return t >= 1 && t <= QMV_MOE_MAX_TOKENS && n_experts >= 1 && n_experts <= QMV_MOE_MAX_EXPERTS && top_k >= 1 &&
         top_k <= QMV_MOE_MAX_TOP_K && top_k <= n_experts && hidden > 0 && ffn > 0 && hidden % 256 == 0 &&
         ffn % 256 == 0 &&
         (f == MoeFormat::kQ4K ? qmv::layout::q4k_moe_fits_lds(t, hidden, ffn, top_k)
                               : qmv::layout::iq4xs_moe_fits_lds(t, hidden, ffn, top_k));
}

// Host-side checks of a routed-expert decode call of t tokens. caller_ws: the
// call brings its own workspace (ws, ws_bytes); otherwise it runs in the
// library's fixed scratch array, which must hold the call's workspace.
int moe_check(MoeFormat f, const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
              const float *logits, const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w,
              int32_t *pairs, void *ws, size_t ws_bytes, int t, int hidden, int ffn, int n_experts,
              int top_k, bool caller_ws = true) {
  if (!w_gate || !w_up || !w_down || !logits || !x_bf16 || !y) return QMV_ERR_NULL;
  if (t < 1 || t > QMV_MOE_MAX_TOKENS || n_experts < 1 || n_experts > QMV_MOE_MAX_EXPERTS ||
      top_k < 1 || top_k > QMV_MOE_MAX_TOP_K || top_k > n_experts)
    return QMV_ERR_RANGE;
  if (hidden <= 0 || ffn <= 0 || hidden % 256 || ffn % 256) return QMV_ERR_SHAPE;
  if (!moe_args_ok(f, t, hidden, ffn, n_experts, top_k)) return QMV_ERR_RANGE;
  const size_t block_bytes = f == MoeFormat::kQ4K ? 144 : 136;
  const size_t w_align = f == MoeFormat::kQ4K ? 16 : 8;
  size_t expert_bytes = 0, bank = 0;
  if (!mul_size((size_t)ffn, (size_t)(hidden / 256) * block_bytes, &expert_bytes) ||
      !mul_size(expert_bytes, (size_t)n_experts, &bank) || bank_bytes != bank)
    return QMV_ERR_SIZE;
  if (!aligned(w_gate, w_align) || !aligned(w_up, w_align) || !aligned(w_down, w_align) || !aligned(x_bf16, 16) ||
      !aligned(logits, 4) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(pairs, 4) ||
      !aligned(ws, 256))
    return QMV_ERR_ALIGN;
  const size_t need = qmv::layout::moe_workspace(t, ffn, top_k);
  if (caller_ws ? (!ws || ws_bytes < need) : need > qmv::layout::kMoeNoAllocBytes) return QMV_ERR_WORKSPACE;

  // every output (and the workspace) must be disjoint from every input and from each other
  const size_t ta = (size_t)t;
  const size_t yb = ta * hidden * 4, idb = ta * top_k * 4, pb = ta * top_k * 8;
  const void *in_p[] = {w_gate, w_up, w_down, logits, x_bf16};
  const size_t in_b[] = {bank, bank, bank, ta * n_experts * 4, ta * hidden * 2};
  const void *out_p[] = {y, topk_ids, topk_w, pairs, ws};
  const size_t out_b[] = {yb, topk_ids ? idb : 0, topk_w ? idb : 0, pairs ? pb : 0, caller_ws ? need : 0};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlap(out_p[o], out_b[o], in_p[i], in_b[i])) return QMV_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 5; ++o2)
      if (overlap(out_p[o], out_b[o], out_p[o2], out_b[o2])) return QMV_ERR_ALIAS;
  }
  return QMV_OK;
}

int moe_launch(MoeFormat f, const void *w_gate, const void *w_up, const void *w_down, const float *logits,
               const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int t,
               int hidden, int ffn, int n_experts, int top_k, void *stream) {
  if (f == MoeFormat::kQ4K)
    return qmv::launch_q4_k_moe(w_gate, w_up, w_down, logits, x_bf16, y, topk_ids, topk_w, pairs, ws, t, hidden,
                                ffn, n_experts, top_k, stream);
  return qmv::launch_iq4_xs_moe(w_gate, w_up, w_down, logits, x_bf16, y, topk_ids, topk_w, pairs, ws, t, hidden, ffn,
                                n_experts, top_k, stream);
}

int moe_entry(MoeFormat f, const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
              const float *logits, const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w,
              int32_t *pairs, void *ws, size_t ws_bytes, int t, int hidden, int ffn, int n_experts, int top_k,
              void *stream) {
  const int rc = moe_check(f, w_gate, w_up, w_down, bank_bytes, logits, x_bf16, y, topk_ids, topk_w, pairs, ws,
                           ws_bytes, t, hidden, ffn, n_experts, top_k);
  if (rc) return rc;
  return moe_launch(f, w_gate, w_up, w_down, logits, x_bf16, y, topk_ids, topk_w, pairs, ws, t, hidden, ffn,
                    n_experts, top_k, stream);
}

}  // namespace

extern "C" {

int qmv_version(void) { return kVersion; }

const char *qmv_last_error(void) { return qmv::g_error_detail; }

const char *qmv_strerror(int code) {
  switch (code) {
    case QMV_OK: return "ok";
    case QMV_ERR_NULL: return "a required pointer is NULL";
    case QMV_ERR_SHAPE: return "shape: a dimension is not positive or not a multiple of the block size";
    case QMV_ERR_SIZE: return "size: the byte count does not match the stated shape (truncated or oversized buffer)";
    case QMV_ERR_ALIGN: return "alignment: a pointer lacks the alignment its argument requires";
    case QMV_ERR_RANGE: return "range: a count or size limit is exceeded";
    case QMV_ERR_WORKSPACE: return "workspace: NULL or smaller than the required size";
    case QMV_ERR_ALIAS: return "alias: an output overlaps an input or another output";
    case QMV_ERR_HIP: return "the HIP runtime refused the launch";
    default: return "unknown status code";
  }
}

int qmv_q8_0(const void *w, size_t w_bytes, const float *x, float *y, int m, int n, int k, void *stream) {
  if (!w || !x || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 32, 34, 4);
  if (rc) return rc;
  if (qmv::layout::q80_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 4, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_q8_0_gemv(w, x, y, m, n, k, stream);
}

int qmv_q4_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  if (qmv::layout::q4k_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_q4_k_gemv(w, x_bf16, y, m, n, k, stream);
}

int qmv_q4_k_pair(const void *w0, const void *w1, size_t w_bytes, const uint16_t *x_bf16, float *y0, float *y1, int m,
                  int n, int k, void *stream) {
  if (!w0 || !w1 || !x_bf16 || !y0 || !y1) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w0, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  rc = check_matrix(w1, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  if (n > QMV_MAX_MATRIX_ROWS / 2 || !qmv::layout::matrix_in_range(2 * n, k)) return QMV_ERR_RANGE;   // one grid of 2n rows
  if (qmv::layout::q4k_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y0, 4) || !aligned(y1, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  const float *outs[2] = {y0, y1};
  for (const float *yo : outs)
    if (overlap(yo, yb, w0, w_bytes) || overlap(yo, yb, w1, w_bytes) || overlap(yo, yb, x_bf16, xb))
      return QMV_ERR_ALIAS;
  if (overlap(y0, yb, y1, yb)) return QMV_ERR_ALIAS;
  return qmv::launch_q4_k_gemv_pair(w0, w1, x_bf16, y0, y1, m, n, k, stream);
}

int qmv_iq4_xs(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 256, 136, 8);
  if (rc) return rc;
  if (qmv::layout::iq4xs_gemv_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_iq4_xs_gemv(w, x_bf16, y, m, n, k, stream);
}

size_t qmv_q4_k_moe_workspace(int t, int hidden, int ffn, int n_experts, int top_k) {
  if (!moe_args_ok(MoeFormat::kQ4K, t, hidden, ffn, n_experts, top_k)) return 0;
  return qmv::layout::moe_workspace(t, ffn, top_k);
}

int qmv_q4_k_moe(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes, const float *logits,
                 const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws,
                 size_t ws_bytes, int t, int hidden, int ffn, int n_experts, int top_k, void *stream) {
  return moe_entry(MoeFormat::kQ4K, w_gate, w_up, w_down, bank_bytes, logits, x_bf16, y, topk_ids, topk_w, pairs, ws,
                   ws_bytes, t, hidden, ffn, n_experts, top_k, stream);
}

int qmv_q4_k_moe_noalloc(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                         const float *logits, const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w,
                         int32_t *pairs, int t, int hidden, int ffn, int n_experts, int top_k, void *stream) {
  const int rc = moe_check(MoeFormat::kQ4K, w_gate, w_up, w_down, bank_bytes, logits, x_bf16, y, topk_ids, topk_w,
                           pairs, nullptr, 0, t, hidden, ffn, n_experts, top_k, false);
  if (rc) return rc;
  return qmv::launch_q4_k_moe_noalloc(w_gate, w_up, w_down, logits, x_bf16, y, topk_ids, topk_w, pairs, t, hidden,
                                      ffn, n_experts, top_k, stream);
}

size_t qmv_q4_k_moe_prefill_workspace(int t, int hidden, int ffn, int n_experts, int top_k) {
  if (t < 1 || t > QMV_MOE_PREFILL_MAX_TOKENS || n_experts < 1 || n_experts > QMV_MOE_MAX_EXPERTS || top_k < 1 ||
      top_k > QMV_MOE_MAX_TOP_K || top_k > n_experts || hidden <= 0 || ffn <= 0 || hidden % 256 || ffn % 256 ||
      !qmv::layout::group_fits_lds(hidden, ffn))
    return 0;
  return qmv::layout::group_layout(t, hidden, ffn, n_experts, top_k).total;
}

int qmv_q4_k_moe_prefill(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                         const float *logits, const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w,
                         void *ws, size_t ws_bytes, int t, int hidden, int ffn, int n_experts, int top_k,
                         void *stream) {
  if (!w_gate || !w_up || !w_down || !logits || !x_bf16 || !y) return QMV_ERR_NULL;
  if (t < 1 || t > QMV_MOE_PREFILL_MAX_TOKENS || n_experts < 1 || n_experts > QMV_MOE_MAX_EXPERTS || top_k < 1 ||
      top_k > QMV_MOE_MAX_TOP_K || top_k > n_experts)
    return QMV_ERR_RANGE;
  if (hidden <= 0 || ffn <= 0 || hidden % 256 || ffn % 256) return QMV_ERR_SHAPE;
  if (!qmv::layout::group_fits_lds(hidden, ffn)) return QMV_ERR_RANGE;
  size_t expert_bytes = 0, bank = 0;
  if (!mul_size((size_t)ffn, (size_t)(hidden / 256) * 144, &expert_bytes) ||
      !mul_size(expert_bytes, (size_t)n_experts, &bank) || bank_bytes != bank)
    return QMV_ERR_SIZE;
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) || !aligned(x_bf16, 16) ||
      !aligned(logits, 4) || !aligned(y, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(ws, 256))
    return QMV_ERR_ALIGN;
  const size_t need = qmv::layout::group_layout(t, hidden, ffn, n_experts, top_k).total;
  if (!ws || ws_bytes < need) return QMV_ERR_WORKSPACE;
  const size_t ta = (size_t)t, yb = ta * hidden * 4, idb = ta * top_k * 4;
  const void *in_p[] = {w_gate, w_up, w_down, logits, x_bf16};
  const size_t in_b[] = {bank, bank, bank, ta * n_experts * 4, ta * hidden * 2};
  const void *out_p[] = {y, topk_ids, topk_w, ws};
  const size_t out_b[] = {yb, topk_ids ? idb : 0, topk_w ? idb : 0, need};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlap(out_p[o], out_b[o], in_p[i], in_b[i])) return QMV_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(out_p[o], out_b[o], out_p[o2], out_b[o2])) return QMV_ERR_ALIAS;
  }
  return qmv::launch_q4_k_moe_grouped(w_gate, w_up, w_down, logits, x_bf16, y, topk_ids, topk_w, ws, t, hidden, ffn,
                                      n_experts, top_k, stream);
}

size_t qmv_iq4_xs_moe_workspace(int t, int hidden, int ffn, int n_experts, int top_k) {
  if (!moe_args_ok(MoeFormat::kIQ4XS, t, hidden, ffn, n_experts, top_k)) return 0;
  return qmv::layout::moe_workspace(t, ffn, top_k);
}

int qmv_iq4_xs_moe(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes, const float *logits,
                   const uint16_t *x_bf16, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws,
                   size_t ws_bytes, int t, int hidden, int ffn, int n_experts, int top_k, void *stream) {
  return moe_entry(MoeFormat::kIQ4XS, w_gate, w_up, w_down, bank_bytes, logits, x_bf16, y, topk_ids, topk_w, pairs,
                   ws, ws_bytes, t, hidden, ffn, n_experts, top_k, stream);
}

size_t qmm_q4_k_prefill_workspace(int m, int n, int k) {
  if (m < 1 || n < 1 || k < 256 || k % 256 || !qmv::layout::prefill_in_range(m, n, k)) return 0;
  return qmv::layout::prefill_plan_bytes(qmv::layout::prefill_plan(m, n, k));
}

int qmm_q4_k_prefill(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  if (!qmv::layout::prefill_in_range(m, n, k)) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 16) || !aligned(ws, 256)) return QMV_ERR_ALIGN;
  // no overflow: m * k / 8 <= 2^32 and the tile count (so m * n / 2^14) < 2^31
  const size_t xb = (size_t)m * (size_t)k * 2, yb = (size_t)m * (size_t)n * 4;
  const size_t need = qmv::layout::prefill_plan_bytes(qmv::layout::prefill_plan(m, n, k));
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  if (need && (!ws || ws_bytes < need)) return QMV_ERR_WORKSPACE;
  if (need && (overlap(ws, need, w, w_bytes) || overlap(ws, need, x_bf16, xb) || overlap(ws, need, y, yb)))
    return QMV_ERR_ALIAS;
  return qmv::launch_q4_k_prefill(w, x_bf16, y, need ? ws : nullptr, m, n, k, stream);
}

int qmv_q5_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 256, 176, 16);
  if (rc) return rc;
  if (qmv::layout::q4k_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_q5_k_gemv(w, x_bf16, y, m, n, k, stream);
}

int qmv_dequant_q5_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 256, 176, 16);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q5_k(w, out, n, k, stream);
}

int qmv_q4_0(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  if (k <= 0 || k % 256) return QMV_ERR_SHAPE;   // the kernel steps over groups of eight blocks
  int rc = check_matrix(w, w_bytes, n, k, 32, 18, 16);
  if (rc) return rc;
  if (qmv::layout::q4k_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_q4_0_gemv(w, x_bf16, y, m, n, k, stream);
}

int qmv_dequant_q4_0_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 32, 18, 2);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q4_0(w, out, n, k, stream);
}

int qmv_q6_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y, int m, int n, int k, void *stream) {
  if (!w || !x_bf16 || !y) return QMV_ERR_NULL;
  if (m < 1 || m > QMV_MAX_ROWS) return QMV_ERR_RANGE;
  int rc = check_matrix(w, w_bytes, n, k, 256, 210, 16);
  if (rc) return rc;
  if (qmv::layout::q6k_x_lds(m, k) > qmv::layout::kLdsBudget) return QMV_ERR_RANGE;
  if (!aligned(x_bf16, 16) || !aligned(y, 4)) return QMV_ERR_ALIGN;
  const size_t xb = (size_t)m * k * 2, yb = (size_t)m * n * 4;
  if (overlap(y, yb, w, w_bytes) || overlap(y, yb, x_bf16, xb)) return QMV_ERR_ALIAS;
  return qmv::launch_q6_k_gemv(w, x_bf16, y, m, n, k, stream);
}

int qmv_dequant_q6_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 256, 210, 16);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q6_k(w, out, n, k, stream);
}

int qmv_dequant_q4_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q4_k(w, out, false, n, k, stream);
}

int qmv_dequant_q4_k_bf16(const void *w, size_t w_bytes, uint16_t *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 256, 144, 16);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 2, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q4_k(w, out, true, n, k, stream);
}

int qmv_dequant_iq4_xs_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 256, 136, 8);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_iq4_xs(w, out, n, k, stream);
}

int qmv_dequant_q8_0_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream) {
  if (!w || !out) return QMV_ERR_NULL;
  int rc = check_matrix(w, w_bytes, n, k, 32, 34, 4);
  if (rc) return rc;
  if (!aligned(out, 16)) return QMV_ERR_ALIGN;
  if (overlap(out, (size_t)n * k * 4, w, w_bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_dequant_q8_0(w, out, n, k, stream);
}

int qmv_stream_read(const void *p, size_t bytes, uint32_t *sink, int grid, int depth, int nontemporal,
                    void *stream) {
  if (!p || !sink) return QMV_ERR_NULL;
  if (bytes == 0 || bytes % 16) return QMV_ERR_SIZE;
  if (grid < 1 || grid > 65536 || (depth != 1 && depth != 2 && depth != 4 && depth != 8) ||
      (nontemporal != 0 && nontemporal != 1))
    return QMV_ERR_RANGE;
  if (!aligned(p, 16) || !aligned(sink, 4)) return QMV_ERR_ALIGN;
  if (overlap(sink, (size_t)grid * 4, p, bytes)) return QMV_ERR_ALIAS;
  return qmv::launch_stream_read(p, bytes, sink, grid, depth, nontemporal, stream);
}

}  // extern "C"
