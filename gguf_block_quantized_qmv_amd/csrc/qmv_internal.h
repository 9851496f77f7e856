// Internal launch interface between the C-ABI layer (qmv_api.cpp, pure host
// code) and the HIP kernel files. Arguments are already validated when these
// are called; each returns QMV_OK or QMV_ERR_HIP. The sizes both sides use
// are in qmv_layout.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qmv {

void set_error_detail(const char *what, int hip_code, const char *hip_text);

int launch_q8_0_gemv(const void *w, const float *x, float *y, int m, int n, int k, void *stream);
int launch_q4_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream);
int launch_q4_k_gemv_pair(const void *w0, const void *w1, const uint16_t *x, float *y0, float *y1, int m, int n, int k,
                          void *stream);
int launch_q5_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream);
int launch_q6_k_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream);
int launch_q4_0_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream);
int launch_iq4_xs_gemv(const void *w, const uint16_t *x, float *y, int m, int n, int k, void *stream);
int launch_dequant_iq4_xs(const void *w, float *out, int n, int k, void *stream);
int launch_dequant_q4_k(const void *w, void *out, bool bf16, int n, int k, void *stream);
int launch_dequant_q5_k(const void *w, float *out, int n, int k, void *stream);
int launch_dequant_q6_k(const void *w, float *out, int n, int k, void *stream);
int launch_dequant_q4_0(const void *w, float *out, int n, int k, void *stream);
int launch_dequant_q8_0(const void *w, float *out, int n, int k, void *stream);
int launch_q4_k_moe(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                    const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs,
                    void *ws, int t, int hidden, int ffn, int n_experts, int top_k, void *stream);
int launch_q4_k_moe_noalloc(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                            const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, int t,
                            int hidden, int ffn, int n_experts, int top_k, void *stream);
int launch_q4_k_moe_grouped(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                            const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, void *ws, int t,
                            int hidden, int ffn, int n_experts, int top_k, void *stream);
int launch_iq4_xs_moe(const void *w_gate, const void *w_up, const void *w_down, const float *logits,
                      const uint16_t *x, float *y, int32_t *topk_ids, float *topk_w, int32_t *pairs, void *ws, int t,
                      int hidden, int ffn, int n_experts, int top_k, void *stream);
int launch_q4_k_prefill(const void *w, const uint16_t *x, float *y, void *ws, int m, int n, int k, void *stream);
int launch_stream_read(const void *p, size_t bytes, uint32_t *sink, int grid, int depth, int nontemporal, void *stream);

}  // namespace qmv
