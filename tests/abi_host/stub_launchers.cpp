// Stand-in launchers for the host-only build of the argument checks.
//
// qmv_api.cpp is linked with these instead of the HIP kernel files, and with no
// HIP runtime at all: if validation reached a HIP function the link would fail.
// Each stand-in only counts the call and records its arguments, so the driver
// can tell a call that passed every check (it reaches the launcher) from one
// that was refused (it returns a QMV_ERR_* code first).
#include <stddef.h>
#include <stdint.h>

#include "stub_launchers.h"

namespace stub {
int launches = 0;
const void *last_ws = nullptr;
int last_m = 0, last_n = 0, last_k = 0;
}  // namespace stub

namespace qmv {

static int note(int m, int n, int k, const void *ws = nullptr) {
  ++stub::launches;
  stub::last_m = m;
  stub::last_n = n;
  stub::last_k = k;
  stub::last_ws = ws;
  return 0;
}

int launch_q8_0_gemv(const void *, const float *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_q4_k_gemv(const void *, const uint16_t *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_q4_k_gemv_pair(const void *, const void *, const uint16_t *, float *, float *, int m, int n, int k, void *) {
  return note(m, n, k);
}
int launch_q5_k_gemv(const void *, const uint16_t *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_q6_k_gemv(const void *, const uint16_t *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_q4_0_gemv(const void *, const uint16_t *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_iq4_xs_gemv(const void *, const uint16_t *, float *, int m, int n, int k, void *) { return note(m, n, k); }
int launch_dequant_iq4_xs(const void *, float *, int n, int k, void *) { return note(0, n, k); }
int launch_dequant_q4_k(const void *, void *, bool, int n, int k, void *) { return note(0, n, k); }
int launch_dequant_q5_k(const void *, float *, int n, int k, void *) { return note(0, n, k); }
int launch_dequant_q6_k(const void *, float *, int n, int k, void *) { return note(0, n, k); }
int launch_dequant_q4_0(const void *, float *, int n, int k, void *) { return note(0, n, k); }
int launch_dequant_q8_0(const void *, float *, int n, int k, void *) { return note(0, n, k); }
int launch_q4_k_moe(const void *, const void *, const void *, const float *, const uint16_t *, float *, int32_t *,
                    float *, int32_t *, void *ws, int t, int hidden, int ffn, int, int, void *) {
  return note(t, hidden, ffn, ws);
}
int launch_q4_k_moe_noalloc(const void *, const void *, const void *, const float *, const uint16_t *, float *,
                            int32_t *, float *, int32_t *, int t, int hidden, int ffn, int, int, void *) {
  return note(t, hidden, ffn, nullptr);
}
int launch_q4_k_moe_grouped(const void *, const void *, const void *, const float *, const uint16_t *, float *,
                            int32_t *, float *, void *ws, int t, int hidden, int ffn, int, int, void *) {
  return note(t, hidden, ffn, ws);
}
int launch_iq4_xs_moe(const void *, const void *, const void *, const float *, const uint16_t *, float *, int32_t *,
                      float *, int32_t *, void *ws, int t, int hidden, int ffn, int, int, void *) {
  return note(t, hidden, ffn, ws);
}
int launch_q4_k_prefill(const void *, const uint16_t *, float *, void *ws, int m, int n, int k, void *) {
  return note(m, n, k, ws);
}
int launch_stream_read(const void *, size_t, uint32_t *, int grid, int depth, int nt, void *) { return note(grid, depth, nt); }

}  // namespace qmv
