/*
 * qmv.h -- C ABI of the MI355X (gfx950) block-quantized matrix-vector library.
 *
 * The library computes products of GGUF block-quantized weight matrices with a
 * few activation rows: the weight stream of plain decode and of speculative
 * verify, its routed-expert MoE form, and a prefill-sized GEMM form. The memra
 * pages this follows name the workload -- GGUF Q4_K_M and Q8_0 models decoded
 * on one GPU, dense and MoE (memra README: model support table, speed table),
 * speculative decode with K=2..3 drafts that must be byte-identical to plain
 * decode (memra-bench card, "Drafts"; memra summary page, tagline), and the
 * rule that one request is never served under two numerical programs (memra
 * README, recent-fixes list) -- but print no kernel interface, so this ABI is
 * this library's own.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named w*, x*, y*, out*, logits, topk_*, pairs, ws are DEVICE
 *    pointers (HIP device memory of the current device). The caller owns every
 *    buffer; the library never allocates, frees or synchronises. Its only
 *    process state never affects a result: per kernel and device, the largest
 *    dynamic-LDS size already granted (an atomic, so the attribute is set once),
 *    per host thread the text behind qmv_last_error(), and for
 *    qmv_q4_k_moe_noalloc its fixed device array (part of the library's code
 *    object) and that array's address per device. Calls from several host
 *    threads are safe, except overlapping qmv_q4_k_moe_noalloc calls on one GPU.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued on it asynchronously; a return of QMV_OK means the work
 *    was enqueued, not that it finished.
 *  - Every argument is validated on the host before any HIP call is made; the
 *    checks, workspace sizes and launch plans depend on the arguments alone,
 *    never on a device query. Invalid arguments return a negative QMV_ERR_*
 *    code and touch no memory.
 *    A failed launch returns QMV_ERR_HIP. Faults during execution surface as
 *    HIP errors on the caller's next synchronisation.
 *  - Quantized matrices are row-major: row n (one output feature) is the
 *    contiguous run of its K/QK blocks along the input dimension K, rows follow
 *    each other with no padding. `w_bytes` must equal the exact byte size of
 *    that layout; any other value (a truncated or oversized buffer) is
 *    QMV_ERR_SIZE. n <= QMV_MAX_MATRIX_ROWS, k <= QMV_MAX_MATRIX_K and
 *    n * k <= 2^40, else QMV_ERR_RANGE.
 *  - bf16 values travel as uint16_t bit patterns. Outputs are fp32.
 *  - Outputs must not overlap any input (QMV_ERR_ALIAS).
 *  - Results are bitwise deterministic from run to run. For the GEMV entry
 *    points, row r of the output depends only on activation row r: the same
 *    row gives bit-identical results for every row count 1..4.
 *
 * Block formats (the public GGUF layouts; the pages name them, they do not print them)
 * -------------
 *  Q8_0 : 34 bytes per 32 weights: fp16 d (little-endian), then int8 q[32];
 *         w = d * q.
 *  Q4_K : 144 bytes per 256 weights: fp16 d, fp16 dmin, 12 bytes holding eight
 *         6-bit scales sc_j and eight 6-bit mins m_j of the 32-weight
 *         sub-blocks j = 0..7, then 128 bytes of 4-bit quants q (byte 32c + l
 *         holds weight 64c + l in its low nibble and 64c + 32 + l in its high
 *         nibble); w = d * sc_j * q - dmin * m_j.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define QMV_OK             0
#define QMV_ERR_NULL      -1  /* a required pointer is NULL                          */
#define QMV_ERR_SHAPE     -2  /* N, K, H or F not positive / not a block multiple    */
#define QMV_ERR_SIZE      -3  /* a byte count does not match the stated shape         */
#define QMV_ERR_ALIGN     -4  /* a pointer lacks the alignment stated for it          */
#define QMV_ERR_RANGE     -5  /* a count (M, T, E, top_k) or a size limit is exceeded */
#define QMV_ERR_WORKSPACE -6  /* workspace NULL or smaller than the required size     */
#define QMV_ERR_ALIAS     -7  /* an output overlaps an input or another output        */
#define QMV_ERR_HIP       -8  /* the HIP runtime refused a launch                     */

/* ---- limits ------------------------------------------------------------ */
#define QMV_MAX_ROWS        4      /* activation rows per GEMV call (verify: K<=3 drafts + 1) */
#define QMV_LDS_X_BYTES     163840 /* LDS budget for staged activations per workgroup (160 KiB) */
#define QMV_MOE_MAX_TOKENS  4
#define QMV_MOE_MAX_EXPERTS 256
#define QMV_MOE_MAX_TOP_K   8
#define QMV_MOE_PREFILL_MAX_TOKENS 65536 /* tokens per qmv_q4_k_moe_prefill call */
#define QMV_MAX_MATRIX_ROWS (1 << 30)      /* n of any quantized matrix (QMV_ERR_RANGE above) */
#define QMV_MAX_MATRIX_K    (1 << 24)      /* k of any quantized matrix; also n * k <= 2^40 */

/* Diagnostics. The memra README's recent-fixes list holds its engine to
 * contextual errors instead of crashes on malformed or truncated input; these
 * three calls give a caller that context. */

/* Library version as 10000*major + 100*minor + patch. */
int qmv_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *qmv_strerror(int code);

/* Detail of the last QMV_ERR_HIP returned to the calling thread: which launch
 * or attribute call failed and the HIP error code and text ("" if none yet).
 * The text is thread-local and valid until that thread's next failing call. */
const char *qmv_last_error(void);

/*
 * Q8_0 matrix times fp32 activation rows (decode / verify).
 *   w       [n rows][k/32 blocks] Q8_0, 4-byte aligned; w_bytes == n*(k/32)*34
 *   x       fp32 [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 4-byte aligned
 *   1 <= m <= QMV_MAX_ROWS, n >= 1, k >= 32 and k % 32 == 0,
 *   m*k*4 <= QMV_LDS_X_BYTES (m=4 allows k up to 10240).
 * y[r][i] = sum_k dequant(w)[i][k] * x[r][k], accumulated in fp32.
 * Workload: the Q8_0 GEMV of the memra README's support table (Q8_0 models and
 * MTP heads) and the memra-bench card's Q8_0 drafts.
 */
int qmv_q8_0(const void *w, size_t w_bytes, const float *x, float *y,
             int m, int n, int k, void *stream);

/*
 * Q4_K matrix times bf16 activation rows (decode m=1, speculative verify m=2..4).
 *   w       [n rows][k/256 blocks] Q4_K, 16-byte aligned; w_bytes == n*(k/256)*144
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 4-byte aligned
 *   1 <= m <= QMV_MAX_ROWS, n >= 1, k >= 256 and k % 256 == 0,
 *   m*((k/128)*272 + (k/32)*4) <= QMV_LDS_X_BYTES (the activations are staged
 *   with one 16-byte pad per 128 values; m=4 allows k up to 18176).
 * y[r][i] = sum_k dequant(w)[i][k] * x[r][k] with the quants and bf16 inputs
 * exact and fp32 accumulation. Row r of y is bit-identical for every m.
 * Workload: the per-token weight stream of the memra README's dense Q4_K_M
 * models (plain decode) and of the memra-bench card's K-draft verify.
 */
int qmv_q4_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
             int m, int n, int k, void *stream);

/*
 * Two Q4_K matrices of the same shape times the same bf16 activation rows, in
 * one launch: y0 = W0 x and y1 = W1 x, as two qmv_q4_k calls would give them,
 * bit for bit (every row runs the same instructions). A decode step multiplies
 * the FFN's gate and up matrices by the same activation, and one launch over
 * both rows pays the launch's fixed start and drain once.
 *   w0, w1  two [n rows][k/256 blocks] Q4_K matrices, 16-byte aligned, each of
 *           w_bytes == n*(k/256)*144 bytes
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y0, y1  fp32 [m][n] row-major each, 4-byte aligned, overlapping no input
 *           and not each other
 *   the limits of qmv_q4_k, and 2n rows within QMV_MAX_MATRIX_ROWS.
 * Workload: the gate and up products of the memra README's dense Q4_K_M models
 * at plain decode, and of the memra-bench card's K-draft verify.
 */
int qmv_q4_k_pair(const void *w0, const void *w1, size_t w_bytes, const uint16_t *x_bf16,
                  float *y0, float *y1, int m, int n, int k, void *stream);

/*
 * Q5_K matrix times bf16 activation rows (m = 1..4): the K-quant sibling that
 * Q4_K_M files mix in (memra README model support table; the memra-bench card
 * flags a Q5_K expert mix). 176-byte blocks: the Q4_K header, 32 bytes whose
 * bit 2c (2c + 1) of byte l is the fifth bit of weight 64c + l (64c + 32 + l),
 * then the Q4_K nibbles; weight = d*sc_j*q - dmin*m_j with q in [0, 31].
 *   w       [n rows][k/256 blocks] Q5_K, 16-byte aligned; w_bytes == n*(k/256)*176
 *   x_bf16, y, m, n, k and the LDS limit as for qmv_q4_k.
 * The quants enter the products as the exact bf16 values 128 + q and 128 times
 * each sub-block's activation sum is taken off in fp32, so the result carries
 * fp32 rounding only. Row r of y is bit-identical for every m.
 */
int qmv_q5_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
             int m, int n, int k, void *stream);

/*
 * Q4_0 matrix times bf16 activation rows (m = 1..4): the format of the Gemma-4
 * QAT models on the memra README model support table. 18-byte blocks of 32
 * weights: fp16 d, then 16 bytes whose byte i holds weight i in its low nibble
 * and weight 16 + i in its high nibble; w = d * (q - 8).
 *   w       [n rows][k/32 blocks] Q4_0, 16-byte aligned (blocks themselves are
 *           only 2-byte aligned); w_bytes == n*(k/32)*18
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 4-byte aligned
 *   1 <= m <= QMV_MAX_ROWS, n >= 1, k >= 256 and k % 256 == 0 (the kernel steps
 *   over groups of eight blocks, 144 bytes, as over a Q4_K super-block; other k
 *   give QMV_ERR_SHAPE), and the LDS limit of qmv_q4_k.
 * y[r][i] = sum_k w[i][k] * x[r][k] with the quants and bf16 inputs exact and
 * fp32 accumulation (per block d * sum(q x) - 8 d * sum(x)). Row r of y is
 * bit-identical for every m.
 * Returns QMV_ERR_NULL, _SHAPE, _SIZE, _ALIGN, _RANGE, _ALIAS before any HIP
 * call, or QMV_ERR_HIP on a launch failure.
 */
int qmv_q4_0(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
             int m, int n, int k, void *stream);

/*
 * Q6_K matrix times bf16 activation rows (m = 1..4): the other K-quant that
 * Q4_K_M files mix in (memra README model support table, Q4_K_M files).
 * 210-byte blocks of 256 weights: 128 bytes of low quant nibbles, 64 bytes of
 * top quant bit pairs, 16 int8 scales (one per 16 weights), fp16 d. Weight
 * 128h + 32c + l takes its low bits from byte 64h + 32(c & 1) + l (low nibble
 * for c < 2, high for c >= 2), its top bits from bits 2c, 2c + 1 of byte
 * 128 + 32h + l, its scale from byte 192 + 8h + 2c + l/16;
 * w = d * sc * (low + 16 top - 32).
 *   w       [n rows][k/256 blocks] Q6_K, 16-byte aligned (blocks themselves are
 *           only 2-byte aligned); w_bytes == n*(k/256)*210
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 4-byte aligned
 *   1 <= m <= QMV_MAX_ROWS, n >= 1, k >= 256 and k % 256 == 0,
 *   m*(k*2 + (k/16)*4) <= QMV_LDS_X_BYTES (m = 4 allows k up to 18176).
 * The quants enter the products as the exact bf16 values 160 + q and 160 times
 * each 16-weight group's activation sum is taken off in fp32, so the result
 * carries fp32 rounding only. Row r of y is bit-identical for every m.
 * Returns QMV_ERR_NULL, _SHAPE, _SIZE, _ALIGN, _RANGE, _ALIAS before any HIP
 * call, or QMV_ERR_HIP on a launch failure.
 */
int qmv_q6_k(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
             int m, int n, int k, void *stream);

/*
 * IQ4_XS matrix times bf16 activation rows (decode m=1, verify m=2..4).
 *   w       [n rows][k/256 blocks] IQ4_XS (136-byte super-blocks of 256 weights:
 *           fp16 d, 16 bits holding the top two bits of eight 6-bit sub-block
 *           scales, 4 bytes holding their low four bits, 128 bytes of 4-bit
 *           indices into the format's 16-value grid), 8-byte aligned;
 *           w_bytes == n*(k/256)*136
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 4-byte aligned
 *   1 <= m <= QMV_MAX_ROWS, n >= 1, k >= 256 and k % 256 == 0,
 *   1024 + m*((k/32)*64 + (k/128)*16) <= QMV_LDS_X_BYTES (m=4 allows k up to 18944).
 * y[r][i] = sum_k w[i][k] * x[r][k], w = d * (ls_j - 32) * grid[index], with
 * the weights and bf16 inputs exact and fp32 accumulation. Row r of y is
 * bit-identical for every m.
 * Workload: the memra README model support table's 35B-A3B MoE in IQ4_XS and
 * the memra-bench card's UD-IQ4_XS draft of it (the expert and attention
 * matrices of that model).
 */
int qmv_iq4_xs(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
               int m, int n, int k, void *stream);

/*
 * Workspace bytes qmv_q4_k_moe needs for t tokens (0 if an argument is out of
 * range): 4 KiB of routing tables, then h as fp32 [t * top_k][ffn]. The caller
 * allocates it in device memory, 256-byte aligned. (The pages describe no
 * kernel interface; a caller-owned workspace is this library's own convention,
 * so that the library never allocates.)
 */
size_t qmv_q4_k_moe_workspace(int t, int hidden, int ffn, int n_experts, int top_k);

/*
 * Routed-expert MoE feed-forward on Q4_K experts, for t tokens at once.
 *   w_gate, w_up  n_experts matrices of [ffn rows][hidden/256 blocks], expert-major
 *   w_down        n_experts matrices of [hidden rows][ffn/256 blocks], expert-major
 *   bank_bytes    byte size of EACH of the three arrays; must equal
 *                 n_experts*ffn*(hidden/256)*144 (== n_experts*hidden*(ffn/256)*144)
 *   logits        fp32 [t][n_experts] router logits (finite values)
 *   x_bf16        bf16 bits [t][hidden], 16-byte aligned
 *   y             fp32 [t][hidden]
 *   topk_ids      int32 [t][top_k] out, may be NULL: selected experts, rank order
 *   topk_w        fp32  [t][top_k] out, may be NULL: their renormalised weights
 *   pairs         int32 [t*top_k][2] out, may be NULL: every (expert, token) pair,
 *                 sorted by expert then token (the gather list)
 *   ws, ws_bytes  workspace of at least qmv_q4_k_moe_workspace(...) bytes, 256-B aligned
 *   1 <= t <= QMV_MOE_MAX_TOKENS, 1 <= top_k <= min(QMV_MOE_MAX_TOP_K, n_experts),
 *   1 <= n_experts <= QMV_MOE_MAX_EXPERTS, hidden and ffn multiples of 256.
 *   The staged activations (with the routing rows) and h must fit in LDS next
 *   to 4 KiB of tables: t*((hidden/128)*272 + (hidden/32)*4 + 2048) and
 *   t*top_k*((ffn/64)*272 + (ffn/32)*4) bytes each <= QMV_LDS_X_BYTES - 4096,
 *   else QMV_ERR_RANGE.
 * Per token: the top_k largest logits (ties -> lower expert id) select experts
 * e_j; r_j = softmax over the selected logits; h = silu(W_gate x) * (W_up x) in
 * fp32; y = sum_j r_j * W_down[e_j] h, summed in rank order j. Each selected
 * expert's weights are read once per call however many tokens chose it, and a
 * token's result does not depend on the other tokens in the call.
 * Workload: the memra README speed table's 35B-A3B MoE decode (128 experts,
 * top-8) and the memra-bench card's K=2 drafts on it.
 */
int qmv_q4_k_moe(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                 const float *logits, const uint16_t *x_bf16, float *y,
                 int32_t *topk_ids, float *topk_w, int32_t *pairs,
                 void *ws, size_t ws_bytes,
                 int t, int hidden, int ffn, int n_experts, int top_k, void *stream);

/*
 * qmv_q4_k_moe without a workspace argument, for callers that cannot allocate
 * device memory: code recorded into a HIP graph, tight serving loops, and
 * harnesses that forbid allocation. The routing tables and h live in one
 * fixed 160 KiB device array per GPU (QMV_MOE_NOALLOC_BYTES), which the
 * library holds until the process ends; the call allocates and frees nothing.
 * Every call that passes qmv_q4_k_moe's limits fits in it (the LDS limit on h
 * bounds the workspace to under 150 KiB); a call whose workspace would exceed
 * it returns QMV_ERR_WORKSPACE. Arguments, results (bit for bit), routing
 * outputs and the other error codes are those of qmv_q4_k_moe. All calls on
 * one GPU share the array, which keeps the last call's contents (each call
 * writes every value it reads, so nothing needs clearing): calls that overlap
 * in time on one GPU -- on different streams, or from different host threads
 * without ordering -- race and give undefined results.
 */
#define QMV_MOE_NOALLOC_BYTES 163840
int qmv_q4_k_moe_noalloc(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                         const float *logits, const uint16_t *x_bf16, float *y,
                         int32_t *topk_ids, float *topk_w, int32_t *pairs,
                         int t, int hidden, int ffn, int n_experts, int top_k, void *stream);

/*
 * Routed-expert MoE feed-forward for a prompt's tokens (prefill), Q4_K experts.
 * Arguments, routing, outputs and error codes as qmv_q4_k_moe, except:
 *   1 <= t <= QMV_MOE_PREFILL_MAX_TOKENS; logits, x_bf16, y, topk_ids and
 *   topk_w hold all t tokens; there is no gather-list output;
 *   16 rows of x (bf16) and of h (three bf16 parts) must fit in
 *   QMV_LDS_X_BYTES with their per-32 sums (QMV_ERR_RANGE otherwise): hidden
 *   up to 4608 and ffn up to 1536;
 *   ws, ws_bytes  at least qmv_q4_k_moe_prefill_workspace(...) bytes: the
 *                 routing, the per-expert pair lists, h (t top_k ffn fp32)
 *                 and the per-pair down products (t top_k hidden fp32),
 *                 each 256-byte aligned; it grows linearly with t.
 * The (token, expert) pairs are grouped by expert into chunks of 16, and each
 * chunk's gate/up and down products run on the matrix cores (bf16 MFMA, exact
 * quants; h enters the down product as three bf16 parts that keep about 24
 * bits of it), so each expert's weights are read once per 16 of its tokens.
 * Results are within the same 2e-3 floored relative bound of the exact layer
 * as qmv_q4_k_moe, but not bit-identical to it: the products are summed in
 * another order. A token's result does not depend on the other tokens in the
 * call, and repeated calls are bitwise identical.
 * Workload: the prompt phase of the memra README's 35B-A3B MoE (its summary
 * page's time-to-first-token figures).
 */
size_t qmv_q4_k_moe_prefill_workspace(int t, int hidden, int ffn, int n_experts, int top_k);
int qmv_q4_k_moe_prefill(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                         const float *logits, const uint16_t *x_bf16, float *y,
                         int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                         int t, int hidden, int ffn, int n_experts, int top_k, void *stream);

/*
 * Workspace bytes qmv_iq4_xs_moe needs for t tokens (0 if an argument is out of
 * range); the same layout and size as qmv_q4_k_moe's.
 */
size_t qmv_iq4_xs_moe_workspace(int t, int hidden, int ffn, int n_experts, int top_k);

/*
 * Routed-expert MoE feed-forward on IQ4_XS experts (the memra README's model
 * support table lists its 35B-A3B MoE in IQ4_XS). Arguments, routing, outputs
 * and error codes as qmv_q4_k_moe, except:
 *   w_gate, w_up, w_down  8-byte aligned banks of 136-byte IQ4_XS blocks;
 *                 bank_bytes must equal n_experts*ffn*(hidden/256)*136
 *   LDS limits    t*((hidden/32)*68 + 2048) and t*top_k*(ffn/32)*144 bytes
 *                 each <= QMV_LDS_X_BYTES - 8192, else QMV_ERR_RANGE.
 * h = silu(W_gate x) * (W_up x) is formed in fp32 from bf16 weight pairs and
 * bf16 activations (dot2, fp32 accumulation) and W_down h in fp32 (fma). The
 * selection, its tie rule, the weights and the rank-order combine are those
 * of qmv_q4_k_moe.
 */
int qmv_iq4_xs_moe(const void *w_gate, const void *w_up, const void *w_down, size_t bank_bytes,
                   const float *logits, const uint16_t *x_bf16, float *y,
                   int32_t *topk_ids, float *topk_w, int32_t *pairs,
                   void *ws, size_t ws_bytes,
                   int t, int hidden, int ffn, int n_experts, int top_k, void *stream);

/*
 * Workspace bytes qmm_q4_k_prefill needs for an m x n x k product (0 if none,
 * or if an argument is out of range). It depends on the shape alone. The
 * 256 x 128 output tiles (rows of X x rows of W) run on 256 workgroup slots
 * (a 256-CU MI355X at one workgroup per CU); when the tile count is not a
 * multiple of 256, the tiles past the last multiple run as parts of whole
 * 256-value K blocks so that the last round fills the slots, and this many
 * bytes hold the parts' fp32 sums.
 * (A caller-owned workspace is this library's own convention: the pages
 * describe no kernel interface.)
 */
size_t qmm_q4_k_prefill_workspace(int m, int n, int k);

/*
 * Prefill-sized product Y = X W^T on bf16 matrix cores.
 *   w       [n rows][k/256 blocks] Q4_K, 16-byte aligned; w_bytes == n*(k/256)*144
 *   x_bf16  bf16 bits [m][k] row-major, 16-byte aligned
 *   y       fp32 [m][n] row-major, 16-byte aligned
 *   ws      device memory of ws_bytes >= qmm_q4_k_prefill_workspace(m, n, k),
 *           256-byte aligned (its contents on entry do not matter); may be
 *           NULL only when that size is 0, else QMV_ERR_WORKSPACE
 *   m >= 1, n >= 1, k % 256 == 0; m * k / 8 <= 2^32 (activation granules are
 *   indexed in 32 bits) and at most 2^31 - 1 output tiles, else QMV_ERR_RANGE.
 * Weights are dequantized to fp32, rounded once to bf16 (round to nearest
 * even) and multiplied with the bf16 activations, accumulating in fp32.
 * Each output tile is one workgroup's sequential fp32 sum over K, except the
 * split tiles: there each part sums a run of whole K blocks and a second
 * launch adds the parts in K order. The summation order -- and so every bit
 * of the result -- depends only on (m, n, k) and the inputs, on any device.
 * Workload: prompt processing ahead of decode (the time-to-first-token figures
 * of the memra summary page's performance table).
 */
int qmm_q4_k_prefill(const void *w, size_t w_bytes, const uint16_t *x_bf16, float *y,
                     int m, int n, int k, void *ws, size_t ws_bytes, void *stream);

/*
 * Dequantization to dense matrices, of the GGUF formats the memra README's
 * model support table names. They expose the weights exactly as the products
 * above decode them, so that decoding can be checked bit for bit against an
 * independent decoder.
 *   out  fp32 [n][k] or bf16 bits [n][k], 16-byte aligned
 * fp32: each weight is the exact block value rounded once to fp32 (nearest
 * even; Q8_0 and IQ4_XS weights are exact in fp32). bf16: that fp32 value
 * rounded to bf16 (nearest even). IQ4_XS: w is 8-byte aligned, 136-byte blocks.
 * Q5_K: 16-byte aligned, 176-byte blocks. Q6_K: 16-byte aligned, 210-byte blocks.
 * Q4_0: 2-byte aligned, 18-byte blocks, any k % 32 == 0 (weights exact in fp32).
 */
int qmv_dequant_q4_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);
int qmv_dequant_q4_k_bf16(const void *w, size_t w_bytes, uint16_t *out, int n, int k, void *stream);
int qmv_dequant_q8_0_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);
int qmv_dequant_iq4_xs_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);
int qmv_dequant_q5_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);
int qmv_dequant_q6_k_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);
int qmv_dequant_q4_0_f32(const void *w, size_t w_bytes, float *out, int n, int k, void *stream);

/*
 * Measurement aid, outside the product path: reads `bytes` of device memory
 * with plain coalesced 16-byte loads (a grid-strided walk over `grid`
 * workgroups of 256 threads, `depth` loads in flight per thread; non-temporal
 * loads if `nontemporal` is 1) and writes the XOR of each workgroup's 32-bit
 * words to sink[0 .. grid). The rate
 * it reaches over the GEMVs' own weight pool is the achievable HBM read ceiling
 * their rates are read against (the roofline stays the 8 TB/s peak).
 *   p     16-byte aligned, bytes > 0 and a multiple of 16
 *   sink  uint32 [grid], 4-byte aligned, not overlapping p
 *   1 <= grid <= 65536, depth in {1, 2, 4, 8}, nontemporal in {0, 1}, else QMV_ERR_RANGE.
 * (This library's own: the pages measure no kernel.)
 */
int qmv_stream_read(const void *p, size_t bytes, uint32_t *sink, int grid, int depth, int nontemporal,
                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
