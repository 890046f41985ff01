/*
 * qr.h -- C ABI of the MI355X (gfx950) quantized-actor W8A8 linear library, libqr.so.
 *
 * The layer that quantized rollout runs at every decode step, from the pages
 *   [QuRL] "QuRL: Efficient Reinforcement Learning with Quantized Rollout"
 *   [QaRL] "QaRL: Rollout-Aligned Quantization-Aware RL for Fast and Stable Training under Training-Inference
 *          Mismatch"
 * in four calls: weight quantization (once per RL step, [QuRL] section 4), per-token activation
 * quantization, the W8A8 linear with its dequantization epilogue, and a grouped variant for MoE experts
 * ([QuRL] section 5; [QaRL] sections 2.2 and 3.1).
 *
 * Common contract
 *  - Layouts: W[n,k], X[m,k], Y[m,n] row-major with the last index contiguous. Codes are one byte per element:
 *    INT8 two's complement, or the OCP E4M3FN bit pattern for FP8. Scales are fp32, one per row of the
 *    quantized tensor. Codes and scales are a canonical, bit-exact format ([QaRL] 3.1: the learner publishes
 *    the low-bit tensors themselves to the inference engine), so no call reorders or pre-shuffles them.
 *  - Pointers are device pointers unless stated otherwise. The caller owns every buffer; the library keeps no
 *    pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call only enqueues work on it
 *    and never synchronizes; device faults surface at the caller's next synchronization.
 *  - k must be a positive multiple of 16; code and activation pointers must be 16-byte aligned; scale
 *    pointers 4-byte aligned; y and accumulator outputs 16-byte aligned.
 *  - m == 0, n == 0 or total_rows == 0: QR_OK, nothing is launched.
 *  - Arguments are validated on the host before anything is launched; a failed check returns its status
 *    and qr_last_error() (thread-local) explains it. A failed launch returns QR_ERR_HIP with the HIP error
 *    text. Inputs must be finite (NaN/Inf give unspecified codes).
 *  - Calls on different streams must not share a workspace buffer.
 *  - Kernel choice is automatic and depends only on the arguments. Tuning overrides for kernel sweeps
 *    (environment variables QR_GEMV_*, QR_GEMM_*, QR_GROUPED_*, QR_W4_*, QR_COUNT_*, QR_FUSE_*,
 *    QR_FORCE_VARIANT, and the plan trace QR_TRACE) are read only if QR_TUNE is set (non-empty, not "0") when
 *    the library is loaded; without it no variable is consulted, so the output bits of a call cannot change
 *    with the environment.
 *  - Test and debug hooks (read when the library is first used; neither changes an output bit):
 *    QR_FAULT_INJECT=launch makes every call that passes validation return QR_ERR_HIP ("launch failure
 *    injected") instead of launching, as a refused launch would; QR_DEBUG (non-empty, not "0"), or
 *    qr_set_debug(1), adds device checks of device-side inputs that the host cannot see (the grouped linear's
 *    token lists), after which the call waits on its stream for their verdict: a debug-mode call
 *    synchronizes and must not be captured into a graph.
 */
#ifndef QR_H
#define QR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized in C and C++ alike; in C++ they are declared with int as their underlying type, so
 * that an out-of-range value a caller passes is a value the library can examine and refuse, not undefined
 * behaviour. */
#ifdef __cplusplus
#define QR_ENUM_BASE : int
#else
#define QR_ENUM_BASE
#endif

typedef enum qr_status QR_ENUM_BASE {
    QR_OK = 0,
    QR_ERR_ARG = 1,         /* null pointer, negative or inconsistent size, bad enum          */
    QR_ERR_UNSUPPORTED = 2, /* k not a multiple of 16, or a size beyond the supported range     */
    QR_ERR_ALIGN = 3,       /* pointer alignment                                                */
    QR_ERR_WORKSPACE = 4,   /* workspace missing or smaller than qr_workspace_bytes()           */
    QR_ERR_HIP = 5          /* the HIP runtime refused a launch                                 */
} qr_status;

typedef enum qr_dtype QR_ENUM_BASE { QR_F32 = 0, QR_BF16 = 1 } qr_dtype;

/* INT8: symmetric, codes in [-127, 127], scale = max|row| / 127.
 * FP8:  E4M3FN (bias 7, largest finite 448, no infinity), scale = max|row| / 448. */
typedef enum qr_qtype QR_ENUM_BASE { QR_INT8 = 0, QR_FP8_E4M3 = 1 } qr_qtype;

/*
 * Weight quantization, one scale per output channel ([QuRL] 5: channel-wise weight scales; [QaRL] 2.2: the
 * integer and floating-point Quant equations with zero point 0 and s = max|W| / alpha; [QuRL] 4.3: the
 * invariant scaling W X = (W / s)(s X), here with the per-input-channel vector folded as W diag(s)).
 *
 * For every row r of w[n,k] (fp32 or bfloat16, selected by w_type):
 *   w'_j = w[r,j] * s[j] rounded to fp32 (or w[r,j] when s == NULL)
 *   S    = max_j |w'_j| / qmax rounded to fp32, qmax = 127 or 448 (S = 1 when that rounds to 0: an all-zero
 *          row, or one whose largest magnitude is below qmax * 2^-150)
 *   code = INT8: round-half-even(clamp(w'_j / S, -127, 127)); FP8: E4M3 nearest-even of clamp(w'_j / S, +-448)
 * with IEEE fp32 division and the sign of zero kept in FP8 (a negative value that rounds to 0 gives 0x80).
 * Writes w_codes[n,k] and w_scales[n]. s: device fp32 [k] or NULL.
 */
qr_status qr_quantize_weights(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s, qr_qtype q,
                              void *w_codes, float *w_scales, void *stream);

/*
 * Per-token dynamic activation quantization ([QuRL] 5: token-wise activation scales). Identical to
 * qr_quantize_weights row by row, with x'_j = x[r,j] * (1 / s[j]) (the reciprocal rounded to fp32 first,
 * then the product rounded to fp32), the X diag(1/s) side of the invariant scaling of [QuRL] 4.3.
 * Writes x_codes[m,k] and x_scales[m].
 */
qr_status qr_quantize_acts(const void *x, qr_dtype x_type, int64_t m, int64_t k, const float *s, qr_qtype q,
                           void *x_codes, float *x_scales, void *stream);

/*
 * W8A8 linear with dequantization epilogue ([QuRL] 5 and [QaRL] 3.1: W8A8 rollout; [QaRL] 2.2 Dequant):
 *   acc[i,c] = sum_j xq[i,j] * wq[c,j]   (INT8: exact int32; FP8: fp32 accumulation of exact products)
 *   y[i,c]   = acc[i,c] * x_scales[i] * w_scales[c], stored as y_type (bfloat16 rounded to nearest even).
 * acc_out: optional [m,n] int32 (INT8) or fp32 (FP8) copy of the accumulators, or NULL.
 * workspace: device memory of at least qr_workspace_bytes(q, m, n, k, 1) bytes, 256-byte aligned, or NULL when
 * that is 0. It is nonzero only where K is split across workgroups: large batches with too few output tiles
 * to occupy the GPU, and decode batches of 33..64 tokens on few output tiles with a deep K. The workspace
 * then holds the int32 (INT8) or fp32 (FP8) partial sums, splits x m x n x 4 bytes, which a second kernel
 * adds in a fixed order. Its contents need no initialisation and are not preserved.
 * INT8 results are bitwise independent of m (row i depends only on row i of the inputs) and deterministic;
 * FP8 results are deterministic for a given (m, n, k).
 * Limits: k <= 131072 (INT8 accumulators stay below 2^31).
 */
qr_status qr_w8a8_linear(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes, const float *x_scales,
                         const void *w_codes, const float *w_scales, void *y, qr_dtype y_type, void *acc_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The W8A8 linear of qr_w8a8_linear for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and the same result bit for bit (y and
 * acc_out) as qr_w8a8_linear, with no workspace argument. Where K is split across workgroups the partial sums go
 * to a device scratch array of QR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends; a call whose plan needs more (qr_workspace_bytes(q, m, n, k, 1) > QR_NOALLOC_SCRATCH_BYTES)
 * returns QR_ERR_UNSUPPORTED before launching anything. The call allocates nothing and calls no allocating
 * routine. The scratch of the current device is used, so `stream` must belong to the current device; every
 * call on one GPU shares that scratch, so calls that overlap on one GPU (on different streams, or from
 * different threads) race on it and must be serialized by the caller. Its contents are not preserved
 * between calls and need no initialisation. Other arguments, limits and errors as for qr_w8a8_linear.
 */
#define QR_NOALLOC_SCRATCH_BYTES (64u << 20)
qr_status qr_w8a8_linear_noalloc(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes,
                                 const float *x_scales, const void *w_codes, const float *w_scales, void *y,
                                 qr_dtype y_type, void *acc_out, void *stream);

/*
 * RMSNorm fused with the per-token activation quantization of the next linear's input (next row: the activation
 * quantization fused into its producer; [QuRL] 4.3: the X side of W X = (W / s)(s X), here h diag(1/s); [QuRL] 5:
 * token-wise activation scales). The pages give no normalization; this is the RMSNorm ahead of the attention and
 * MLP blocks of the Qwen decoders they quantize, whose output is the next linear's activation X:
 *   h[r, j] = bf16(x[r, j] * q_r * gamma[j]), q_r = 1 / sqrt(sum_j x[r, j]^2 / k + eps) (q_r = 0 when the
 *             radicand is 0), evaluated in fp64 with the products taken left to right, rounded once to
 *             bfloat16 (nearest even);
 *   h_codes [rows, k], h_scales [rows]: exactly qr_quantize_acts(h, QR_BF16, rows, k, s, q, ...),
 * so the fused call gives the same bits as the normalization followed by the quantizer, in one pass over x.
 * x: device bfloat16 [rows, k]; gamma: device fp32 [k] (the norm weight; bfloat16 weights convert exactly);
 * eps: finite and >= 0; s: device fp32 [k] or NULL; h: device bfloat16 [rows, k] or NULL (the normalized
 * activation itself, when wanted). x, gamma, h_codes and h 16-byte aligned; s and h_scales 4-byte aligned.
 * k: a positive multiple of 16. rows == 0: nothing is launched. Errors: QR_ERR_ARG (negative rows, a null
 * pointer, eps negative or not finite), QR_ERR_UNSUPPORTED (k, rows), QR_ERR_ALIGN.
 */
qr_status qr_rmsnorm_quantize(const void *x, int64_t rows, int64_t k, const float *gamma, float eps, const float *s,
                              qr_qtype q, void *h_codes, float *h_scales, void *h, void *stream);

/*
 * The W8A8 linear on bfloat16 activations (next row: the activation quantization fused with the linear):
 * the same result, bit for bit, as qr_quantize_acts(x, QR_BF16, m, k, s, q, ...) followed by qr_w8a8_linear on
 * its codes and scales (including acc_out). For single-token decode (m = 1; with FP8 for k <= 8192) the
 * activation quantization runs inside the linear's kernel (each workgroup quantizes the token row into its
 * LDS), saving one launch and the codes' round trip through memory; otherwise the two steps run one after the
 * other, the activation codes in the workspace. x: device bfloat16 [m,k], 16-byte aligned; s: device fp32 [k] or NULL (X diag(1/s)).
 * workspace: at least qr_w8a8_linear_bf16_workspace_bytes(q, m, n, k) bytes, 256-byte aligned, or NULL when
 * that is 0. Other arguments and limits as for qr_w8a8_linear.
 */
qr_status qr_w8a8_linear_bf16(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x, const float *s,
                              const void *w_codes, const float *w_scales, void *y, qr_dtype y_type, void *acc_out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Device bytes of workspace qr_w8a8_linear_bf16 needs (0 when the activation quantization runs inside it). */
size_t qr_w8a8_linear_bf16_workspace_bytes(qr_qtype q, int64_t m, int64_t n, int64_t k);

/*
 * Grouped (MoE) W8A8 linear over per-expert token lists (the expert FFNs of the Qwen3-30B-A3B model in the
 * [QaRL] abstract, run in W8A8 as in [QaRL] 3.1). Output rows are grouped by expert in CSR form:
 *   for e in [0, num_experts), j in [expert_offsets[e], expert_offsets[e+1]):
 *     r = row_ids ? row_ids[j] : j;    y[j,:] = (x_codes[r,:] . w_codes[e]^T) * x_scales[r] * w_scales[e,:]
 * expert_offsets: device int32 [num_experts+1], non-decreasing, expert_offsets[0] == 0,
 *                 expert_offsets[num_experts] == total_rows (the host passes total_rows).
 * row_ids: device int32 [total_rows] with values in [0, x_rows), or NULL for the identity.
 * w_codes: [num_experts, n, k]; w_scales: [num_experts, n]; y: [total_rows, n].
 * The device trusts the token lists but never reads outside them: a row whose row_ids entry is outside
 * [0, x_rows) gets zeros, and offsets are clamped to [0, total_rows]. In debug mode (QR_DEBUG, qr_set_debug)
 * the lists are checked on the device first, and a violation returns QR_ERR_ARG, naming the failed
 * condition, before the linear is launched.
 * workspace: as for qr_w8a8_linear, qr_workspace_bytes(q, total_rows, n, k, num_experts) bytes.
 */
qr_status qr_w8a8_grouped_linear(qr_qtype q, int64_t num_experts, int64_t n, int64_t k,
                                 const int32_t *expert_offsets, const int32_t *row_ids, int64_t total_rows,
                                 int64_t x_rows, const void *x_codes, const float *x_scales, const void *w_codes,
                                 const float *w_scales, void *y, qr_dtype y_type, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Changed-code count between two published code sets of the same tensor ([QuRL] 4.3: weight updates between
 * RL steps are much smaller than the quantization error, so most codes do not change).
 *   out3[0] = #{i : a[i] != b[i]}                         (bytes)
 *   out3[1] = #{i : value(a[i]) != value(b[i])}           (FP8 +0 and -0 are one value)
 *   out3[2] = #{r : bits(sa[r]) != bits(sb[r])}           (scales; sa/sb may be NULL with n_scales == 0)
 * out3: device int64 [3], overwritten. a, b: device codes [count], 16-byte aligned.
 */
qr_status qr_count_code_changes(const void *a, const void *b, int64_t count, qr_qtype q, const float *sa,
                                const float *sb, int64_t n_scales, int64_t *out3, void *stream);

/*
 * One publish of updated weights (next row: [QaRL] 3.1 publishes the low-bit weights to the inference engine
 * after every optimizer step; [QuRL] 4.3: the update between steps is much smaller than the quantization error,
 * so few codes change). In one pass over w it does two things:
 *   - it quantizes w exactly as qr_quantize_weights does (same codes and scales, written to w_codes, w_scales);
 *   - it compares each row with the previous publish (prev_codes [n,k], prev_scales [n]):
 *       row_counts[r] = { #j: prev_codes[r,j] != w_codes[r,j],
 *                         #j: value(prev_codes[r,j]) != value(w_codes[r,j])   (FP8 +0 and -0 are one value),
 *                         bits(prev_scales[r]) != bits(w_scales[r]) }          (device int32 [n][3])
 *       out3 = the sums of row_counts over the rows (device int64 [3], overwritten), which equals
 *              qr_count_code_changes(prev_codes, w_codes, n*k, q, prev_scales, w_scales, n).
 * prev_codes may be w_codes and prev_scales may be w_scales (publish in place); otherwise they must not overlap.
 * k: a positive multiple of 16. Alignment as for qr_quantize_weights, row_counts 4-byte, out3 8-byte aligned.
 */
qr_status qr_requantize_weights(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s, qr_qtype q,
                                const void *prev_codes, const float *prev_scales, void *w_codes, float *w_scales,
                                int32_t *row_counts, int64_t *out3, void *stream);

/*
 * W4A16 weight quantization ([QaRL] 3.1: W4A16 rollouts; the integer Quant of [QaRL] 2.2 with z = 0). Group-wise
 * symmetric INT4 over groups of QR_W4_GROUP consecutive input channels of each row:
 *   w'_j = w[r,j] * s[j] rounded to fp32 (or w[r,j] when s == NULL)
 *   S    = max_{j in group} |w'_j| / 7 rounded to fp32 (S = 1 when that rounds to 0)
 *   q_j  = round-half-even(clamp(w'_j / S, -7, 7)) with IEEE fp32 division
 * Writes w_codes[n, k/2] (channel 2i in the low nibble of byte i, 2i + 1 in the high nibble; each nibble sign
 * and magnitude: bit 3 set for a negative code, bits 0-2 = |q|, zero stored as 0) and w_scales[n, k/QR_W4_GROUP]
 * (fp32). w: device [n,k] fp32 or bf16; s: device fp32 [k] or NULL.
 * k must be a positive multiple of QR_W4_GROUP; w, w_codes and s 16-byte aligned, w_scales 4-byte aligned.
 */
#define QR_W4_GROUP 128
qr_status qr_quantize_weights_w4(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s,
                                 void *w_codes, float *w_scales, void *stream);

/*
 * W4A16 linear ([QaRL] 3.1; Dequant W_hat = s * W_q of [QaRL] 2.2 per group):
 *   y[i,c] = sum_g w_scales[c,g] * sum_{j in g} x[i,j] * q[c,j]      (x bfloat16 [m,k], exact products,
 *                                                                      fp32 sums)
 * stored as y_type (bfloat16 rounded to nearest even, or fp32). x and w_codes 16-byte aligned, w_scales 4-byte
 * aligned, y 16-byte aligned; k a positive multiple of QR_W4_GROUP; m <= 1048560; the codes of one weight
 * (n k / 2 bytes) under 4 GiB, else QR_ERR_UNSUPPORTED. No workspace. Deterministic.
 */
qr_status qr_w4a16_linear(int64_t m, int64_t n, int64_t k, const void *x, const void *w_codes, const float *w_scales,
                          void *y, qr_dtype y_type, void *stream);

/*
 * MoE routing (next row: the glue around qr_w8a8_grouped_linear for the expert FFNs of the Qwen3-30B-A3B model in
 * the [QaRL] abstract; the pages give no routing rule, so the library reads it as the usual top-k softmax router):
 *   for each token t, its top_k largest logits[t, :] (fp32 [num_tokens, num_experts]); equal logits go to the
 *   lower expert index, and -0 equals +0;
 *   topk_expert[t, j] (int32 [num_tokens, top_k]): the chosen experts in ascending expert order;
 *   topk_weight[t, j] (fp32): exp(l_j - max) / sum_i exp(l_i - max) over the chosen logits, in fp64 with the sum
 *     taken in expert order, rounded once to fp32;
 *   expert_offsets (int32 [num_experts + 1]), row_ids (int32 [num_tokens * top_k]): CSR lists of the
 *     (token, expert) rows grouped by expert, tokens ascending within an expert -- the expert_offsets / row_ids
 *     arguments of qr_w8a8_grouped_linear; row_weights (fp32 [num_tokens * top_k]): each row's weight;
 *   pair_rows[t, j] (int32 [num_tokens, top_k]): the row of token t's j-th choice.
 * Deterministic. Every output is device memory, 4-byte aligned; expert_offsets is written also when
 * num_tokens == 0. Limits: 1 <= num_experts <= 512, 1 <= top_k <= min(num_experts, 32),
 * num_tokens * top_k < 2^31. Logits must be finite.
 */
qr_status qr_moe_route(const float *logits, int64_t num_tokens, int64_t num_experts, int64_t top_k,
                       int32_t *topk_expert, float *topk_weight, int32_t *expert_offsets, int32_t *row_ids,
                       float *row_weights, int32_t *pair_rows, void *stream);

/*
 * SiLU-gated product of the expert FFN fused with the per-row activation quantization of the down projection's
 * input (next row: MoE glue; per-row codes as qr_quantize_acts, the token-wise scales of [QuRL] 5):
 *   h[r, j] = bf16(silu(g) * u) with g = y_gu[r, j], u = y_gu[r, inter + j], silu(g) = g / (1 + exp(-g)),
 *             evaluated in fp64 and rounded once to bfloat16 (nearest even);
 *   h_codes [rows, inter], h_scales [rows]: exactly qr_quantize_acts(h, QR_BF16, rows, inter, s, q, ...).
 * y_gu: device bfloat16 [rows, 2 * inter] (the gate/up output, gate columns first), 16-byte aligned;
 * h: device bfloat16 [rows, inter] or NULL (the product itself, when wanted), 16-byte aligned;
 * s: device fp32 [inter] or NULL (h diag(1/s)). inter: a positive multiple of 16. rows == 0: nothing is launched.
 */
qr_status qr_silu_mul_quantize(const void *y_gu, int64_t rows, int64_t inter, const float *s, qr_qtype q,
                               void *h_codes, float *h_scales, void *h, void *stream);

/*
 * Routing-weighted combine of the expert outputs (next row: MoE glue):
 *   out[t, c] = bf16(sum_j topk_weight[t, j] * y_down[pair_rows[t, j], c]), j = 0 .. top_k-1 in order, in fp64,
 *   rounded once to bfloat16 (nearest even).
 * y_down: device bfloat16 [rows, hidden]; topk_weight: fp32 [num_tokens, top_k]; pair_rows: int32
 * [num_tokens, top_k] (as written by qr_moe_route); out: bfloat16 [num_tokens, hidden]. A pair row outside
 * [0, rows) adds nothing. hidden: a positive multiple of 8; y_down and out 16-byte aligned.
 */
qr_status qr_moe_combine(const void *y_down, int64_t rows, int64_t hidden, const float *topk_weight,
                         const int32_t *pair_rows, int64_t num_tokens, int64_t top_k, void *out, void *stream);

/* Device bytes of workspace a linear (num_experts == 1, m rows) or grouped call (m = total_rows) needs. */
size_t qr_workspace_bytes(qr_qtype q, int64_t m, int64_t n, int64_t k, int64_t num_experts);

/* Debug mode on (1) or off (0) for every later call in the process, overriding QR_DEBUG (see the common
 * contract): device checks of device-side inputs, with a wait for their verdict. Not for captured streams. */
void qr_set_debug(int on);

/* Text of the last error on the calling thread ("" when none). */
const char *qr_last_error(void);

/* Library version, "major.minor.patch". */
const char *qr_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QR_H */
