/*
 * qr_oracle.h -- plain, slow CPU oracle for the quantized-actor W8A8 linear.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this library. The product (the HIP library and its Python binding) never includes, links or
 * calls it, and this file shares no header, helper or table with the product.
 *
 * Sources (the pages):
 *   [QuRL]  "QuRL: Efficient Reinforcement Learning with Quantized Rollout"
 *           - section 3, Eq. (2): the floating-point quantization format;
 *           - section 4: one-shot quantization of the old actor before every rollout;
 *           - section 4.3: invariant scaling W X = (W / s)(s X);
 *           - section 5: channel-wise weight scales, token-wise activation scales, INT8 and FP8.
 *   [QaRL]  "QaRL: Rollout-Aligned Quantization-Aware RL ..."
 *           - section 2.2: integer Quant/Dequant with clamp and round-to-nearest, and the floating-point
 *             variant with scale s = max|W| / alpha and W_q = [W / s]_FPk;
 *           - section 3.1: W8A8 rollout, low-bit tensors published to the inference engine each step.
 *
 * Conventions: W[n,k] row-major (K contiguous), X[m,k] row-major, Y[m,n] row-major; codes are one byte
 * (int8 two's complement, or the E4M3FN bit pattern); scales are fp32.
 */
#ifndef QR_ORACLE_H
#define QR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* input / output element types */
#define OR_F32  0
#define OR_BF16 1
/* code formats */
#define OR_INT8 0
#define OR_FP8  1
/* invariant-scale modes */
#define OR_S_NONE      0 /* no invariant scale                              */
#define OR_S_MUL       1 /* weights: w' = fl32(w * s[k])     (W diag(s))      */
#define OR_S_MUL_RECIP 2 /* activations: x' = fl32(x * fl32(1 / s[k]))  (X diag(1/s)) */

/* ---- codecs ---------------------------------------------------------------------------------------- */
float    or_bf16_to_f32(uint16_t b);
double   or_rne(double x);                /* nearest integer, ties to even                     */
uint8_t  or_e4m3_encode(float v);         /* |v| <= 448: nearest E4M3FN value, ties to even     */
uint8_t  or_e4m3_encode_search(float v);  /* same result, by search over the decoded code set   */
double   or_e4m3_decode(uint8_t c);       /* NaN for 0x7F / 0xFF                                */
int32_t  or_e4m3_decode_units(uint8_t c); /* value / 2^-9 as an exact integer (finite codes)    */
uint16_t or_round_to_bf16(double v);      /* one rounding, to nearest even, to bfloat16 bits    */
void     or_e4m3_encode_array(const float *v, int64_t n, uint8_t *out);
void     or_e4m3_encode_search_array(const float *v, int64_t n, uint8_t *out);
/* patterns in [lo, hi) (clamped to +-448, NaN skipped) on which the two encoders differ; the first in *first_bad */
int64_t  or_e4m3_encoders_disagree(uint32_t lo, uint32_t hi, uint32_t *first_bad);

/* ---- the four steps of the path -------------------------------------------------------------------- */
/* One absmax scale per row (a weight row = output channel, an activation row = token). */
void or_quantize_rows(const void *in, int in_type, int64_t rows, int64_t k, const float *s, int s_mode,
                      int qtype, uint8_t *codes, float *scales);

/* acc_i32: [m,n] exact integer accumulators (INT8 only, may be NULL).
 * acc_f64: [m,n] exact accumulators as doubles (both formats; exact for the sizes allowed, may be NULL).
 * y: [m,n] fp32 or bf16 bits, from the exact accumulator, computed in fp64 and rounded once. */
int or_linear(int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *x_codes, const float *x_scales,
              const uint8_t *w_codes, const float *w_scales, int y_type, void *y, int32_t *acc_i32,
              double *acc_f64);

/* abs_f64: [m,n] exact sums of |x_j w_j| over the decoded codes (the scale of the fp32 summation bound). */
int or_linear_abs_sum(int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *x_codes, const uint8_t *w_codes,
                      double *abs_f64);

/* Tolerance of an FP8 accumulator on the matrix cores (measured hardware reading; not a step of the method):
 * trunc_f64[i,c] = sum_j (|x_j w_j| mod 2^(E_j - 13)), E_j the largest exponent sum of the products in the
 * 128-aligned K block of j and its two neighbours. */
int or_fp8_mfma_truncation(int64_t m, int64_t n, int64_t k, const uint8_t *x_codes, const uint8_t *w_codes,
                           double *trunc_f64);

/* Grouped (MoE) linear over CSR token lists: for expert e and j in [off[e], off[e+1]), output row j uses
 * activation row row_ids[j] (or j when row_ids is NULL) and expert e's weights w_codes[e] / w_scales[e]. */
int or_grouped_linear(int qtype, int64_t num_experts, int64_t n, int64_t k, const int32_t *expert_offsets,
                      const int32_t *row_ids, int64_t x_rows, const uint8_t *x_codes, const float *x_scales,
                      const uint8_t *w_codes, const float *w_scales, int y_type, void *y);

/* out3[0] = bytes that differ, out3[1] = decoded values that differ, out3[2] = scales that differ
 * (bitwise; scale arrays may be NULL with n_scales = 0). */
void or_count_code_changes(const uint8_t *a, const uint8_t *b, int64_t count, int qtype, const float *sa,
                           const float *sb, int64_t n_scales, int64_t *out3);

/* next row: MoE glue. Routing (top-k by logit, ties to the lower expert; softmax weights over the k logits;
 * CSR rows by expert then token), h = bf16(silu(g) u) over gate/up rows [g | u], and the routing-weighted
 * combine out[t] = bf16(sum_j w[t][j] y_down[pair_rows[t][j]]) over the pair rows inside [0, R). */
void or_moe_route(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *topk_expert, float *topk_weight,
                  int32_t *offsets, int32_t *row_ids, float *row_weights, int32_t *pair_rows);
void or_silu_mul(const uint16_t *y_gu, int64_t R, int64_t I, uint16_t *h);
void or_moe_combine(const uint16_t *y_down, int64_t R, const float *topk_weight, const int32_t *pair_rows,
                    int64_t T, int64_t k, int64_t H, uint16_t *out);

/* next row: the producer form of the fused activation quantization. h = bf16(x q gamma) per row with
 * q = 1 / sqrt(mean(x^2) + eps) (0 for a zero radicand), in double; the codes of h are those of
 * or_quantize_rows on h. */
void or_rmsnorm(const uint16_t *x, int64_t R, int64_t K, const float *gamma, float eps, uint16_t *h);

/* next row: one publish of W + dW: the a1 quantizer, then per row the a5 triple against the previous
 * publish (row_counts [rows][3]: bytes, values, scale changed) and its sums in out3 */
void or_requantize_weights(const void *in, int in_type, int64_t rows, int64_t k, const float *s, int qtype,
                           const uint8_t *prev_codes, const float *prev_scales, uint8_t *codes, float *scales,
                           int32_t *row_counts, int64_t *out3);

/* ---- next row: W4A16 ------------------------------------------------------------------------------- */
/* Group-wise symmetric INT4 weights, q in [-7, 7], S = max|w'| / 7 per group of `group` input channels;
 * two codes per byte (even channel in the low nibble), each sign and magnitude; scales[rows, k/group]. */
void or_quantize_w4(const void *in, int in_type, int64_t rows, int64_t k, const float *s, int64_t group,
                    uint8_t *codes, float *scales);
int  or_w4_code(const uint8_t *row_codes, int64_t j);
/* y = sum_g S[n,g] * sum_{j in g} x[m,j] q[n,j] (x bfloat16), exact up to double rounding */
void or_w4a16_linear(int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                     const float *scales, int64_t group, int y_type, void *y, double *y_f64);

#ifdef __cplusplus
}
#endif
#endif
