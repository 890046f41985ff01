/*
 * oracle_sanitize.c -- runs every function of the CPU oracle (oracle/qr_oracle.c) once on small inputs and
 * the edge shapes the tests use (one row, k = 16, ragged n, an empty expert, an out-of-range row id), built
 * with the host address and undefined-behaviour sanitizers by tests/test_sanitizers_cpu.py. It checks memory
 * safety and defined behaviour only: the values are pinned by the oracle tests. Prints "ok" and exits 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qr_oracle.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            exit(1);                                                      \
        }                                                                 \
    } while (0)

static uint32_t rng = 12345u;
static float frand(void) { /* xorshift32 in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return (float)((double)rng / 2147483648.0 - 1.0);
}

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void run_linear_case(int qtype, int64_t m, int64_t n, int64_t k) {
    float *x = malloc((size_t)(m * k) * 4), *w = malloc((size_t)(n * k) * 4), *s = malloc((size_t)k * 4);
    uint16_t *wb = malloc((size_t)(n * k) * 2);
    uint8_t *xc = malloc((size_t)(m * k)), *wc = malloc((size_t)(n * k));
    float *xs = malloc((size_t)m * 4), *wsc = malloc((size_t)n * 4), *yf = malloc((size_t)(m * n) * 4);
    uint16_t *yb = malloc((size_t)(m * n) * 2);
    int32_t *acc = malloc((size_t)(m * n) * 4);
    double *accd = malloc((size_t)(m * n) * 8), *abs_sum = malloc((size_t)(m * n) * 8);
    int64_t i;
    for (i = 0; i < m * k; ++i) x[i] = frand() * 3.0f;
    for (i = 0; i < n * k; ++i) {
        w[i] = frand() * 0.02f;
        wb[i] = to_bf16(w[i]);
    }
    for (i = 0; i < k; ++i) s[i] = 0.5f + 0.25f * (float)(i % 7);
    or_quantize_rows(x, OR_F32, m, k, s, OR_S_MUL_RECIP, qtype, xc, xs);
    or_quantize_rows(wb, OR_BF16, n, k, s, OR_S_MUL, qtype, wc, wsc);
    or_quantize_rows(w, OR_F32, n, k, NULL, OR_S_NONE, qtype, wc, wsc);
    CHECK(or_linear(qtype, m, n, k, xc, xs, wc, wsc, OR_F32, yf, qtype == OR_INT8 ? acc : NULL, accd) == 0);
    CHECK(or_linear(qtype, m, n, k, xc, xs, wc, wsc, OR_BF16, yb, NULL, NULL) == 0);
    CHECK(or_linear_abs_sum(qtype, m, n, k, xc, wc, abs_sum) == 0);
    if (qtype == OR_FP8) CHECK(or_fp8_mfma_truncation(m, n, k, xc, wc, abs_sum) == 0);
    free(x), free(w), free(s), free(wb), free(xc), free(wc), free(xs), free(wsc), free(yf), free(yb), free(acc);
    free(accd), free(abs_sum);
}

static void run_grouped_case(int qtype) {
    const int64_t E = 3, n = 21, k = 64, x_rows = 5, total = 6; /* the identity would need x_rows >= 6 */
    const int32_t offsets[4] = {0, 2, 2, 6}; /* expert 1 is empty */
    int32_t rows[6] = {4, 0, 1, 1, 3, 2};
    uint8_t *xc = malloc((size_t)(x_rows * k)), *wc = malloc((size_t)(E * n * k));
    float *xs = malloc((size_t)x_rows * 4), *wsc = malloc((size_t)(E * n) * 4), *y = malloc((size_t)(total * n) * 4);
    int64_t i;
    for (i = 0; i < x_rows * k; ++i) xc[i] = (uint8_t)(i * 37 + 11) & 0x77;
    for (i = 0; i < E * n * k; ++i) wc[i] = (uint8_t)(i * 53 + 5) & 0x77;
    for (i = 0; i < x_rows; ++i) xs[i] = 0.01f * (float)(i + 1);
    for (i = 0; i < E * n; ++i) wsc[i] = 0.002f * (float)(i % 5 + 1);
    CHECK(or_grouped_linear(qtype, E, n, k, offsets, rows, x_rows, xc, xs, wc, wsc, OR_F32, y) == 0);
    rows[3] = 7; /* a row id outside [0, x_rows) is refused */
    CHECK(or_grouped_linear(qtype, E, n, k, offsets, rows, x_rows, xc, xs, wc, wsc, OR_F32, y) == -1);
    CHECK(or_grouped_linear(qtype, E, n, k, offsets, NULL, x_rows, xc, xs, wc, wsc, OR_BF16, y) == -1);
    free(xc), free(wc), free(xs), free(wsc), free(y);
}

static void run_moe_case(void) {
    const int64_t T = 5, E = 6, K = 2, I = 24, H = 16, R = T * K;
    float *logits = malloc((size_t)(T * E) * 4), *tw = malloc((size_t)(T * K) * 4), *rw = malloc((size_t)R * 4);
    int32_t *te = malloc((size_t)(T * K) * 4), *off = malloc((size_t)(E + 1) * 4), *rows = malloc((size_t)R * 4);
    int32_t *pairs = malloc((size_t)(T * K) * 4);
    uint16_t *ygu = malloc((size_t)(R * 2 * I) * 2), *h = malloc((size_t)(R * I) * 2);
    uint16_t *yd = malloc((size_t)(R * H) * 2), *out = malloc((size_t)(T * H) * 2);
    int64_t i;
    for (i = 0; i < T * E; ++i) logits[i] = (float)((i * 7) % 5) - 2.0f; /* ties between experts */
    or_moe_route(logits, T, E, K, te, tw, off, rows, rw, pairs);
    CHECK(off[0] == 0 && off[E] == R);
    for (i = 0; i < R * 2 * I; ++i) ygu[i] = to_bf16(frand() * 4.0f);
    or_silu_mul(ygu, R, I, h);
    for (i = 0; i < R * H; ++i) yd[i] = to_bf16(frand());
    or_moe_combine(yd, R, tw, pairs, T, K, H, out);
    pairs[1] = (int32_t)R + 3; /* a pair row outside [0, R) adds nothing */
    or_moe_combine(yd, R, tw, pairs, T, K, H, out);
    free(logits), free(tw), free(rw), free(te), free(off), free(rows), free(pairs), free(ygu), free(h), free(yd);
    free(out);
}

static void run_publish_case(int qtype, int with_s) {
    const int64_t rows = 7, k = 80;
    float *w = malloc((size_t)(rows * k) * 4), *s = malloc((size_t)k * 4), *ps = malloc((size_t)rows * 4);
    float *sc = malloc((size_t)rows * 4);
    uint8_t *pc = malloc((size_t)(rows * k)), *c = malloc((size_t)(rows * k));
    int32_t *rc = malloc((size_t)(rows * 3) * 4);
    int64_t out3[3], i;
    for (i = 0; i < rows * k; ++i) w[i] = frand() * 0.05f;
    for (i = 0; i < k; ++i) s[i] = 1.0f + 0.125f * (float)(i % 3);
    or_quantize_rows(w, OR_F32, rows, k, with_s ? s : NULL, with_s ? OR_S_MUL : OR_S_NONE, qtype, pc, ps);
    for (i = 0; i < rows * k; i += 9) w[i] += 1e-3f;
    or_requantize_weights(w, OR_F32, rows, k, with_s ? s : NULL, qtype, pc, ps, c, sc, rc, out3);
    or_count_code_changes(pc, c, rows * k, qtype, ps, sc, rows, out3);
    or_count_code_changes(pc, c, rows * k, qtype, NULL, NULL, 0, out3);
    CHECK(out3[0] >= out3[1] && out3[2] == 0);
    free(w), free(s), free(ps), free(sc), free(pc), free(c), free(rc);
}

static void run_w4_case(void) {
    const int64_t m = 3, n = 5, k = 256, group = 128;
    float *w = malloc((size_t)(n * k) * 4), *s = malloc((size_t)k * 4), *sc = malloc((size_t)(n * k / group) * 4);
    float *yf = malloc((size_t)(m * n) * 4);
    uint8_t *codes = malloc((size_t)(n * k / 2));
    uint16_t *x = malloc((size_t)(m * k) * 2), *yb = malloc((size_t)(m * n) * 2);
    double *yd = malloc((size_t)(m * n) * 8);
    int64_t i;
    for (i = 0; i < n * k; ++i) w[i] = frand() * 0.03f;
    for (i = 0; i < k; ++i) s[i] = 0.75f + 0.5f * (float)(i % 2);
    for (i = 0; i < m * k; ++i) x[i] = to_bf16(frand());
    or_quantize_w4(w, OR_F32, n, k, s, group, codes, sc);
    or_quantize_w4(w, OR_F32, n, k, NULL, group, codes, sc);
    for (i = 0; i < k; ++i) CHECK(or_w4_code(codes, i) >= -7 && or_w4_code(codes, i) <= 7);
    or_w4a16_linear(m, n, k, x, codes, sc, group, OR_F32, yf, yd);
    or_w4a16_linear(m, n, k, x, codes, sc, group, OR_BF16, yb, NULL);
    free(w), free(s), free(sc), free(yf), free(codes), free(x), free(yb), free(yd);
}

static void run_rmsnorm_case(int qtype) {
    const int64_t R = 3, K = 40;
    uint16_t *x = malloc((size_t)(R * K) * 2), *h = malloc((size_t)(R * K) * 2);
    float *g = malloc((size_t)K * 4), *s = malloc((size_t)K * 4), *sc = malloc((size_t)R * 4);
    uint8_t *c = malloc((size_t)(R * K));
    int64_t i;
    for (i = 0; i < R * K; ++i) x[i] = i < K ? 0 : to_bf16(frand() * 3.0f); /* row 0 all zero */
    for (i = 0; i < K; ++i) g[i] = 0.5f + frand() * 0.25f, s[i] = 1.0f + 0.5f * (float)(i % 2);
    or_rmsnorm(x, R, K, g, 0.0f, h);
    for (i = 0; i < K; ++i) CHECK(h[i] == 0 || h[i] == 0x8000); /* a zero row stays zero (no 0 * inf) */
    or_rmsnorm(x, R, K, g, 1e-6f, h);
    or_quantize_rows(h, OR_BF16, R, K, s, OR_S_MUL_RECIP, qtype, c, sc);
    free(x), free(h), free(g), free(s), free(sc), free(c);
}

int main(void) {
    static const float probes[] = {0.0f, -0.0f, 1.0f, -448.0f, 448.0f, 1e-9f, 0.0009765625f, 3.14159f, -240.5f};
    uint8_t enc[9], enc2[9];
    uint32_t first = 0;
    size_t i;
    for (i = 0; i < 9; ++i) {
        const uint8_t c = or_e4m3_encode(probes[i]);
        CHECK(c == or_e4m3_encode_search(probes[i]));
        (void)or_e4m3_decode(c);
        (void)or_e4m3_decode_units(c);
        (void)or_round_to_bf16((double)probes[i]);
        (void)or_rne((double)probes[i] * 2.5);
    }
    (void)or_e4m3_decode(0x7F);
    (void)or_bf16_to_f32(0x3F80);
    or_e4m3_encode_array(probes, 9, enc);
    or_e4m3_encode_search_array(probes, 9, enc2);
    CHECK(memcmp(enc, enc2, 9) == 0);
    CHECK(or_e4m3_encoders_disagree(0x3F800000u, 0x3F800000u + 65536u, &first) == 0);
    CHECK(or_e4m3_encoders_disagree(0xBF000000u, 0xBF000000u + 4096u, &first) == 0);
    run_linear_case(OR_INT8, 3, 5, 48);
    run_linear_case(OR_FP8, 3, 5, 48);
    run_linear_case(OR_FP8, 1, 7, 272); /* K blocks of 128 and a ragged last block */
    run_linear_case(OR_INT8, 1, 1, 16);
    run_grouped_case(OR_INT8);
    run_grouped_case(OR_FP8);
    run_moe_case();
    run_publish_case(OR_INT8, 0);
    run_publish_case(OR_FP8, 1);
    run_w4_case();
    run_rmsnorm_case(OR_INT8);
    run_rmsnorm_case(OR_FP8);
    printf("ok\n");
    return 0;
}
