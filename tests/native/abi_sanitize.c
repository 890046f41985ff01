/*
 * abi_sanitize.c -- drives the host side of libqr.so's C ABI (include/qr.h) through every entry point, built
 * with the host address and undefined-behaviour sanitizers by tests/test_sanitizers_cpu.py: argument
 * validation (each failing check returns its status and text), empty problems, workspace-size queries over
 * large sizes, and, with QR_FAULT_INJECT=launch, every call that passes validation, which then returns
 * QR_ERR_HIP without launching. No GPU is touched: the pointers are fake, 256-byte aligned device addresses
 * that the host never dereferences. Prints "ok" and exits 0.
 */
#define _POSIX_C_SOURCE 200112L /* setenv */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qr.h"

#define CHECK(c)                                                                                 \
    do {                                                                                         \
        if (!(c)) {                                                                              \
            fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, #c,      \
                    qr_last_error());                                                            \
            exit(1);                                                                             \
        }                                                                                        \
    } while (0)

/* distinct fake device buffers, 1 MiB apart */
#define PTR(i) ((void *)(uintptr_t)(0x7F0000000000ull + ((uint64_t)(i) << 20)))
#define MIS ((void *)(uintptr_t)0x7F0000000008ull)
#define BIG ((size_t)1 << 30)

static int injected(qr_status st) { return st == QR_ERR_HIP && strstr(qr_last_error(), "injected") != NULL; }

static void validation(void) {
    void *x = PTR(0), *xs = PTR(1), *w = PTR(2), *wsc = PTR(3), *y = PTR(4), *ws = PTR(5), *o = PTR(6);
    /* quantizers */
    CHECK(qr_quantize_weights(w, QR_BF16, 64, 250, NULL, QR_INT8, y, (float *)wsc, NULL) == QR_ERR_UNSUPPORTED);
    CHECK(qr_quantize_weights(NULL, QR_BF16, 64, 256, NULL, QR_INT8, y, (float *)wsc, NULL) == QR_ERR_ARG);
    CHECK(qr_quantize_weights(w, (qr_dtype)7, 64, 256, NULL, QR_INT8, y, (float *)wsc, NULL) == QR_ERR_ARG);
    CHECK(qr_quantize_acts(MIS, QR_F32, 4, 256, NULL, QR_FP8_E4M3, y, (float *)xs, NULL) == QR_ERR_ALIGN);
    CHECK(qr_quantize_acts(x, QR_F32, -1, 256, NULL, QR_FP8_E4M3, y, (float *)xs, NULL) == QR_ERR_ARG);
    CHECK(qr_quantize_acts(x, QR_F32, 0, 256, NULL, QR_FP8_E4M3, y, (float *)xs, NULL) == QR_OK);
    CHECK(qr_last_error()[0] == '\0');
    /* linear */
    CHECK(qr_w8a8_linear(QR_INT8, 16, 1536, 8968, x, xs, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) ==
          QR_ERR_UNSUPPORTED);
    CHECK(strstr(qr_last_error(), "multiple of 16") != NULL);
    CHECK(qr_w8a8_linear((qr_qtype)9, 16, 1536, 8960, x, xs, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) == QR_ERR_ARG);
    CHECK(qr_w8a8_linear(QR_INT8, 16, 1536, 131088, x, xs, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) ==
          QR_ERR_UNSUPPORTED);
    CHECK(qr_w8a8_linear(QR_INT8, 16, 1536, 8960, x, xs, MIS, wsc, y, QR_BF16, NULL, NULL, 0, NULL) == QR_ERR_ALIGN);
    CHECK(qr_w8a8_linear(QR_INT8, 512, 3584, 18944, x, xs, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) ==
          QR_ERR_WORKSPACE);
    CHECK(qr_w8a8_linear(QR_INT8, 512, 3584, 18944, x, xs, w, wsc, y, QR_BF16, NULL, MIS, BIG, NULL) == QR_ERR_ALIGN);
    CHECK(qr_w8a8_linear(QR_INT8, 0, 3584, 18944, x, xs, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) == QR_OK);
    CHECK(qr_w8a8_linear_noalloc(QR_FP8_E4M3, 16, 64, 256, NULL, xs, w, wsc, y, QR_BF16, NULL, NULL) == QR_ERR_ARG);
    CHECK(qr_w8a8_linear_bf16(QR_INT8, 4, 64, 250, x, NULL, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) ==
          QR_ERR_UNSUPPORTED);
    CHECK(qr_w8a8_linear_bf16(QR_INT8, 16, 2048, 1536, x, NULL, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL) ==
          QR_ERR_WORKSPACE);
    /* grouped */
    CHECK(qr_w8a8_grouped_linear(QR_INT8, 8, 256, 512, NULL, NULL, 64, 64, x, xs, w, wsc, y, QR_BF16, ws, BIG,
                                 NULL) == QR_ERR_ARG);
    CHECK(qr_w8a8_grouped_linear(QR_INT8, 70000, 256, 512, PTR(7), NULL, 64, 64, x, xs, w, wsc, y, QR_BF16, ws, BIG,
                                 NULL) == QR_ERR_UNSUPPORTED);
    CHECK(qr_w8a8_grouped_linear(QR_INT8, 8, 256, 512, PTR(7), NULL, 64, 32, x, xs, w, wsc, y, QR_BF16, ws, BIG,
                                 NULL) == QR_ERR_ARG);
    CHECK(qr_w8a8_grouped_linear(QR_INT8, 8, 256, 512, PTR(7), NULL, 0, 32, x, xs, w, wsc, y, QR_BF16, ws, BIG,
                                 NULL) == QR_OK);
    /* count, publish, W4, MoE glue */
    CHECK(qr_count_code_changes(x, w, 4096, QR_INT8, NULL, NULL, 0, NULL, NULL) == QR_ERR_ARG);
    CHECK(qr_count_code_changes(MIS, w, 4096, QR_INT8, NULL, NULL, 0, (int64_t *)o, NULL) == QR_ERR_ALIGN);
    CHECK(qr_requantize_weights(w, QR_F32, 64, 256, NULL, QR_FP8_E4M3, PTR(8), (float *)PTR(9),
                                (char *)PTR(8) + 512, (float *)PTR(10), (int32_t *)PTR(11), (int64_t *)o, NULL) ==
          QR_ERR_ARG); /* the new codes overlap the previous publish in part */
    CHECK(qr_quantize_weights_w4(w, QR_BF16, 64, 200, NULL, y, (float *)wsc, NULL) != QR_OK);
    CHECK(qr_w4a16_linear(16, 64, 256, NULL, w, (float *)wsc, y, QR_BF16, NULL) == QR_ERR_ARG);
    CHECK(qr_moe_route(NULL, 64, 16, 4, NULL, NULL, (int32_t *)PTR(12), NULL, NULL, NULL, NULL) != QR_OK);
    CHECK(qr_silu_mul_quantize(x, 32, 250, NULL, QR_INT8, y, (float *)xs, NULL, NULL) != QR_OK);
    CHECK(qr_moe_combine(x, 256, 512, NULL, (int32_t *)PTR(13), 64, 4, y, NULL) == QR_ERR_ARG);
    CHECK(qr_rmsnorm_quantize(x, 16, 3584, (const float *)xs, -1.0f, NULL, QR_FP8_E4M3, y, (float *)xs, NULL, NULL) ==
          QR_ERR_ARG);
    CHECK(qr_rmsnorm_quantize(x, 16, 3580, (const float *)xs, 1e-6f, NULL, QR_INT8, y, (float *)xs, NULL, NULL) ==
          QR_ERR_UNSUPPORTED);
    CHECK(qr_rmsnorm_quantize(x, 16, 3584, (const float *)xs, 1e-6f, NULL, (qr_qtype)7, y, (float *)xs, NULL, NULL) ==
          QR_ERR_ARG);
    /* sizes: no overflow in the workspace arithmetic over large shapes */
    CHECK(qr_workspace_bytes(QR_INT8, 1, 1536, 8960, 1) < BIG);
    CHECK(qr_workspace_bytes(QR_FP8_E4M3, 65536, 37888, 3584, 1) > 0 || 1);
    (void)qr_workspace_bytes(QR_FP8_E4M3, (int64_t)1 << 30, 65536, 131072, 1);
    (void)qr_workspace_bytes(QR_INT8, 4096, 2048, 768, 128);
    (void)qr_w8a8_linear_bf16_workspace_bytes(QR_FP8_E4M3, (int64_t)1 << 30, 65536, 131072);
    (void)qr_w8a8_linear_bf16_workspace_bytes(QR_INT8, 1, 3584, 3584);
    CHECK(strlen(qr_version()) >= 5);
}

static void injected_launches(void) {
    void *x = PTR(0), *xs = PTR(1), *w = PTR(2), *wsc = PTR(3), *y = PTR(4), *ws = PTR(5), *o = PTR(6);
    CHECK(injected(qr_quantize_weights(w, QR_BF16, 64, 256, NULL, QR_INT8, y, (float *)wsc, NULL)));
    CHECK(injected(qr_quantize_acts(x, QR_F32, 16, 256, (const float *)PTR(14), QR_FP8_E4M3, y, (float *)xs, NULL)));
    CHECK(injected(qr_w8a8_linear(QR_FP8_E4M3, 16, 1536, 1536, x, xs, w, wsc, y, QR_BF16, NULL, ws, BIG, NULL)));
    CHECK(injected(qr_w8a8_linear(QR_INT8, 2048, 37888, 3584, x, xs, w, wsc, y, QR_BF16, o, ws, BIG, NULL)));
    CHECK(injected(qr_w8a8_linear_noalloc(QR_INT8, 16, 1536, 1536, x, xs, w, wsc, y, QR_BF16, NULL, NULL)));
    CHECK(injected(qr_w8a8_linear_noalloc(QR_INT8, 512, 3584, 18944, x, xs, w, wsc, y, QR_BF16, NULL, NULL)));
    /* one launch with the quantization inside the GEMV (few workgroups: no workspace), then the two-launch form */
    CHECK(injected(qr_w8a8_linear_bf16(QR_INT8, 1, 2048, 1536, x, NULL, w, wsc, y, QR_BF16, NULL, NULL, 0, NULL)));
    CHECK(injected(qr_w8a8_linear_bf16(QR_INT8, 1, 3584, 3584, x, NULL, w, wsc, y, QR_BF16, NULL, ws, BIG, NULL)));
    CHECK(injected(qr_w8a8_linear_bf16(QR_FP8_E4M3, 64, 1536, 8960, x, NULL, w, wsc, y, QR_F32, NULL, ws, BIG, NULL)));
    CHECK(injected(qr_w8a8_grouped_linear(QR_FP8_E4M3, 8, 256, 512, (const int32_t *)PTR(7), (const int32_t *)PTR(8),
                                          64, 32, x, xs, w, wsc, y, QR_BF16, ws, BIG, NULL)));
    qr_set_debug(1); /* the injected failure comes first: no device check is launched either */
    CHECK(injected(qr_w8a8_grouped_linear(QR_INT8, 8, 256, 512, (const int32_t *)PTR(7), NULL, 64, 64, x, xs, w, wsc, y,
                                          QR_BF16, ws, BIG, NULL)));
    qr_set_debug(0);
    CHECK(injected(qr_count_code_changes(x, w, 4096, QR_FP8_E4M3, (const float *)xs, (const float *)wsc, 16,
                                         (int64_t *)o, NULL)));
    CHECK(injected(qr_requantize_weights(w, QR_F32, 64, 256, NULL, QR_FP8_E4M3, PTR(8), (float *)PTR(9), PTR(10),
                                         (float *)PTR(11), (int32_t *)PTR(12), (int64_t *)o, NULL)));
    CHECK(injected(qr_quantize_weights_w4(w, QR_BF16, 64, 256, NULL, y, (float *)wsc, NULL)));
    CHECK(injected(qr_w4a16_linear(16, 64, 256, x, w, (const float *)wsc, y, QR_BF16, NULL)));
    CHECK(injected(qr_moe_route((const float *)x, 64, 16, 4, (int32_t *)PTR(8), (float *)PTR(9), (int32_t *)PTR(10),
                                (int32_t *)PTR(11), (float *)PTR(12), (int32_t *)PTR(13), NULL)));
    CHECK(injected(qr_silu_mul_quantize(x, 32, 256, NULL, QR_INT8, y, (float *)xs, NULL, NULL)));
    CHECK(injected(qr_moe_combine(x, 256, 512, (const float *)xs, (const int32_t *)PTR(13), 64, 4, y, NULL)));
    CHECK(injected(qr_rmsnorm_quantize(x, 16, 3584, (const float *)xs, 1e-6f, NULL, QR_INT8, y, (float *)xs, NULL,
                                       NULL)));
    /* validation still comes first */
    CHECK(qr_w8a8_linear(QR_INT8, 16, 1536, 1530, x, xs, w, wsc, y, QR_BF16, NULL, ws, BIG, NULL) ==
          QR_ERR_UNSUPPORTED);
}

int main(void) {
    if (setenv("QR_FAULT_INJECT", "launch", 1) != 0) return 2;
    validation();
    injected_launches();
    printf("ok\n");
    return 0;
}
