// qr_abi.hip -- the extern "C" boundary of libqr.so (declared in include/qr.h).
//
// Host-side validation of every argument before anything is enqueued, dispatch to the gfx950 kernels,
// thread-local error text. No call allocates, synchronizes or keeps a pointer.
#include "qr.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "qr_internal.hpp"

namespace {

thread_local char g_err[512] = "";

qr_status fail(qr_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

qr_status ok() {
    g_err[0] = '\0';
    return QR_OK;
}

qr_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(QR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Test hook: with QR_FAULT_INJECT=launch in the environment when the library is first used, every call that
// passes validation returns QR_ERR_HIP instead of launching, as a refused launch would (no GPU is touched).
bool inject_launch() {
    static const bool on = [] {
        const char *v = getenv("QR_FAULT_INJECT");
        return v != nullptr && strcmp(v, "launch") == 0;
    }();
    return on;
}

qr_status injected(const char *what) {
    return fail(QR_ERR_HIP, "%s: launch failure injected (QR_FAULT_INJECT=launch)", what);
}

// Debug checks of device-side inputs (QR_DEBUG set, non-empty and not "0", when the library is first used, or
// qr_set_debug): they run on the call's stream and the call waits for their verdict before launching.
std::atomic<int> g_debug{-1};  // -1 until the environment is read

bool debug_on() {
    int d = g_debug.load(std::memory_order_relaxed);
    if (d < 0) {
        const char *v = getenv("QR_DEBUG");
        const int from_env = (v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0) ? 1 : 0;
        g_debug.compare_exchange_strong(d, from_env);
        d = g_debug.load(std::memory_order_relaxed);
    }
    return d > 0;
}

constexpr int64_t kMaxK = 131072;           // INT8 accumulators: k * 127^2 < 2^31
constexpr int64_t kMaxRows = 2147483647;    // grid dimension limit

qr_status check_q(qr_qtype q) {
    if (q != QR_INT8 && q != QR_FP8_E4M3) return fail(QR_ERR_ARG, "unknown qtype %d", (int)q);
    return QR_OK;
}

qr_status check_dtype(qr_dtype t, const char *name) {
    if (t != QR_F32 && t != QR_BF16) return fail(QR_ERR_ARG, "unknown %s %d", name, (int)t);
    return QR_OK;
}

qr_status check_k(int64_t k) {
    if (k <= 0) return fail(QR_ERR_ARG, "k must be positive (got %lld)", (long long)k);
    if (k % 16 != 0) return fail(QR_ERR_UNSUPPORTED, "k must be a multiple of 16 (got %lld)", (long long)k);
    if (k > kMaxK) return fail(QR_ERR_UNSUPPORTED, "k = %lld exceeds %lld", (long long)k, (long long)kMaxK);
    return QR_OK;
}

qr_status quantize_common(const void *in, qr_dtype in_type, int64_t rows, int64_t k, const float *s, qr_qtype q,
                          void *codes, float *scales, void *stream, int s_mode) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if ((st = check_dtype(in_type, "input dtype")) != QR_OK) return st;
    if (rows < 0) return fail(QR_ERR_ARG, "negative row count %lld", (long long)rows);
    if (rows > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "row count %lld too large", (long long)rows);
    if (k <= 0 || k % 16 != 0) {
        if (k <= 0) return fail(QR_ERR_ARG, "k must be positive (got %lld)", (long long)k);
        return fail(QR_ERR_UNSUPPORTED, "k must be a multiple of 16 (got %lld)", (long long)k);
    }
    if (rows == 0) return ok();
    if (in == nullptr || codes == nullptr || scales == nullptr)
        return fail(QR_ERR_ARG, "null input, code or scale pointer");
    if (!aligned(in, 16) || !aligned(codes, 16)) return fail(QR_ERR_ALIGN, "input and codes must be 16-byte aligned");
    if (!aligned(scales, 4) || (s != nullptr && !aligned(s, 4)))
        return fail(QR_ERR_ALIGN, "scale vectors must be 4-byte aligned");
    if (inject_launch()) return injected("quantize launch");
    const hipError_t e =
        qr::launch_quantize_rows(in, in_type == QR_BF16, rows, k, s, s == nullptr ? qr::kSNone : s_mode, (int)q,
                                 static_cast<uint8_t *>(codes), scales, static_cast<hipStream_t>(stream),
                                 s_mode == qr::kSMul);
    return hip_status(e, "quantize launch");
}

// validation shared by the two W8A8 linear entry points; on QR_OK, *p is the plan and *empty tells whether the
// call has nothing to do (m == 0 or n == 0)
qr_status check_linear(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes, const float *x_scales,
                       const void *w_codes, const float *w_scales, const void *y, qr_dtype y_type,
                       const void *acc_out, qr::LinearPlan *p, bool *empty) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if ((st = check_dtype(y_type, "output dtype")) != QR_OK) return st;
    if (m < 0 || n < 0) return fail(QR_ERR_ARG, "negative size m=%lld n=%lld", (long long)m, (long long)n);
    if ((st = check_k(k)) != QR_OK) return st;
    if (m > kMaxRows || n > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "m or n too large");
    *empty = m == 0 || n == 0;
    if (*empty) return ok();
    if (x_codes == nullptr || x_scales == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
        return fail(QR_ERR_ARG, "null operand pointer");
    if (!aligned(x_codes, 16) || !aligned(w_codes, 16)) return fail(QR_ERR_ALIGN, "codes must be 16-byte aligned");
    if (!aligned(x_scales, 4) || !aligned(w_scales, 4)) return fail(QR_ERR_ALIGN, "scales must be 4-byte aligned");
    if (!aligned(y, 16) || (acc_out != nullptr && !aligned(acc_out, 16)))
        return fail(QR_ERR_ALIGN, "y and acc_out must be 16-byte aligned");
    *p = qr::plan_linear((int)q, m, n, k);
    return QR_OK;
}

qr_status run_linear(const qr::LinearPlan &p, qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes,
                     const float *x_scales, const void *w_codes, const float *w_scales, void *y, qr_dtype y_type,
                     void *acc_out, void *workspace, void *stream) {
    if (qr::trace_enabled())
        fprintf(stderr, "[qr] linear q=%d m=%lld n=%lld k=%lld kind=%d mt=%d waves=%d unroll=%d tiles=%d pf=%d ksub=%d gemm=%d "
                "bm=%d splits=%d dp=%d ws=%zu bn=%d band=%lld\n",
                (int)q, (long long)m, (long long)n, (long long)k, p.kind, p.m_tiles, p.waves, p.unroll, p.tiles,
                p.prefetch ? 1 : 0, p.kind == 0 ? p.ksub : 1, p.gemm.tile, p.gemm.bm, p.kind == 0 ? p.splits : p.gemm.splits,
                p.kind == 0 ? 0 : p.gemm.dp_tiles, p.ws_bytes, p.gemm.bn,
                p.kind == 1 && p.gemm.band ? (long long)p.gemm.band_n0 : -1LL);
    if (inject_launch()) return injected("linear launch");
    const hipError_t e = qr::launch_linear(p, (int)q, m, n, k, static_cast<const uint8_t *>(x_codes), x_scales,
                                           static_cast<const uint8_t *>(w_codes), w_scales, y, y_type == QR_BF16,
                                           acc_out, workspace, static_cast<hipStream_t>(stream));
    return hip_status(e, "linear launch");
}

// Device scratch of qr_w8a8_linear_noalloc: the split-K partial sums of a linear whose K is split across
// workgroups, for callers that cannot allocate. Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` is only a host-side stand-in for the symbol: its device address on each device
// comes from hipGetSymbolAddress (taken once per device, with that device current) and only that address is
// ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[QR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// the device address of the current device's scratch (looked up on the first call on that device)
qr_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(QR_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the device scratch");
            if (ptr == nullptr) return fail(QR_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch");
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return QR_OK;
}

}  // namespace

extern "C" {

qr_status qr_quantize_weights(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s, qr_qtype q,
                              void *w_codes, float *w_scales, void *stream) {
    return quantize_common(w, w_type, n, k, s, q, w_codes, w_scales, stream, qr::kSMul);
}

qr_status qr_quantize_acts(const void *x, qr_dtype x_type, int64_t m, int64_t k, const float *s, qr_qtype q,
                           void *x_codes, float *x_scales, void *stream) {
    return quantize_common(x, x_type, m, k, s, q, x_codes, x_scales, stream, qr::kSMulRecip);
}

size_t qr_workspace_bytes(qr_qtype q, int64_t m, int64_t n, int64_t k, int64_t num_experts) {
    if ((q != QR_INT8 && q != QR_FP8_E4M3) || m <= 0 || n <= 0 || k <= 0) return 0;
    if (num_experts > 1) return qr::grouped_workspace_bytes((int)q, m, n, k, num_experts);
    return qr::plan_linear((int)q, m, n, k).ws_bytes;
}

qr_status qr_w8a8_linear(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes, const float *x_scales,
                         const void *w_codes, const float *w_scales, void *y, qr_dtype y_type, void *acc_out,
                         void *workspace, size_t workspace_bytes, void *stream) {
    qr::LinearPlan p;
    bool empty = false;
    qr_status st = check_linear(q, m, n, k, x_codes, x_scales, w_codes, w_scales, y, y_type, acc_out, &p, &empty);
    if (st != QR_OK || empty) return st;
    if (p.ws_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < p.ws_bytes)
            return fail(QR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                        workspace == nullptr ? (size_t)0 : workspace_bytes);
        if (!aligned(workspace, 256)) return fail(QR_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
    return run_linear(p, q, m, n, k, x_codes, x_scales, w_codes, w_scales, y, y_type, acc_out, workspace, stream);
}

qr_status qr_w8a8_linear_noalloc(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x_codes,
                                 const float *x_scales, const void *w_codes, const float *w_scales, void *y,
                                 qr_dtype y_type, void *acc_out, void *stream) {
    qr::LinearPlan p;
    bool empty = false;
    qr_status st = check_linear(q, m, n, k, x_codes, x_scales, w_codes, w_scales, y, y_type, acc_out, &p, &empty);
    if (st != QR_OK || empty) return st;
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        if (p.ws_bytes > (size_t)QR_NOALLOC_SCRATCH_BYTES)
            return fail(QR_ERR_UNSUPPORTED,
                        "this linear splits K over %zu bytes of partial sums, more than the %zu-byte device scratch "
                        "of qr_w8a8_linear_noalloc; call qr_w8a8_linear with a workspace",
                        p.ws_bytes, (size_t)QR_NOALLOC_SCRATCH_BYTES);
        if (inject_launch()) return injected("linear launch");
        if ((st = scratch_address(&ws)) != QR_OK) return st;
    }
    return run_linear(p, q, m, n, k, x_codes, x_scales, w_codes, w_scales, y, y_type, acc_out, ws, stream);
}

size_t qr_w8a8_linear_bf16_workspace_bytes(qr_qtype q, int64_t m, int64_t n, int64_t k) {
    if ((q != QR_INT8 && q != QR_FP8_E4M3) || m <= 0 || n <= 0 || k <= 0) return 0;
    return qr::linear_bf16_workspace_bytes(qr::plan_linear_bf16((int)q, m, n, k), (int)q, m, k);
}

qr_status qr_w8a8_linear_bf16(qr_qtype q, int64_t m, int64_t n, int64_t k, const void *x, const float *s,
                              const void *w_codes, const float *w_scales, void *y, qr_dtype y_type, void *acc_out,
                              void *workspace, size_t workspace_bytes, void *stream) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if ((st = check_dtype(y_type, "output dtype")) != QR_OK) return st;
    if (m < 0 || n < 0) return fail(QR_ERR_ARG, "negative size m=%lld n=%lld", (long long)m, (long long)n);
    if ((st = check_k(k)) != QR_OK) return st;
    if (m > kMaxRows || n > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "m or n too large");
    if (m == 0 || n == 0) return ok();
    if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
        return fail(QR_ERR_ARG, "null operand pointer");
    if (!aligned(x, 16) || !aligned(w_codes, 16)) return fail(QR_ERR_ALIGN, "x and codes must be 16-byte aligned");
    if (!aligned(w_scales, 4) || (s != nullptr && !aligned(s, 4)))
        return fail(QR_ERR_ALIGN, "scale vectors must be 4-byte aligned");
    if (!aligned(y, 16) || (acc_out != nullptr && !aligned(acc_out, 16)))
        return fail(QR_ERR_ALIGN, "y and acc_out must be 16-byte aligned");
    const qr::LinearPlan p = qr::plan_linear_bf16((int)q, m, n, k);
    const size_t need = qr::linear_bf16_workspace_bytes(p, (int)q, m, k);
    if (need > 0) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(QR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace == nullptr ? (size_t)0 : workspace_bytes);
        if (!aligned(workspace, 256)) return fail(QR_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
    if (qr::trace_enabled())
        fprintf(stderr, "[qr] linear_bf16 q=%d m=%lld n=%lld k=%lld fused=%d kind=%d mt=%d waves=%d unroll=%d tiles=%d "
                "ksub=%d ws=%zu\n",
                (int)q, (long long)m, (long long)n, (long long)k, qr::linear_bf16_fused(p, (int)q, m, k) ? 1 : 0, p.kind,
                p.m_tiles, p.waves, p.unroll, p.tiles, p.kind == 0 ? p.ksub : 1, need);
    if (inject_launch()) return injected("linear launch");
    const hipError_t e = qr::launch_linear_bf16(p, (int)q, m, n, k, static_cast<const uint16_t *>(x), s,
                                                static_cast<const uint8_t *>(w_codes), w_scales, y,
                                                y_type == QR_BF16, acc_out, workspace,
                                                static_cast<hipStream_t>(stream));
    return hip_status(e, "linear launch");
}

qr_status qr_w8a8_grouped_linear(qr_qtype q, int64_t num_experts, int64_t n, int64_t k,
                                 const int32_t *expert_offsets, const int32_t *row_ids, int64_t total_rows,
                                 int64_t x_rows, const void *x_codes, const float *x_scales, const void *w_codes,
                                 const float *w_scales, void *y, qr_dtype y_type, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    qr_status st;
    (void)workspace;
    (void)workspace_bytes;
    if ((st = check_q(q)) != QR_OK) return st;
    if ((st = check_dtype(y_type, "output dtype")) != QR_OK) return st;
    if (num_experts < 0 || n < 0 || total_rows < 0 || x_rows < 0)
        return fail(QR_ERR_ARG, "negative size");
    if ((st = check_k(k)) != QR_OK) return st;
    if (num_experts > 65535) return fail(QR_ERR_UNSUPPORTED, "at most 65535 experts");
    if (n > kMaxRows || total_rows > kMaxRows || x_rows > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "size too large");
    if (num_experts == 0 || n == 0 || total_rows == 0) return ok();
    if (expert_offsets == nullptr || x_codes == nullptr || x_scales == nullptr || w_codes == nullptr ||
        w_scales == nullptr || y == nullptr)
        return fail(QR_ERR_ARG, "null operand pointer");
    if (x_rows == 0 && row_ids != nullptr) return fail(QR_ERR_ARG, "row_ids given but x has no rows");
    if (row_ids == nullptr && x_rows < total_rows)
        return fail(QR_ERR_ARG, "identity rows need x_rows >= total_rows (%lld < %lld)", (long long)x_rows,
                    (long long)total_rows);
    if (!aligned(x_codes, 16) || !aligned(w_codes, 16)) return fail(QR_ERR_ALIGN, "codes must be 16-byte aligned");
    if (!aligned(x_scales, 4) || !aligned(w_scales, 4) || !aligned(expert_offsets, 4) ||
        (row_ids != nullptr && !aligned(row_ids, 4)))
        return fail(QR_ERR_ALIGN, "scales and index arrays must be 4-byte aligned");
    if (!aligned(y, 16)) return fail(QR_ERR_ALIGN, "y must be 16-byte aligned");
    if (inject_launch()) return injected("grouped launch");
    if (debug_on()) {
        int bits = 0;
        const hipError_t ce = qr::check_token_lists(expert_offsets, num_experts, row_ids, total_rows, x_rows, &bits,
                                                    static_cast<hipStream_t>(stream));
        if (ce != hipSuccess) return hip_status(ce, "token-list check");
        if (bits != 0)
            return fail(QR_ERR_ARG, "debug check of the token lists failed:%s%s%s%s",
                        (bits & 1) ? " expert_offsets[0] != 0;" : "",
                        (bits & 2) ? " expert_offsets[num_experts] != total_rows;" : "",
                        (bits & 4) ? " expert_offsets decreases;" : "",
                        (bits & 8) ? " a row id outside [0, x_rows);" : "");
    }
    const hipError_t e = qr::launch_grouped((int)q, num_experts, n, k, expert_offsets, row_ids, total_rows, x_rows,
                                            static_cast<const uint8_t *>(x_codes), x_scales,
                                            static_cast<const uint8_t *>(w_codes), w_scales, y, y_type == QR_BF16,
                                            static_cast<hipStream_t>(stream));
    return hip_status(e, "grouped launch");
}

qr_status qr_count_code_changes(const void *a, const void *b, int64_t count, qr_qtype q, const float *sa,
                                const float *sb, int64_t n_scales, int64_t *out3, void *stream) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if (count < 0 || n_scales < 0) return fail(QR_ERR_ARG, "negative count");
    if (out3 == nullptr) return fail(QR_ERR_ARG, "null out3");
    if (!aligned(out3, 8)) return fail(QR_ERR_ALIGN, "out3 must be 8-byte aligned");
    if (count > 0 && (a == nullptr || b == nullptr)) return fail(QR_ERR_ARG, "null code pointer");
    if (n_scales > 0 && (sa == nullptr || sb == nullptr)) return fail(QR_ERR_ARG, "null scale pointer");
    if ((a != nullptr && !aligned(a, 16)) || (b != nullptr && !aligned(b, 16)))
        return fail(QR_ERR_ALIGN, "codes must be 16-byte aligned");
    if ((sa != nullptr && !aligned(sa, 4)) || (sb != nullptr && !aligned(sb, 4)))
        return fail(QR_ERR_ALIGN, "scales must be 4-byte aligned");
    if (inject_launch()) return injected("count launch");
    const hipError_t e = qr::launch_count_changes(static_cast<const uint8_t *>(a), static_cast<const uint8_t *>(b),
                                                  count, (int)q, sa, sb, n_scales, out3,
                                                  static_cast<hipStream_t>(stream));
    return hip_status(e, "count launch");
}

qr_status qr_requantize_weights(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s, qr_qtype q,
                                const void *prev_codes, const float *prev_scales, void *w_codes, float *w_scales,
                                int32_t *row_counts, int64_t *out3, void *stream) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if ((st = check_dtype(w_type, "input dtype")) != QR_OK) return st;
    if (n < 0) return fail(QR_ERR_ARG, "negative row count %lld", (long long)n);
    if (n > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "row count %lld too large", (long long)n);
    if (k <= 0) return fail(QR_ERR_ARG, "k must be positive (got %lld)", (long long)k);
    if (k % 16 != 0) return fail(QR_ERR_UNSUPPORTED, "k must be a multiple of 16 (got %lld)", (long long)k);
    if (k > INT32_MAX) return fail(QR_ERR_UNSUPPORTED, "k %lld too large for the per-row counts", (long long)k);
    if (out3 == nullptr) return fail(QR_ERR_ARG, "null out3");
    if (!aligned(out3, 8)) return fail(QR_ERR_ALIGN, "out3 must be 8-byte aligned");
    if (n > 0 && (w == nullptr || prev_codes == nullptr || prev_scales == nullptr || w_codes == nullptr ||
                  w_scales == nullptr || row_counts == nullptr))
        return fail(QR_ERR_ARG, "null input, code, scale or count pointer");
    if (n > 0) {
        if (!aligned(w, 16) || !aligned(prev_codes, 16) || !aligned(w_codes, 16) || (s != nullptr && !aligned(s, 4)))
            return fail(QR_ERR_ALIGN, "input and codes must be 16-byte aligned, s 4-byte aligned");
        if (!aligned(prev_scales, 4) || !aligned(w_scales, 4) || !aligned(row_counts, 4))
            return fail(QR_ERR_ALIGN, "scales and row counts must be 4-byte aligned");
        // the previous publish is either the output itself (in place) or disjoint from it
        auto overlap = [](const void *a, const void *b, int64_t bytes) {
            const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
            return x != y && x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
        };
        if (overlap(prev_codes, w_codes, n * k) || overlap(prev_scales, w_scales, n * 4))
            return fail(QR_ERR_ARG, "previous and new codes (or scales) overlap without being the same buffer");
    }
    if (inject_launch()) return injected("requantize launch");
    const hipError_t e = qr::launch_requantize(w, w_type == QR_BF16, n, k, s, (int)q,
                                               static_cast<const uint8_t *>(prev_codes), prev_scales,
                                               static_cast<uint8_t *>(w_codes), w_scales, row_counts, out3,
                                               static_cast<hipStream_t>(stream));
    return hip_status(e, "requantize launch");
}

qr_status qr_quantize_weights_w4(const void *w, qr_dtype w_type, int64_t n, int64_t k, const float *s,
                                 void *w_codes, float *w_scales, void *stream) {
    qr_status st;
    if ((st = check_dtype(w_type, "input dtype")) != QR_OK) return st;
    if (n < 0) return fail(QR_ERR_ARG, "negative row count %lld", (long long)n);
    if (k <= 0) return fail(QR_ERR_ARG, "k must be positive (got %lld)", (long long)k);
    if (k % qr::kW4Group != 0)
        return fail(QR_ERR_UNSUPPORTED, "k must be a multiple of %d (got %lld)", (int)qr::kW4Group, (long long)k);
    if (n > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "row count %lld too large", (long long)n);
    if (n == 0) return ok();
    if (w == nullptr || w_codes == nullptr || w_scales == nullptr)
        return fail(QR_ERR_ARG, "null input, code or scale pointer");
    if (!aligned(w, 16) || !aligned(w_codes, 16) || (s != nullptr && !aligned(s, 16)))
        return fail(QR_ERR_ALIGN, "input, codes and s must be 16-byte aligned");
    if (!aligned(w_scales, 4)) return fail(QR_ERR_ALIGN, "scales must be 4-byte aligned");
    if (inject_launch()) return injected("w4 quantize launch");
    const hipError_t e = qr::launch_quantize_w4(w, w_type == QR_BF16, n, k, s, static_cast<uint8_t *>(w_codes),
                                                w_scales, static_cast<hipStream_t>(stream));
    return hip_status(e, "w4 quantize launch");
}

qr_status qr_w4a16_linear(int64_t m, int64_t n, int64_t k, const void *x, const void *w_codes, const float *w_scales,
                          void *y, qr_dtype y_type, void *stream) {
    qr_status st;
    if ((st = check_dtype(y_type, "output dtype")) != QR_OK) return st;
    if (m < 0 || n < 0) return fail(QR_ERR_ARG, "negative size m=%lld n=%lld", (long long)m, (long long)n);
    if (k <= 0) return fail(QR_ERR_ARG, "k must be positive (got %lld)", (long long)k);
    if (k % qr::kW4Group != 0)
        return fail(QR_ERR_UNSUPPORTED, "k must be a multiple of %d (got %lld)", (int)qr::kW4Group, (long long)k);
    if (m > 65535 * 16 || n > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "m or n too large");
    if (n * (k / 2) > (int64_t)UINT32_MAX)
        return fail(QR_ERR_UNSUPPORTED, "codes of %lld x %lld exceed 4 GiB", (long long)n, (long long)k);
    if (m == 0 || n == 0) return ok();
    if (x == nullptr || w_codes == nullptr || w_scales == nullptr || y == nullptr)
        return fail(QR_ERR_ARG, "null operand pointer");
    if (!aligned(x, 16) || !aligned(w_codes, 16)) return fail(QR_ERR_ALIGN, "x and codes must be 16-byte aligned");
    if (!aligned(w_scales, 4)) return fail(QR_ERR_ALIGN, "scales must be 4-byte aligned");
    if (!aligned(y, 16)) return fail(QR_ERR_ALIGN, "y must be 16-byte aligned");
    const qr::W4Plan p = qr::plan_w4a16(m, n, k);
    if (qr::trace_enabled())
        fprintf(stderr, "[qr] w4a16 m=%lld n=%lld k=%lld ring=%d tiles=%d waves=%d wk=%d depth=%d xlds=%d\n",
                (long long)m, (long long)n, (long long)k, p.ring ? 1 : 0, p.tiles, p.waves, p.wk, p.depth,
                p.x_lds ? 1 : 0);
    if (inject_launch()) return injected("w4a16 launch");
    const hipError_t e = qr::launch_w4a16(p, m, n, k, static_cast<const uint16_t *>(x),
                                          static_cast<const uint8_t *>(w_codes), w_scales, y, y_type == QR_BF16,
                                          static_cast<hipStream_t>(stream));
    return hip_status(e, "w4a16 launch");
}

qr_status qr_moe_route(const float *logits, int64_t num_tokens, int64_t num_experts, int64_t top_k,
                       int32_t *topk_expert, float *topk_weight, int32_t *expert_offsets, int32_t *row_ids,
                       float *row_weights, int32_t *pair_rows, void *stream) {
    if (num_tokens < 0) return fail(QR_ERR_ARG, "negative token count %lld", (long long)num_tokens);
    if (num_experts < 1) return fail(QR_ERR_ARG, "at least one expert is needed");
    if (num_experts > qr::moe_max_experts())
        return fail(QR_ERR_UNSUPPORTED, "at most %d experts (got %lld)", qr::moe_max_experts(), (long long)num_experts);
    if (top_k < 1 || top_k > num_experts || top_k > 32)
        return fail(QR_ERR_ARG, "top_k must be in [1, min(num_experts, 32)] (got %lld)", (long long)top_k);
    if (num_tokens * top_k > (int64_t)INT32_MAX)
        return fail(QR_ERR_UNSUPPORTED, "num_tokens * top_k must stay below 2^31");
    if (expert_offsets == nullptr) return fail(QR_ERR_ARG, "null expert_offsets");
    if (!aligned(expert_offsets, 4)) return fail(QR_ERR_ALIGN, "expert_offsets must be 4-byte aligned");
    if (num_tokens > 0) {
        if (logits == nullptr || topk_expert == nullptr || topk_weight == nullptr || row_ids == nullptr ||
            row_weights == nullptr || pair_rows == nullptr)
            return fail(QR_ERR_ARG, "null pointer");
        if (!aligned(logits, 4) || !aligned(topk_expert, 4) || !aligned(topk_weight, 4) || !aligned(row_ids, 4) ||
            !aligned(row_weights, 4) || !aligned(pair_rows, 4))
            return fail(QR_ERR_ALIGN, "routing arrays must be 4-byte aligned");
    }
    if (inject_launch()) return injected("route launch");
    const hipError_t e = qr::launch_moe_route(logits, num_tokens, (int)num_experts, (int)top_k, topk_expert,
                                              topk_weight, expert_offsets, row_ids, row_weights, pair_rows,
                                              static_cast<hipStream_t>(stream));
    return hip_status(e, "route launch");
}

qr_status qr_rmsnorm_quantize(const void *x, int64_t rows, int64_t k, const float *gamma, float eps, const float *s,
                              qr_qtype q, void *h_codes, float *h_scales, void *h, void *stream) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if (rows < 0) return fail(QR_ERR_ARG, "negative row count %lld", (long long)rows);
    if (rows > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "row count %lld too large", (long long)rows);
    if ((st = check_k(k)) != QR_OK) return st;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(QR_ERR_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
    if (rows == 0) return ok();
    if (x == nullptr || gamma == nullptr || h_codes == nullptr || h_scales == nullptr)
        return fail(QR_ERR_ARG, "null pointer");
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(h_codes, 16) || (h != nullptr && !aligned(h, 16)))
        return fail(QR_ERR_ALIGN, "x, gamma, h_codes and h must be 16-byte aligned");
    if (!aligned(h_scales, 4) || (s != nullptr && !aligned(s, 4)))
        return fail(QR_ERR_ALIGN, "scale vectors must be 4-byte aligned");
    if (inject_launch()) return injected("rmsnorm launch");
    const hipError_t e = qr::launch_rmsnorm_quant(static_cast<const uint16_t *>(x), rows, k, gamma, eps, s, (int)q,
                                                  static_cast<uint8_t *>(h_codes), h_scales,
                                                  static_cast<uint16_t *>(h), static_cast<hipStream_t>(stream));
    return hip_status(e, "rmsnorm launch");
}

qr_status qr_silu_mul_quantize(const void *y_gu, int64_t rows, int64_t inter, const float *s, qr_qtype q,
                               void *h_codes, float *h_scales, void *h, void *stream) {
    qr_status st;
    if ((st = check_q(q)) != QR_OK) return st;
    if (rows < 0) return fail(QR_ERR_ARG, "negative row count %lld", (long long)rows);
    if (rows > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "row count %lld too large", (long long)rows);
    if ((st = check_k(inter)) != QR_OK) return st;
    if (rows == 0) return ok();
    if (y_gu == nullptr || h_codes == nullptr || h_scales == nullptr) return fail(QR_ERR_ARG, "null pointer");
    if (!aligned(y_gu, 16) || !aligned(h_codes, 16) || (h != nullptr && !aligned(h, 16)))
        return fail(QR_ERR_ALIGN, "y_gu, h_codes and h must be 16-byte aligned");
    if (!aligned(h_scales, 4) || (s != nullptr && !aligned(s, 4)))
        return fail(QR_ERR_ALIGN, "scale vectors must be 4-byte aligned");
    if (inject_launch()) return injected("silu launch");
    const hipError_t e = qr::launch_silu_mul_quant(static_cast<const uint16_t *>(y_gu), rows, inter, s, (int)q,
                                                   static_cast<uint8_t *>(h_codes), h_scales,
                                                   static_cast<uint16_t *>(h), static_cast<hipStream_t>(stream));
    return hip_status(e, "silu launch");
}

qr_status qr_moe_combine(const void *y_down, int64_t rows, int64_t hidden, const float *topk_weight,
                         const int32_t *pair_rows, int64_t num_tokens, int64_t top_k, void *out, void *stream) {
    if (rows < 0 || num_tokens < 0) return fail(QR_ERR_ARG, "negative size");
    if (hidden <= 0) return fail(QR_ERR_ARG, "hidden must be positive (got %lld)", (long long)hidden);
    if (hidden % 8 != 0)
        return fail(QR_ERR_UNSUPPORTED, "hidden must be a multiple of 8 (got %lld)", (long long)hidden);
    if (top_k < 1 || top_k > 32) return fail(QR_ERR_ARG, "top_k must be in [1, 32] (got %lld)", (long long)top_k);
    if (num_tokens > kMaxRows || rows > kMaxRows) return fail(QR_ERR_UNSUPPORTED, "size too large");
    if (num_tokens == 0) return ok();
    if (topk_weight == nullptr || pair_rows == nullptr || out == nullptr || (rows > 0 && y_down == nullptr))
        return fail(QR_ERR_ARG, "null pointer");
    if ((y_down != nullptr && !aligned(y_down, 16)) || !aligned(out, 16))
        return fail(QR_ERR_ALIGN, "y_down and out must be 16-byte aligned");
    if (!aligned(topk_weight, 4) || !aligned(pair_rows, 4))
        return fail(QR_ERR_ALIGN, "topk_weight and pair_rows must be 4-byte aligned");
    if (inject_launch()) return injected("combine launch");
    const hipError_t e = qr::launch_moe_combine(static_cast<const uint16_t *>(y_down), rows, topk_weight, pair_rows,
                                                num_tokens, (int)top_k, hidden, static_cast<uint16_t *>(out),
                                                static_cast<hipStream_t>(stream));
    return hip_status(e, "combine launch");
}

void qr_set_debug(int on) { g_debug.store(on ? 1 : 0, std::memory_order_relaxed); }

const char *qr_last_error(void) { return g_err; }

const char *qr_version(void) { return "0.1.0"; }

}  // extern "C"
