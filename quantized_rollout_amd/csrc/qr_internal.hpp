// qr_internal.hpp -- host-side declarations shared by the translation units of libqr.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

// invariant-scale modes of the row quantizer
enum SMode { kSNone = 0, kSMul = 1, kSMulRecip = 2 };

// Row quantizer: one absmax scale per row of in[rows, k] (k % 16 == 0). streaming: non-temporal loads of the input
// and stores of the codes (weights, read and written once); activations keep their codes cached for the linear.
hipError_t launch_quantize_rows(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int s_mode,
                                int qtype, uint8_t *codes, float *scales, hipStream_t stream, bool streaming = false);
// The RMSNorm producer of a linear's quantized input: bf16 x [rows, k] (k % 16 == 0), fp32 gamma [k].
hipError_t launch_rmsnorm_quant(const uint16_t *x, int64_t rows, int64_t k, const float *gamma, float eps,
                                const float *s, int qtype, uint8_t *codes, float *scales, uint16_t *h_out,
                                hipStream_t stream);
// the weight quantizer with the changed-code triple of every row against the previous publish (which may be
// the output itself), then out3 = the triples' sums
hipError_t launch_requantize(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int qtype,
                             const uint8_t *prev_codes, const float *prev_scales, uint8_t *codes, float *scales,
                             int32_t *row_counts, int64_t *out3, hipStream_t stream);

// Plan of a W8A8 linear (which kernel, its split of K and the workspace it needs).
// Tiled MFMA GEMM for large m (qr_gemm.hip).
constexpr int kGemmRing = 0;
constexpr int kGemmWide = 4;
struct GemmPlan {
    int tile;              // kGemmRing = LDS-ring kernel, kGemmWide = wide-wave kernel (128 x 128 per wavefront);
                           // register-staged 1 = 256x128, 2 = 128x256, 3 = 128x128
    int bm;                // ring: activation rows per tile (128 or 256)
    int bn;                // ring: channels per tile (256, 128 or 64); the wide kernel: 256
    int splits;            // ring: K splits (1 = none; else partial sums in the workspace + a reduction)
    int stages_per_split;  // ring / wide: K stages per split (64 bytes each for the ring, 128 for the wide kernel)
    int dp_tiles;          // ring: > 0: the first dp_tiles tiles (whole CU rounds) run over all of K and only the
                           // remaining tiles, a band of output columns from n_lo, are split; 0: every tile alike
    int64_t n_lo;          // ring: first column of the split band (0 unless dp_tiles > 0)
    bool band;             // wide kernel over all of K: columns from band_n0 run as 256 x 160 tiles, a second launch
    int64_t band_n0;
    size_t ws_bytes;       // splits x m x (n - n_lo) x 4 when split, else 0
};
GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k);
// adds splits x [m, n - n_lo] partial sums (int32 for INT8, fp32 for FP8) in split order, then the epilogue
// into columns n_lo .. n - 1 of y [m, n]
void launch_splitk_reduce(int qtype, int64_t m, int64_t n, int splits, const void *partial, const float *xs,
                          const float *ws, void *y, bool y_bf16, void *acc_out, hipStream_t stream,
                          int64_t n_lo = 0);
hipError_t launch_gemm(const GemmPlan &g, int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *xq,
                       const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                       void *workspace, hipStream_t stream);

struct LinearPlan {
    int kind;          // 0 = small-M MFMA GEMV, 1 = LDS-tiled MFMA GEMM
    int m_tiles;       // GEMV: 16-token tiles per block
    int waves;         // GEMV: waves per block (they split K)
    int unroll;        // GEMV: 64-byte K steps per slice (1-KiB weight loads per tile per slice)
    int tiles;         // GEMV: 16-channel tiles per block
    int64_t n_tiles;   // GEMV: 16-channel tiles
    int splits;        // GEMV: K splits across blocks (> 1: partial sums in the workspace, then a reduction)
    bool prefetch;     // GEMV: two register stages (the next K slice's loads in flight during the current MFMAs)
    int ksub;          // GEMV: K parts inside each MFMA (1, 2, 4, 8): tiles of 16 / ksub channels, m <= 16 / ksub
    GemmPlan gemm;     // GEMM (kind 1)
    size_t ws_bytes;   // workspace bytes
};

// fused_quant: the plan is for the in-kernel activation quantization (qr_w8a8_linear_bf16)
LinearPlan plan_linear(int qtype, int64_t m, int64_t n, int64_t k, int max_unroll = 8, bool fused_quant = false);

hipError_t launch_linear(const LinearPlan &p, int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *xq,
                         const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                         void *workspace, hipStream_t stream);
// the linear on bfloat16 activations: the activation quantization inside the GEMV for one-token-tile plans with
// m <= QR_FUSE_MAX_M (default 1, at most 4) and, for FP8, k <= 8192; else the activation quantizer into the
// workspace, then the linear
LinearPlan plan_linear_bf16(int qtype, int64_t m, int64_t n, int64_t k);
bool linear_bf16_fused(const LinearPlan &p, int qtype, int64_t m, int64_t k);
size_t linear_bf16_workspace_bytes(const LinearPlan &p, int qtype, int64_t m, int64_t k);
hipError_t launch_linear_bf16(const LinearPlan &p, int qtype, int64_t m, int64_t n, int64_t k, const uint16_t *xb,
                              const float *s, const uint8_t *wq, const float *ws, void *y, bool y_bf16,
                              void *acc_out, void *workspace, hipStream_t stream);

size_t grouped_workspace_bytes(int qtype, int64_t total_rows, int64_t n, int64_t k, int64_t num_experts);

hipError_t launch_grouped(int qtype, int64_t num_experts, int64_t n, int64_t k, const int32_t *offsets,
                          const int32_t *row_ids, int64_t total_rows, int64_t x_rows, const uint8_t *xq,
                          const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16,
                          hipStream_t stream);

hipError_t launch_count_changes(const uint8_t *a, const uint8_t *b, int64_t count, int qtype, const float *sa,
                                const float *sb, int64_t n_scales, int64_t *out3, hipStream_t stream);

// Debug check of a grouped call's token lists (one workgroup on the stream, then a wait for its verdict):
// *bits gets 1 if offsets[0] != 0, 2 if offsets[num_experts] != total_rows, 4 if the offsets decrease
// somewhere, 8 if a row id lies outside [0, x_rows); 0 when the lists are valid.
hipError_t check_token_lists(const int32_t *offsets, int64_t num_experts, const int32_t *row_ids, int64_t total_rows,
                             int64_t x_rows, int *bits, hipStream_t stream);

// W4A16 (qr_w4.hip): group-wise INT4 weights, bfloat16 activations.
constexpr int64_t kW4Group = 128;  // input channels per INT4 scale group
struct W4Plan {
    int tiles;   // tiles of 16 output channels per wave (they share each activation operand)
    int waves;   // waves per block
    int wk;      // waves of a channel group that split K (divides waves)
    int depth;   // stages of codes and scales in flight per wave (registers: 1 or 2; LDS ring: 2, 4 or 8)
    bool x_lds;  // the token tile's activation rows staged in LDS
    bool ring;   // codes and scales streamed through a per-wave LDS ring (needs x_lds, one tile per wave)
};
constexpr size_t kW4MaxLds = 65536;       // dynamic LDS bytes per block, register-stage kernel
constexpr size_t kW4MaxRingLds = 163840;  // dynamic LDS bytes per block, LDS-ring kernel (all of a CU's LDS)
W4Plan plan_w4a16(int64_t m, int64_t n, int64_t k);
size_t w4_lds_bytes(const W4Plan &p, int64_t m, int64_t k);
hipError_t launch_w4a16(const W4Plan &p, int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                        const float *scales, void *y, bool y_bf16, hipStream_t stream);
hipError_t launch_quantize_w4(const void *in, bool bf16, int64_t rows, int64_t k, const float *s, uint8_t *codes,
                              float *scales, hipStream_t stream);

// MoE glue (qr_moe.hip): routing into CSR token lists, SiLU-gated product fused with the per-row quantization of
// the down projection's input, routing-weighted combine.
int moe_max_experts();
hipError_t launch_moe_route(const float *logits, int64_t T, int E, int k, int32_t *topk_expert, float *topk_weight,
                            int32_t *offsets, int32_t *row_ids, float *row_weights, int32_t *pair_rows,
                            hipStream_t stream);
hipError_t launch_silu_mul_quant(const uint16_t *y_gu, int64_t rows, int64_t I, const float *s, int qtype,
                                 uint8_t *codes, float *scales, uint16_t *h_out, hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t *y_down, int64_t rows, const float *topk_weight,
                              const int32_t *pair_rows, int64_t T, int k, int64_t H, uint16_t *out,
                              hipStream_t stream);

// Environment overrides used for tuning sweeps (0 / -1 = automatic): read only when QR_TUNE was set when the
// library was loaded (tune_enabled()); otherwise env_int returns dflt without reading the environment.
bool tune_enabled();
int env_int(const char *name, int dflt);
// QR_TRACE (under QR_TUNE): each call prints its plan to stderr
bool trace_enabled();

}  // namespace qr
