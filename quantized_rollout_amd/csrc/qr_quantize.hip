// qr_quantize.hip -- per-row absmax quantization to INT8 / FP8 E4M3 (weights and activations).
//
// One row per wavefront team: rows of up to 512 16-byte chunks (bf16 k <= 4096, fp32 k <= 2048) take one
// wavefront each, four rows per workgroup; longer rows take a workgroup of 2..16 wavefronts. The row is
// streamed from HBM once in coalesced 16-byte chunks and kept in VGPRs (up to 8 chunks per lane); the absmax
// is reduced across the wavefront with shuffles and, for multi-wave rows, across wavefronts through LDS; the
// second pass divides by the scale, rounds and stores the codes. Rows longer than the register budget
// re-read the remainder (it is still in L2).
//
// The arithmetic follows the quantizer of "QaRL: Rollout-Aligned Quantization-Aware RL ...", section 2.2
// (integer Quant with zero point 0; floating-point Quant with s = max|W| / alpha), with per-output-channel
// weight scales and per-token activation scales as in "QuRL: Efficient Reinforcement Learning with Quantized
// Rollout", section 5, and the optional invariant scale of QuRL section 4.3 folded in as W diag(s) or
// X diag(1/s). Each fp32 step is one IEEE operation (the division through div_by_scale, which returns the
// correctly rounded quotient), so codes and scales are bit-identical to any correct implementation.
#include "qr_device.hpp"
#include "qr_internal.hpp"

namespace qr {
namespace {

constexpr int kCMax = 8;  // 16-byte chunks held in registers per lane

template <bool BF16, int SMODE>
__device__ __forceinline__ void expand_chunk(const uint4 &c, const float *__restrict__ s, int64_t k0, float *w) {
    if constexpr (BF16) {
        const uint32_t p[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = bf16_lo(p[i]);
            w[2 * i + 1] = bf16_hi(p[i]);
        }
    } else {
        w[0] = __uint_as_float(c.x);
        w[1] = __uint_as_float(c.y);
        w[2] = __uint_as_float(c.z);
        w[3] = __uint_as_float(c.w);
    }
    constexpr int E = BF16 ? 8 : 4;
    if constexpr (SMODE == kSMul) {
#pragma unroll
        for (int i = 0; i < E; ++i) w[i] = w[i] * s[k0 + i];
    } else if constexpr (SMODE == kSMulRecip) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float rs = 1.0f / s[k0 + i];
            w[i] = w[i] * rs;
        }
    }
}

// THREADS lanes per row, RPB rows per workgroup (RPB > 1 only with one-wavefront rows)
template <bool BF16, int QT, int SMODE, int THREADS, int RPB>
__global__ __launch_bounds__(THREADS * RPB) void quantize_rows_kernel(const void *__restrict__ in, int64_t rows,
                                                                       int64_t k, const float *__restrict__ s,
                                                                       uint8_t *__restrict__ codes,
                                                                       float *__restrict__ scales) {
    static_assert(RPB == 1 || THREADS == 64, "several rows per workgroup only with one-wavefront rows");
    constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr float qmax = QMax<QT>::value;
    const int64_t row = (int64_t)blockIdx.x * RPB + (RPB > 1 ? (int)(threadIdx.x >> 6) : 0);
    if (row >= rows) return;  // whole wavefronts only (RPB > 1 implies one wavefront per row)
    const int t = RPB > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int64_t nch = k / E;
    const uint4 *__restrict__ src =
        reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(in) + row * k * (BF16 ? 2 : 4));

    uint4 keep[kCMax];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kCMax; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) {
            keep[i] = src[c];
            float w[E];
            expand_chunk<BF16, SMODE>(keep[i], s, c * E, w);
#pragma unroll
            for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(w[j]));
        }
    }
    for (int64_t c = t + (int64_t)kCMax * THREADS; c < nch; c += THREADS) {
        float w[E];
        expand_chunk<BF16, SMODE>(src[c], s, c * E, w);
#pragma unroll
        for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(w[j]));
    }

    amax = wave_max(amax);
    if constexpr (THREADS > 64) {
        __shared__ float red[THREADS / 64];
        if ((t & 63) == 0) red[t >> 6] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int i = 1; i < THREADS / 64; ++i) amax = fmaxf(amax, red[i]);
    }

    float S = amax / qmax;  // IEEE division
    if (!(S > 0.0f)) S = 1.0f;  // all-zero row, or a scale that underflows to zero
    const float r = 1.0f / S;
    const bool fast = S >= 0x1p-90f;
    if (t == 0) scales[row] = S;

    uint8_t *__restrict__ dst = codes + row * k;
    auto emit = [&](const uint4 &chunk, int64_t c) {
        float w[E];
        expand_chunk<BF16, SMODE>(chunk, s, c * E, w);
        uint32_t q[E];
#pragma unroll
        for (int j = 0; j < E; ++j) {
            float v = fast ? div_by_scale(w[j], S, r) : w[j] / S;
            v = fminf(fmaxf(v, -qmax), qmax);
            q[j] = encode_code<QT>(v);
        }
        if constexpr (BF16) {
            uint2 o;
            o.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
            o.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
            *reinterpret_cast<uint2 *>(dst + c * 8) = o;
        } else {
            *reinterpret_cast<uint32_t *>(dst + c * 4) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        }
    };
#pragma unroll
    for (int i = 0; i < kCMax; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) emit(keep[i], c);
    }
    for (int64_t c = t + (int64_t)kCMax * THREADS; c < nch; c += THREADS) emit(src[c], c);
}

template <bool BF16, int QT, int SMODE>
hipError_t launch_t(const void *in, int64_t rows, int64_t k, const float *s, uint8_t *codes, float *scales,
                    hipStream_t stream) {
    constexpr int E = BF16 ? 8 : 4;
    const int64_t nch = k / E;
    const dim3 grid((unsigned)rows);
    if (nch <= 64 * kCMax) {
        constexpr int kRows = 4;
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, 64, kRows>), dim3((unsigned)((rows + kRows - 1) / kRows)),
                           dim3(64 * kRows), 0, stream, in, rows, k, s, codes, scales);
    } else if (nch <= 128 * kCMax) {
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, 128, 1>), grid, dim3(128), 0, stream, in, rows, k, s,
                           codes, scales);
    } else if (nch <= 256 * kCMax) {
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, 256, 1>), grid, dim3(256), 0, stream, in, rows, k, s,
                           codes, scales);
    } else if (nch <= 512 * kCMax) {
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, 512, 1>), grid, dim3(512), 0, stream, in, rows, k, s,
                           codes, scales);
    } else {
        hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, 1024, 1>), grid, dim3(1024), 0, stream, in, rows, k,
                           s, codes, scales);
    }
    return hipGetLastError();
}

template <bool BF16, int QT>
hipError_t launch_s(const void *in, int64_t rows, int64_t k, const float *s, int s_mode, uint8_t *codes,
                    float *scales, hipStream_t stream) {
    switch (s_mode) {
        case kSMul:
            return launch_t<BF16, QT, kSMul>(in, rows, k, s, codes, scales, stream);
        case kSMulRecip:
            return launch_t<BF16, QT, kSMulRecip>(in, rows, k, s, codes, scales, stream);
        default:
            return launch_t<BF16, QT, kSNone>(in, rows, k, s, codes, scales, stream);
    }
}

}  // namespace

hipError_t launch_quantize_rows(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int s_mode,
                                int qtype, uint8_t *codes, float *scales, hipStream_t stream) {
    if (in_bf16) {
        return qtype == kInt8 ? launch_s<true, kInt8>(in, rows, k, s, s_mode, codes, scales, stream)
                              : launch_s<true, kFp8>(in, rows, k, s, s_mode, codes, scales, stream);
    }
    return qtype == kInt8 ? launch_s<false, kInt8>(in, rows, k, s, s_mode, codes, scales, stream)
                          : launch_s<false, kFp8>(in, rows, k, s, s_mode, codes, scales, stream);
}

}  // namespace qr
