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

#include <type_traits>

namespace qr {
namespace {

constexpr int kCMax = 8;  // 16-byte chunks held in registers per lane
constexpr int kCDiff = 4;  // the same with the previous publish's codes held too (keeps occupancy at 8 waves/SIMD)

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

// THREADS lanes per row, RPB rows per workgroup (RPB > 1 only with one-wavefront rows). With DIFF the kernel also
// compares every new code and the row's scale with the previous publish (prev_codes / prev_scales, which may be
// codes / scales themselves: each lane reads the previous bytes it then overwrites) and writes the row's
// changed-code triple {bytes, values, scale} to row_counts[row].
// Non-temporal 16-byte load and code stores for the weight quantizer: the masters, the previous codes and the new
// codes each pass through once, so they should not displace cached data (measured on MI355X over the 28-layer
// 1.5B-shaped publish: 740 -> 707 us; the requantize + diff form with the previous codes' loads non-temporal
// too: 1139 -> 1086 us). Activation codes are read right away by the linear and keep the default.
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4 *p) {
    if constexpr (NT) {
        const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
        return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    } else {
        return *p;
    }
}

template <bool NT>
__device__ __forceinline__ void st_codes(uint8_t *p, const uint2 &o) {
    if constexpr (NT) {
        typedef int v2i_t __attribute__((ext_vector_type(2)));
        const v2i_t v = {(int)o.x, (int)o.y};
        __builtin_nontemporal_store(v, reinterpret_cast<v2i_t *>(p));
    } else {
        *reinterpret_cast<uint2 *>(p) = o;
    }
}

template <bool NT>
__device__ __forceinline__ void st_codes(uint8_t *p, uint32_t o) {
    if constexpr (NT)
        __builtin_nontemporal_store(o, reinterpret_cast<uint32_t *>(p));
    else
        *reinterpret_cast<uint32_t *>(p) = o;
}

// non-temporal loads of the previous publish's code words (4 or 8 bytes), read once by the DIFF form
__device__ __forceinline__ uint32_t ld_nt(const uint32_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint2 ld_nt(const uint2 *p) {
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    const v2i_t v = __builtin_nontemporal_load(reinterpret_cast<const v2i_t *>(p));
    return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}

template <bool BF16, int QT, int SMODE, int THREADS, int RPB, bool DIFF, bool NT>
__global__ __launch_bounds__(THREADS * RPB) void quantize_rows_kernel(const void *__restrict__ in, int64_t rows,
                                                                       int64_t k, const float *__restrict__ s,
                                                                       uint8_t *codes, float *scales,
                                                                       const uint8_t *prev_codes,
                                                                       const float *prev_scales,
                                                                       int32_t *row_counts) {
    static_assert(RPB == 1 || THREADS == 64, "several rows per workgroup only with one-wavefront rows");
    constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr int kC = DIFF ? kCDiff : kCMax;  // chunks per lane held in registers
    constexpr float qmax = QMax<QT>::value;
    const int64_t row = (int64_t)blockIdx.x * RPB + (RPB > 1 ? (int)(threadIdx.x >> 6) : 0);
    if (row >= rows) return;  // whole wavefronts only (RPB > 1 implies one wavefront per row)
    const int t = RPB > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int64_t nch = k / E;
    const uint4 *__restrict__ src =
        reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(in) + row * k * (BF16 ? 2 : 4));

    // the previous codes of the chunks held in registers, requested first (their latency overlaps the first
    // pass) and all loaded before any store (the stores may overwrite them)
    typedef typename std::conditional<BF16, uint2, uint32_t>::type cword_t;
    const uint8_t *prev = DIFF ? prev_codes + row * k : nullptr;
    cword_t old_keep[DIFF ? kC : 1];
    if constexpr (DIFF) {
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            const int64_t c = t + (int64_t)i * THREADS;
            if (c < nch) old_keep[i] = ld_nt(reinterpret_cast<const cword_t *>(prev + c * E));
        }
    }

    uint4 keep[kC];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) {
            keep[i] = ld16<NT>(src + c);
            float w[E];
            expand_chunk<BF16, SMODE>(keep[i], s, c * E, w);
#pragma unroll
            for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(w[j]));
        }
    }
    for (int64_t c = t + (int64_t)kC * THREADS; c < nch; c += THREADS) {
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
    uint32_t scale_changed = 0;
    if (t == 0) {
        if constexpr (DIFF) {
            scale_changed = __float_as_uint(prev_scales[row]) != __float_as_uint(S) ? 1u : 0u;
            // in place the store below overwrites the previous scale. The read above is a scalar load (the
            // address is uniform), which is not ordered with a vector store: the comparison has to be complete
            // (so the load has returned) before the store is issued
            asm volatile("" ::"v"(scale_changed) : "memory");
        }
        scales[row] = S;
    }

    uint8_t *dst = codes + row * k;
    unsigned long long nb = 0, nv = 0;
    auto emit = [&](const uint4 &chunk, int64_t c, const cword_t &old) {
        float w[E];
        expand_chunk<BF16, SMODE>(chunk, s, c * E, w);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float v = fast ? div_by_scale(w[j], S, r) : w[j] / S;
            w[j] = fminf(fmaxf(v, -qmax), qmax);
        }
        if constexpr (BF16) {
            uint2 o;
            o.x = encode_code4<QT>(w);
            o.y = encode_code4<QT>(w + 4);
            if constexpr (DIFF) {
                count_word(old.x, o.x, QT == kFp8, nb, nv);
                count_word(old.y, o.y, QT == kFp8, nb, nv);
            }
            st_codes<NT>(dst + c * 8, o);
        } else {
            const uint32_t o = encode_code4<QT>(w);
            if constexpr (DIFF) count_word(old, o, QT == kFp8, nb, nv);
            st_codes<NT>(dst + c * 4, o);
        }
    };
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) emit(keep[i], c, DIFF ? old_keep[i] : cword_t{});
    }
    for (int64_t c = t + (int64_t)kC * THREADS; c < nch; c += THREADS)
        emit(src[c], c, DIFF ? *reinterpret_cast<const cword_t *>(prev + c * E) : cword_t{});

    if constexpr (DIFF) {
        // the row's triple: sums over its lanes (and wavefronts), written by lane 0
        nb = wave_sum_u64(nb);
        nv = wave_sum_u64(nv);
        if constexpr (THREADS > 64) {
            __shared__ unsigned long long cnt[2][THREADS / 64];
            if ((t & 63) == 0) {
                cnt[0][t >> 6] = nb;
                cnt[1][t >> 6] = nv;
            }
            __syncthreads();
            if (t == 0) {
                for (int i = 1; i < THREADS / 64; ++i) {
                    nb += cnt[0][i];
                    nv += cnt[1][i];
                }
            }
        }
        if (t == 0) {
            row_counts[3 * row + 0] = (int32_t)nb;
            row_counts[3 * row + 1] = (int32_t)nv;
            row_counts[3 * row + 2] = (int32_t)scale_changed;
        }
    }
}

// out3 = the column sums of row_counts [rows][3]: one workgroup, 64-bit sums in a fixed order per lane, then
// over the lanes and wavefronts
__global__ __launch_bounds__(1024) void sum_row_counts_kernel(const int32_t *__restrict__ row_counts, int64_t rows,
                                                              int64_t *__restrict__ out3) {
    unsigned long long a[3] = {0, 0, 0};
    for (int64_t r = threadIdx.x; r < rows; r += blockDim.x)
#pragma unroll
        for (int e = 0; e < 3; ++e) a[e] += (unsigned long long)(uint32_t)row_counts[3 * r + e];
    __shared__ unsigned long long part[3][16];
#pragma unroll
    for (int e = 0; e < 3; ++e) {
        a[e] = wave_sum_u64(a[e]);
        if ((threadIdx.x & 63) == 0) part[e][threadIdx.x >> 6] = a[e];
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        unsigned long long sum = 0;
        for (unsigned w = 0; w < blockDim.x / 64; ++w) sum += part[threadIdx.x][w];
        out3[threadIdx.x] = (int64_t)sum;
    }
}

// ---------------------------------------------------------------------------------------------------------
// RMSNorm producer of a linear's quantized input: h = bf16(x q gamma) per row, q = 1 / sqrt(mean(x^2) + eps)
// (0 for a zero radicand), in fp64 and rounded once, then the token-wise quantizer of h (h diag(1/s) with s).
// The same teams as the quantizer: the x chunks held in registers are replaced by their h chunks after the
// sum of squares, so the row is read from HBM once; chunks past the register budget are re-read (from L2) and
// their h recomputed, bit for bit the same. The squares of bfloat16 values are exact in fp64; their sum is
// taken per lane, then over the wavefront and the team in a fixed order.
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ uint4 rms_chunk(const uint4 &xc, const float *__restrict__ gamma, int64_t c, double q) {
    const float4 g0 = *reinterpret_cast<const float4 *>(gamma + 8 * c);
    const float4 g1 = *reinterpret_cast<const float4 *>(gamma + 8 * c + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t p[4] = {xc.x, xc.y, xc.z, xc.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f64_to_bf16((double)bf16_lo(p[i]) * q * (double)g[2 * i]);
        const uint32_t hi = f64_to_bf16((double)bf16_hi(p[i]) * q * (double)g[2 * i + 1]);
        o[i] = lo | (hi << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ double sum_sq_chunk(const uint4 &xc) {
    const uint32_t p[4] = {xc.x, xc.y, xc.z, xc.w};
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double lo = bf16_lo(p[i]), hi = bf16_hi(p[i]);
        a += lo * lo;
        a += hi * hi;
    }
    return a;
}

template <int QT, int SMODE, int THREADS, int RPB>
__global__ __launch_bounds__(THREADS * RPB) void rmsnorm_quant_kernel(const uint16_t *__restrict__ x, int64_t rows,
                                                                      int64_t k, const float *__restrict__ gamma,
                                                                      float eps, const float *__restrict__ s,
                                                                      uint8_t *__restrict__ codes,
                                                                      float *__restrict__ scales,
                                                                      uint16_t *__restrict__ h_out) {
    static_assert(RPB == 1 || THREADS == 64, "several rows per workgroup only with one-wavefront rows");
    constexpr int E = 8, kC = kCMax;
    constexpr float qmax = QMax<QT>::value;
    const int64_t row = (int64_t)blockIdx.x * RPB + (RPB > 1 ? (int)(threadIdx.x >> 6) : 0);
    if (row >= rows) return;  // whole wavefronts only (RPB > 1 implies one wavefront per row)
    const int t = RPB > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int64_t nch = k / E;
    const uint4 *__restrict__ src = reinterpret_cast<const uint4 *>(x + row * k);
    uint4 *__restrict__ hdst = h_out != nullptr ? reinterpret_cast<uint4 *>(h_out + row * k) : nullptr;

    uint4 keep[kC];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) {
            keep[i] = src[c];
            ss += sum_sq_chunk(keep[i]);
        }
    }
    for (int64_t c = t + (int64_t)kC * THREADS; c < nch; c += THREADS) ss += sum_sq_chunk(src[c]);
    ss = wave_sum_f64(ss);
    if constexpr (THREADS > 64) {
        __shared__ double red_ss[THREADS / 64];
        if ((t & 63) == 0) red_ss[t >> 6] = ss;
        __syncthreads();
        ss = red_ss[0];
#pragma unroll
        for (int i = 1; i < THREADS / 64; ++i) ss += red_ss[i];
    }
    const double d = ss / (double)k + (double)eps;
    const double q = d > 0.0 ? 1.0 / sqrt(d) : 0.0;

    float amax = 0.0f;
    auto absmax_of = [&](const uint4 &hc, int64_t c) {
        float w[E];
        expand_chunk<true, SMODE>(hc, s, c * E, w);
#pragma unroll
        for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(w[j]));
    };
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) {
            keep[i] = rms_chunk(keep[i], gamma, c, q);
            if (hdst != nullptr) hdst[c] = keep[i];
            absmax_of(keep[i], c);
        }
    }
    for (int64_t c = t + (int64_t)kC * THREADS; c < nch; c += THREADS) {
        const uint4 hc = rms_chunk(src[c], gamma, c, q);
        if (hdst != nullptr) hdst[c] = hc;
        absmax_of(hc, c);
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

    uint8_t *dst = codes + row * k;
    auto emit = [&](const uint4 &hc, int64_t c) {
        float w[E];
        expand_chunk<true, SMODE>(hc, s, c * E, w);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float v = fast ? div_by_scale(w[j], S, r) : w[j] / S;
            w[j] = fminf(fmaxf(v, -qmax), qmax);
        }
        uint2 o;
        o.x = encode_code4<QT>(w);
        o.y = encode_code4<QT>(w + 4);
        *reinterpret_cast<uint2 *>(dst + c * 8) = o;
    };
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        const int64_t c = t + (int64_t)i * THREADS;
        if (c < nch) emit(keep[i], c);
    }
    for (int64_t c = t + (int64_t)kC * THREADS; c < nch; c += THREADS) emit(rms_chunk(src[c], gamma, c, q), c);
}

// Lanes per row. Weights (many rows, streamed once): the smallest power of two of at least half the row's
// chunks (64..1024), halved while the launch exceeds 2^20 threads. Activations (few to a few thousand rows whose
// latency the next linear waits for): one chunk per lane (up to 1024 lanes), halved while rows x lanes exceeds
// 2^18. Both at least what holds every chunk in kC registers per lane; a row of one wavefront shares its
// workgroup with three others. Measured on MI355X (graph replay, bf16 to FP8; quantizer alone / with RMSNorm):
// K = 3584 at 1 and 16 rows 2.6 / 3.8 us with 512 lanes against 2.9 / 4.2 us with 256, at 2048 rows 5.6 / 10.5
// us with 128 against 6.0 / 11.8 with 256; K = 1536 at 2048 rows 4.0 / 6.6 us with 128; K = 18944 at 512 and
// 2048 rows 6.9 / 13.5 and 22.6 / 40.5 us with 512 lanes against 7.6 / 16.1 and 23.2 / 44.4 with 1024.
int team_lanes(int64_t rows, int64_t nch, int kC, bool acts) {
    int lanes = 64;
    if (acts) {
        while (lanes < 1024 && lanes < nch) lanes *= 2;
        while (lanes > 64 && rows * lanes > ((int64_t)1 << 18)) lanes /= 2;
    } else {
        while (lanes < 1024 && 2 * lanes < nch) lanes *= 2;
        while (lanes > 64 && rows * lanes > ((int64_t)1 << 20)) lanes /= 2;
    }
    const int minimum = nch <= 64 * kC ? 64 : nch <= 128 * kC ? 128 : nch <= 256 * kC ? 256 : nch <= 512 * kC ? 512 : 1024;
    if (lanes < minimum) lanes = minimum;  // the register budget: at most kC chunks per lane held
    const int forced = env_int("QR_QUANT_THREADS", 0);  // tuning sweeps
    if (forced == 64 || forced == 128 || forced == 256 || forced == 512 || forced == 1024) lanes = forced;
    return lanes;
}

struct DiffArgs {
    const uint8_t *prev_codes;
    const float *prev_scales;
    int32_t *row_counts;
};

template <bool BF16, int QT, int SMODE, bool DIFF, bool NT>
hipError_t launch_t(const void *in, int64_t rows, int64_t k, const float *s, uint8_t *codes, float *scales,
                    const DiffArgs &d, hipStream_t stream) {
    constexpr int E = BF16 ? 8 : 4;
    constexpr int kC = DIFF ? kCDiff : kCMax;
    const int64_t nch = k / E;
    const dim3 grid((unsigned)rows);
#define QR_QROWS(T, R, G)                                                                                      \
    hipLaunchKernelGGL((quantize_rows_kernel<BF16, QT, SMODE, T, R, DIFF, NT>), G, dim3(T * R), 0, stream, in, rows, \
                       k, s, codes, scales, d.prev_codes, d.prev_scales, d.row_counts)
    const int lanes = team_lanes(rows, nch, kC, !NT && !DIFF);  // weights stream (NT), activations do not
    if (lanes == 64) {
        constexpr int kRows = 4;
        QR_QROWS(64, kRows, dim3((unsigned)((rows + kRows - 1) / kRows)));
    } else if (lanes == 128) {
        QR_QROWS(128, 1, grid);
    } else if (lanes == 256) {
        QR_QROWS(256, 1, grid);
    } else if (lanes == 512) {
        QR_QROWS(512, 1, grid);
    } else {
        QR_QROWS(1024, 1, grid);
    }
#undef QR_QROWS
    return hipGetLastError();
}

template <bool BF16, int QT, bool DIFF>
hipError_t launch_s(const void *in, int64_t rows, int64_t k, const float *s, int s_mode, bool nt, uint8_t *codes,
                    float *scales, const DiffArgs &d, hipStream_t stream) {
    switch (s_mode) {
        case kSMul:
            return nt ? launch_t<BF16, QT, kSMul, DIFF, true>(in, rows, k, s, codes, scales, d, stream)
                      : launch_t<BF16, QT, kSMul, DIFF, false>(in, rows, k, s, codes, scales, d, stream);
        case kSMulRecip:  // activations only
            return launch_t<BF16, QT, kSMulRecip, DIFF, false>(in, rows, k, s, codes, scales, d, stream);
        default:
            return nt ? launch_t<BF16, QT, kSNone, DIFF, true>(in, rows, k, s, codes, scales, d, stream)
                      : launch_t<BF16, QT, kSNone, DIFF, false>(in, rows, k, s, codes, scales, d, stream);
    }
}

template <bool DIFF>
hipError_t launch_q(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int s_mode, bool nt,
                    int qtype, uint8_t *codes, float *scales, const DiffArgs &d, hipStream_t stream) {
    if (in_bf16) {
        return qtype == kInt8 ? launch_s<true, kInt8, DIFF>(in, rows, k, s, s_mode, nt, codes, scales, d, stream)
                              : launch_s<true, kFp8, DIFF>(in, rows, k, s, s_mode, nt, codes, scales, d, stream);
    }
    return qtype == kInt8 ? launch_s<false, kInt8, DIFF>(in, rows, k, s, s_mode, nt, codes, scales, d, stream)
                          : launch_s<false, kFp8, DIFF>(in, rows, k, s, s_mode, nt, codes, scales, d, stream);
}

}  // namespace

hipError_t launch_quantize_rows(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int s_mode,
                                int qtype, uint8_t *codes, float *scales, hipStream_t stream, bool streaming) {
    return launch_q<false>(in, in_bf16, rows, k, s, s_mode, streaming, qtype, codes, scales,
                           DiffArgs{nullptr, nullptr, nullptr}, stream);
}

hipError_t launch_rmsnorm_quant(const uint16_t *x, int64_t rows, int64_t k, const float *gamma, float eps,
                                const float *s, int qtype, uint8_t *codes, float *scales, uint16_t *h_out,
                                hipStream_t stream) {
    const int64_t nch = k / 8;
    const int lanes = team_lanes(rows, nch, kCMax, true);
    const dim3 grid((unsigned)rows);
#define QR_RMS(QT, SM, T, R, G)                                                                                  \
    hipLaunchKernelGGL((rmsnorm_quant_kernel<QT, SM, T, R>), G, dim3(T * R), 0, stream, x, rows, k, gamma, eps, s, \
                       codes, scales, h_out)
#define QR_RMS_T(QT, SM)                                                                                         \
    do {                                                                                                         \
        if (lanes == 64)                                                                                         \
            QR_RMS(QT, SM, 64, 4, dim3((unsigned)((rows + 3) / 4)));                                             \
        else if (lanes == 128)                                                                                   \
            QR_RMS(QT, SM, 128, 1, grid);                                                                        \
        else if (lanes == 256)                                                                                   \
            QR_RMS(QT, SM, 256, 1, grid);                                                                        \
        else if (lanes == 512)                                                                                   \
            QR_RMS(QT, SM, 512, 1, grid);                                                                        \
        else                                                                                                     \
            QR_RMS(QT, SM, 1024, 1, grid);                                                                       \
    } while (0)
    if (qtype == kInt8) {
        if (s != nullptr) QR_RMS_T(kInt8, kSMulRecip); else QR_RMS_T(kInt8, kSNone);
    } else {
        if (s != nullptr) QR_RMS_T(kFp8, kSMulRecip); else QR_RMS_T(kFp8, kSNone);
    }
#undef QR_RMS_T
#undef QR_RMS
    return hipGetLastError();
}

hipError_t launch_requantize(const void *in, bool in_bf16, int64_t rows, int64_t k, const float *s, int qtype,
                             const uint8_t *prev_codes, const float *prev_scales, uint8_t *codes, float *scales,
                             int32_t *row_counts, int64_t *out3, hipStream_t stream) {
    if (rows > 0) {  // no rows: out3 is still written (zeros)
        const hipError_t e = launch_q<true>(in, in_bf16, rows, k, s, s == nullptr ? kSNone : kSMul, true, qtype,
                                            codes, scales, DiffArgs{prev_codes, prev_scales, row_counts}, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sum_row_counts_kernel, dim3(1), dim3(1024), 0, stream, row_counts, rows, out3);
    return hipGetLastError();
}

}  // namespace qr
