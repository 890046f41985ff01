// qr_w4.hip -- W4A16: group-wise INT4 weight quantization and the INT4-weight x bf16-activation linear.
//
// The rollout engine of "QaRL: Rollout-Aligned Quantization-Aware RL ..." runs W8A8 or W4A16 (section 3.1:
// on large and MoE models W4A16 decodes faster because decode is memory-bound), with the integer Quant /
// Dequant of its section 2.2. Reading (the pages fix neither the group size nor the range): symmetric, z = 0,
// q in [-7, 7], one fp32 scale S = max|w'| / 7 per group of kW4Group = 128 consecutive input channels of a
// weight row, two codes per byte with the even channel in the low nibble. The product is
//   y[m, n] = sum_g S[n, g] * sum_{j in g} x[m, j] * q[n, j]      (x bfloat16, exact products)
// and only the weights are quantized, so the codes are the only integer decision (bit-exact against any
// correct implementation); y is an fp32 sum.
#include "qr_device.hpp"
#include "qr_internal.hpp"

#include <algorithm>

namespace qr {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------------------------------
// Quantizer: one wavefront per weight row; each group of 128 channels is handled by 8 lanes (16 channels
// each), eight groups per pass. Per group: absmax over the 8 lanes (shuffles), S = a / 7 (IEEE division, 1 when
// zero), the correctly rounded quotients w' / S, round half to even, clamp, pack.
// ---------------------------------------------------------------------------------------------------------
template <bool BF16, bool SMUL>
__global__ __launch_bounds__(256) void quantize_w4_kernel(const void *__restrict__ in, int64_t rows, int64_t k,
                                                          const float *__restrict__ s, uint8_t *__restrict__ codes,
                                                          float *__restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // a whole wavefront; the kernel has no block-wide synchronization
    const int gi = lane >> 3, p = lane & 7;
    const int64_t groups = k / kW4Group;
    for (int64_t base = 0; base < groups; base += 8) {
        const int64_t g = base + gi;
        const bool valid = g < groups;
        const int64_t c0 = g * kW4Group + p * 16;  // first channel of this lane
        float w[16];
        if (valid) {
            if constexpr (BF16) {
                const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(in) + row * k + c0);
                const uint4 a = src[0], b = src[1];
                const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    w[2 * i] = bf16_lo(u[i]);
                    w[2 * i + 1] = bf16_hi(u[i]);
                }
            } else {
                const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(in) + row * k + c0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 v = src[i];
                    w[4 * i] = v.x;
                    w[4 * i + 1] = v.y;
                    w[4 * i + 2] = v.z;
                    w[4 * i + 3] = v.w;
                }
            }
            if constexpr (SMUL) {
                const float4 *sv = reinterpret_cast<const float4 *>(s + c0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 v = sv[i];
                    w[4 * i] = w[4 * i] * v.x;
                    w[4 * i + 1] = w[4 * i + 1] * v.y;
                    w[4 * i + 2] = w[4 * i + 2] * v.z;
                    w[4 * i + 3] = w[4 * i + 3] * v.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = 0.0f;
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
        // the 8 lanes of a group are an aligned run of 8: xor 1, 2, 4 stays inside it
        a = fmaxf(a, __shfl_xor(a, 1, 64));
        a = fmaxf(a, __shfl_xor(a, 2, 64));
        a = fmaxf(a, __shfl_xor(a, 4, 64));
        if (!valid) continue;
        float S = a / 7.0f;  // IEEE division
        if (!(S > 0.0f)) S = 1.0f;
        const float r = 1.0f / S;
        const bool fast = S >= 0x1p-90f;
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v = fast ? div_by_scale(w[i], S, r) : w[i] / S;
            v = fminf(fmaxf(v, -7.0f), 7.0f);
            const uint32_t q = (uint32_t)(int32_t)__builtin_rintf(v) & 0xFu;
            packed[i / 8] |= q << (4 * (i % 8));
        }
        *reinterpret_cast<uint2 *>(codes + row * (k / 2) + c0 / 2) = make_uint2(packed[0], packed[1]);
        if (p == 0) scales[row * groups + g] = S;
    }
}

// 8 signed 4-bit codes (channel order: low nibble first) as 8 bfloat16 values (exact: |q| <= 8)
__device__ __forceinline__ v8bf dequant8(uint32_t d) {
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // signed field extract on a signed operand (an unsigned one would make the result unsigned)
        const float lo = (float)(int)__builtin_amdgcn_sbfe((int)d, 8 * i, 4);
        const float hi = (float)(int)__builtin_amdgcn_sbfe((int)d, 8 * i + 4, 4);
        out[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
    v8bf r;
    __builtin_memcpy(&r, out, sizeof r);
    return r;
}

__device__ __forceinline__ v8bf as_v8bf(const uint4 &a) {
    v8bf r;
    __builtin_memcpy(&r, &a, sizeof r);
    return r;
}

// ---------------------------------------------------------------------------------------------------------
// W4A16 GEMV (decode batches): a block owns one tile of 16 output channels and 16 tokens; its waves split the
// K groups, U consecutive groups per wave and round. Per group a lane (j, gq) (j = lane & 15, gq = lane >> 4)
// loads the 16 code bytes of channel j covering channels [32 gq, 32 gq + 32) of the group and the 64 bytes of
// token j's activations over the same channels; four v_mfma_f32_16x16x32_bf16 (A = activations, B = the
// codes unpacked to bfloat16, the same lane -> K map on both sides) give the group's exact-product sums in
// fp32, which are scaled by S[channel, group] and added to the accumulator. The waves' accumulators meet in
// LDS in wave order (deterministic).
// ---------------------------------------------------------------------------------------------------------
template <int U, int WMAX>
__global__ __launch_bounds__(WMAX * 64) void w4a16_gemv_kernel(int64_t m, int64_t n, int64_t k,
                                                               const uint16_t *__restrict__ x,
                                                               const uint8_t *__restrict__ codes,
                                                               const float *__restrict__ scales,
                                                               void *__restrict__ y, int y_bf16) {
    extern __shared__ float wred[];  // [waves][4][64]
    const int waves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int64_t groups = k / kW4Group;
    const int64_t col = (int64_t)blockIdx.x * 16 + j;
    const int64_t colc = col < n ? col : n - 1;       // channels past n re-read the last (never stored)
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int64_t tok = m0 + j < m ? m0 + j : m - 1;   // tokens past m re-read the last (never stored)
    const uint8_t *__restrict__ wrow = codes + colc * (k / 2) + 16 * gq;
    const uint16_t *__restrict__ xrow = x + tok * k + 32 * gq;
    const float *__restrict__ srow = scales + colc * groups;

    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto group_step = [&](const uint4 &wv, const uint4 (&xv)[4], float S) {
        v4f a = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xv[t]), dequant8(wd[t]), a, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(a[i], S, acc[i]);
    };
    // full rounds: wave w takes groups round * waves * U + w * U + u, u < U
    const int64_t per_round = (int64_t)waves * U;
    const int64_t full_rounds = groups / per_round;
    for (int64_t rd = 0; rd < full_rounds; ++rd) {
        const int64_t g0 = rd * per_round + (int64_t)wave * U;
        uint4 wv[U], xv[U][4];
        float S[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u;
            wv[u] = *reinterpret_cast<const uint4 *>(wrow + g * (kW4Group / 2));
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[u][t] = *reinterpret_cast<const uint4 *>(xrow + g * kW4Group + 8 * t);
            S[u] = srow[g];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) group_step(wv[u], xv[u], S[u]);
    }
    // the remaining groups, one at a time
    for (int64_t g = full_rounds * per_round + wave; g < groups; g += waves) {
        uint4 xv[4];
        const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + g * (kW4Group / 2));
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = *reinterpret_cast<const uint4 *>(xrow + g * kW4Group + 8 * t);
        group_step(wv, xv, srow[g]);
    }

    // reduction over the waves, in wave order, by wave 0; then the epilogue
    if (waves > 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wred[(wave * 4 + i) * 64 + lane] = acc[i];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sum = wred[i * 64 + lane];
            for (int w = 1; w < waves; ++w) sum += wred[(w * 4 + i) * 64 + lane];
            acc[i] = sum;
        }
    }
    if (col >= n) return;
    // result C[token 4 gq + i][channel j] sits in this lane's element i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + 4 * gq + i;
        if (row < m) {
            if (y_bf16)
                static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(acc[i]);
            else
                static_cast<float *>(y)[row * n + col] = acc[i];
        }
    }
}

template <int U, int WMAX>
void launch_w4a16_t(int waves, int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                    const float *scales, void *y, bool y_bf16, hipStream_t stream) {
    const dim3 grid((unsigned)((n + 15) / 16), (unsigned)((m + 15) / 16));
    const size_t lds = waves > 1 ? (size_t)waves * 4 * 64 * sizeof(float) : 0;
    hipLaunchKernelGGL((w4a16_gemv_kernel<U, WMAX>), grid, dim3(waves * 64), lds, stream, m, n, k, x, codes, scales,
                       y, y_bf16 ? 1 : 0);
}

}  // namespace

W4Plan plan_w4a16(int64_t m, int64_t n, int64_t k) {
    (void)m;
    W4Plan p{};
    const int64_t groups = k / kW4Group;
    const int64_t tiles = (n + 15) / 16;
    p.unroll = env_int("QR_W4_UNROLL", 2);
    if (p.unroll != 1 && p.unroll != 2 && p.unroll != 4) p.unroll = 2;
    // few waves per block when there are many channel tiles (more blocks resident), more when few
    int64_t waves = std::max<int64_t>(1, std::min<int64_t>(groups / p.unroll, tiles < 128 ? 8 : 4));
    const int fw = env_int("QR_W4_WAVES", 0);
    if (fw >= 1 && fw <= 16) waves = fw;
    p.waves = (int)waves;
    return p;
}

hipError_t launch_w4a16(const W4Plan &p, int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                        const float *scales, void *y, bool y_bf16, hipStream_t stream) {
    switch (p.unroll) {
        case 1: launch_w4a16_t<1, 16>(p.waves, m, n, k, x, codes, scales, y, y_bf16, stream); break;
        case 4: launch_w4a16_t<4, 16>(p.waves, m, n, k, x, codes, scales, y, y_bf16, stream); break;
        default: launch_w4a16_t<2, 16>(p.waves, m, n, k, x, codes, scales, y, y_bf16, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_w4(const void *in, bool bf16, int64_t rows, int64_t k, const float *s, uint8_t *codes,
                              float *scales, hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (bf16) {
        if (s)
            hipLaunchKernelGGL((quantize_w4_kernel<true, true>), grid, dim3(256), 0, stream, in, rows, k, s, codes, scales);
        else
            hipLaunchKernelGGL((quantize_w4_kernel<true, false>), grid, dim3(256), 0, stream, in, rows, k, s, codes,
                               scales);
    } else {
        if (s)
            hipLaunchKernelGGL((quantize_w4_kernel<false, true>), grid, dim3(256), 0, stream, in, rows, k, s, codes,
                               scales);
        else
            hipLaunchKernelGGL((quantize_w4_kernel<false, false>), grid, dim3(256), 0, stream, in, rows, k, s, codes,
                               scales);
    }
    return hipGetLastError();
}

}  // namespace qr
