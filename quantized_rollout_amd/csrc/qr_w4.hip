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
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
            const int32_t qi = (int32_t)__builtin_rintf(v);
            const uint32_t q = qi < 0 ? (uint32_t)(8 - qi) : (uint32_t)qi;  // sign and magnitude
            packed[i / 8] |= q << (4 * (i % 8));
        }
        *reinterpret_cast<uint2 *>(codes + row * (k / 2) + c0 / 2) = make_uint2(packed[0], packed[1]);
        if (p == 0) scales[row * groups + g] = S;
    }
}

// 8 sign-and-magnitude 4-bit codes (channel order: low nibble first) as 8 bfloat16 values, exactly. Each code
// (s, m) is moved into an e4m3 byte [s 0000 mmm], the subnormal (-1)^s m 2^-9, and v_cvt_scalef32_pk_bf16_fp8
// turns two such bytes into two bfloat16 values with the scale 2^9: 12 VALU instructions per 8 codes.
__device__ __forceinline__ v8bf dequant8(uint32_t d) {
    const uint32_t e = (d & 0x07070707u) | ((d << 4) & 0x80808080u);  // even channels 0 2 4 6, one per byte
    const uint32_t o = ((d >> 4) & 0x07070707u) | (d & 0x80808080u);  // odd channels 1 3 5 7
    const uint32_t p0 = __builtin_amdgcn_perm(o, e, 0x05010400u);     // channels 0 1 2 3
    const uint32_t p1 = __builtin_amdgcn_perm(o, e, 0x07030602u);     // channels 4 5 6 7
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p0, 512.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p0, 512.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p1, 512.0f, false);
    const v2bf f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p1, 512.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], f[0], f[1]};
}

__device__ __forceinline__ v8bf as_v8bf(const uint4 &a) {
    v8bf r;
    __builtin_memcpy(&r, &a, sizeof r);
    return r;
}

// ---------------------------------------------------------------------------------------------------------
// W4A16 GEMV (decode batches). A block of W = WT * WK waves owns one tile of 16 tokens and WT groups of NT tiles
// of 16 output channels; wave w works on channel group w / WK and takes the K groups (w % WK), (w % WK) + WK, ...
// of it (WK = 1: one wave streams all of K for its channels; WK > 1: the waves of a channel group split K and
// their partials meet in LDS, summed in wave order -- deterministic either way).
//
// Per K group a lane (j, gq) (j = lane & 15, gq = lane >> 4) takes the 64 bytes of token j's activations over
// channels [32 gq, 32 gq + 32) of the group, and for every tile the 16 code bytes of channel j over the same
// channels and the group's scale; four v_mfma_f32_16x16x32_bf16 per tile (A = activations, B = the codes
// decoded to bfloat16, the same lane -> K map on both sides) give the group's exact-product sums in fp32,
// scaled by S[channel, group] into the tile's accumulator.
//
// Activations: with XL the block first copies its valid token rows (all of K) into LDS and the MFMA operands
// are read from there (token rows past m read the last valid row, a broadcast); without XL (rows too large)
// each lane loads its operands from global memory. Codes and scales stream through a ring of D register
// stages: the loads of group i + D - 1 are issued before the arithmetic of group i.
// ---------------------------------------------------------------------------------------------------------
template <int NT, bool XL>
struct W4Stage {
    uint4 w[NT];
    float s[NT];
    uint4 x[XL ? 1 : 4];  // unused with XL
    int64_t g;
};

__host__ __device__ constexpr int64_t w4_xrow_bytes(int64_t k) { return 2 * k + 16; }  // padded: rows spread over banks

template <int NT, int D, bool XL, int WMAX>
__global__ __launch_bounds__(WMAX * 64) void w4a16_gemv_kernel(int64_t m, int64_t n, int64_t k,
                                                               const uint16_t *__restrict__ x,
                                                               const uint8_t *__restrict__ codes,
                                                               const float *__restrict__ scales,
                                                               void *__restrict__ y, int y_bf16, int wk,
                                                               int x_lds_bytes) {
    extern __shared__ __align__(16) uint8_t smem[];  // XL: [rows][2k + 16] activations; then [waves][NT][4][64] fp32
    float *wred = reinterpret_cast<float *>(smem + x_lds_bytes);
    const int waves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int cg = wave / wk, kp = wave - cg * wk;  // channel group, K part
    const int64_t groups = k / kW4Group;
    const int64_t col0 = ((int64_t)blockIdx.x * (waves / wk) + cg) * (16 * NT);
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int rows = (int)(m - m0 < 16 ? m - m0 : 16);  // valid token rows of this tile
    const int64_t tok = m0 + (j < rows ? j : rows - 1);  // token rows past m read the last (never stored)
    const uint16_t *__restrict__ xrow = x + tok * k + 32 * gq;
    const int64_t xstride = w4_xrow_bytes(k);
    const uint32_t xl = (uint32_t)((j < rows ? j : rows - 1) * xstride + 64 * gq);  // this lane's LDS operand
    // per tile: 32-bit byte offsets of this lane's codes and scales (the codes of one weight are < 4 GiB)
    uint32_t woff[NT], soff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t col = col0 + 16 * t + j;
        const int64_t colc = col < n ? col : n - 1;  // channels past n re-read the last (never stored)
        woff[t] = (uint32_t)(colc * (k / 2) + 16 * gq);
        soff[t] = (uint32_t)(colc * groups * 4);
    }
    const uint8_t *__restrict__ sbytes = reinterpret_cast<const uint8_t *>(scales);

    v4f acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    auto grp = [&](int64_t i) { return kp + i * wk; };  // the K group of this wave's step i
    auto load = [&](W4Stage<NT, XL> &st, int64_t g) {
        st.g = g;
        if constexpr (!XL) {
#pragma unroll
            for (int c = 0; c < 4; ++c) st.x[c] = *reinterpret_cast<const uint4 *>(xrow + g * kW4Group + 8 * c);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st.w[t] = *reinterpret_cast<const uint4 *>(codes + (woff[t] + (uint32_t)g * (kW4Group / 2)));
            st.s[t] = *reinterpret_cast<const float *>(sbytes + (soff[t] + (uint32_t)g * 4));
        }
    };
    auto compute = [&](const W4Stage<NT, XL> &st) {
        uint4 xv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (XL)
                xv[c] = *reinterpret_cast<const uint4 *>(smem + xl + (uint32_t)st.g * (2 * kW4Group) + 16 * c);
            else
                xv[c] = st.x[c];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            v4f a = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            const uint32_t wd[4] = {st.w[t].x, st.w[t].y, st.w[t].z, st.w[t].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xv[c]), dequant8(wd[c]), a, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(a[i], st.s[t], acc[t][i]);
        }
    };
    // steps of this wave (uniform across its lanes)
    const int64_t steps = kp < groups ? (groups - 1 - kp) / wk + 1 : 0;
    W4Stage<NT, XL> st[D];
    const bool ring = steps >= 2 * D - 1;  // enough steps for the unconditional ring below
    // the first loads are in flight while the activations are staged
    if (ring) {
#pragma unroll
        for (int u = 0; u < D - 1; ++u) load(st[u], grp(u));
    } else if (steps > 0) {
        load(st[0], grp(0));
    }
    if constexpr (XL) {
        // the tile's valid token rows, all of K, into LDS: 16-byte pieces, consecutive threads on consecutive
        // pieces of a row
        const int64_t per_row = k / 8;
        for (int64_t i = threadIdx.x; i < rows * per_row; i += blockDim.x) {
            const int64_t r = i / per_row, p = i - r * per_row;
            *reinterpret_cast<uint4 *>(smem + r * xstride + 16 * p) =
                *reinterpret_cast<const uint4 *>(x + (m0 + r) * k + 8 * p);
        }
        __syncthreads();
    }
    if (ring) {
        // steady state: D steps per iteration, every load unconditional (step i + u + D - 1 exists)
        int64_t i = 0;
        for (; i + 2 * D - 2 < steps; i += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                // program order kept: the scheduler would otherwise gather an iteration's loads at its end
                load(st[(u + D - 1) % D], grp(i + u + D - 1));
                __builtin_amdgcn_sched_barrier(0);
                compute(st[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last (fewer than 2D - 1) steps; stage of step i + u is u % D since i is a multiple of D
#pragma unroll
        for (int u = 0; u < 2 * D - 1; ++u) {
            if (i + u + D - 1 < steps) load(st[(u + D - 1) % D], grp(i + u + D - 1));
            if (i + u < steps) compute(st[u % D]);
        }
    } else {
        for (int64_t i = 0; i < steps; ++i) {
            if (i > 0) load(st[0], grp(i));
            compute(st[0]);
        }
    }

    // the waves of a channel group publish their partials; wave kp == t % wk of the group sums tile t over the
    // group's waves in K-part order
    if (wk > 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) wred[((wave * NT + t) * 4 + e) * 64 + lane] = acc[t][e];
        __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (wk > 1) {
            if (t % wk != kp) continue;
            const int w0 = cg * wk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float sum = wred[((w0 * NT + t) * 4 + e) * 64 + lane];
                for (int w = 1; w < wk; ++w) sum += wred[(((w0 + w) * NT + t) * 4 + e) * 64 + lane];
                acc[t][e] = sum;
            }
        }
        const int64_t col = col0 + 16 * t + j;
        if (col >= n) continue;
        // result C[token 4 gq + e][channel j] sits in this lane's element e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t row = m0 + 4 * gq + e;
            if (row < m) {
                if (y_bf16)
                    static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(acc[t][e]);
                else
                    static_cast<float *>(y)[row * n + col] = acc[t][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// W4A16 GEMV, LDS-ring form (the token tile's activation rows fit in LDS; one tile of 16 channels per wave).
// Waves are arranged as in w4a16_gemv_kernel (channel group w / WK, K part w % WK). Each wave streams its codes
// and scales through a private ring of D stages in LDS, filled by buffer loads that write LDS directly and
// counted with vmcnt by hand: the loads of group i + D - 1 are issued before group i is used, so D groups are
// in flight per wave without holding them in registers. Each lane reads back only the bytes its own load
// wrote, so the ring needs no barrier.
// ---------------------------------------------------------------------------------------------------------
constexpr int kW4RingStage = 1024 + 256;  // per stage: 64 lanes x 16 code bytes, then 64 lanes x 4 scale bytes

template <int D>
__global__ __launch_bounds__(1024) void w4a16_ring_kernel(int64_t m, int64_t n, int64_t k,
                                                          const uint16_t *__restrict__ x,
                                                          const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ scales, void *__restrict__ y,
                                                          int y_bf16, int wk, int x_lds_bytes) {
    // [rows][2k + 16] activations | [waves][D][kW4RingStage] rings | [waves][4][64] fp32 partials
    extern __shared__ __align__(16) uint8_t smem[];
    const int waves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int cg = wave / wk, kp = wave - cg * wk;
    const int64_t groups = k / kW4Group;
    const int64_t col = ((int64_t)blockIdx.x * (waves / wk) + cg) * 16 + j;
    const int64_t colc = col < n ? col : n - 1;  // channels past n re-read the last (never stored)
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int rows = (int)(m - m0 < 16 ? m - m0 : 16);
    const int64_t xstride = w4_xrow_bytes(k);
    const uint32_t xl = (uint32_t)((j < rows ? j : rows - 1) * xstride + 64 * gq);
    uint8_t *ring = smem + x_lds_bytes + wave * (D * kW4RingStage);
    float *wred = reinterpret_cast<float *>(smem + x_lds_bytes + waves * (D * kW4RingStage));
    const uint32_t ring_s = lds_addr(ring);
    // byte sizes below 4 GiB (the codes of one weight are checked on entry; the scales are 1/32 of them)
    const v4i rc = make_rsrc(codes, (uint32_t)(n * (k / 2)));
    const v4i rs = make_rsrc(scales, (uint32_t)(n * groups * 4));
    const uint32_t woff = (uint32_t)(colc * (k / 2) + 16 * gq);
    const uint32_t soff = (uint32_t)(colc * groups * 4);
    auto issue = [&](int64_t stage, int64_t g) {
        const uint32_t base = ring_s + (uint32_t)stage * kW4RingStage;
        dma16(rc, base, woff + (uint32_t)g * (kW4Group / 2));
        dma4(rs, base + 1024, soff + (uint32_t)g * 4);
    };
    const int64_t steps = kp < groups ? (groups - 1 - kp) / wk + 1 : 0;
    for (int u = 0; u < D - 1; ++u)
        if (u < steps) issue(u, kp + (int64_t)u * wk);
    {
        // the tile's valid token rows, all of K, into LDS (while the first groups are in flight)
        const int64_t per_row = k / 8;
        for (int64_t i = threadIdx.x; i < rows * per_row; i += blockDim.x) {
            const int64_t r = i / per_row, p = i - r * per_row;
            *reinterpret_cast<uint4 *>(smem + r * xstride + 16 * p) =
                *reinterpret_cast<const uint4 *>(x + (m0 + r) * k + 8 * p);
        }
        __syncthreads();
    }
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t i = 0; i < steps; ++i) {
        if (i + D - 1 < steps) {
            issue((i + D - 1) % D, kp + (i + D - 1) * wk);
            wait_vmcnt<2 * (D - 1)>();  // the two loads of group i have landed
        } else {
            wait_vmcnt<0>();
        }
        asm volatile("" ::: "memory");  // the ring reads below stay after the wait
        const uint8_t *st = ring + (i % D) * kW4RingStage;
        const uint4 wv = *reinterpret_cast<const uint4 *>(st + 16 * lane);
        const float S = *reinterpret_cast<const float *>(st + 1024 + 4 * lane);
        const uint32_t xg = xl + (uint32_t)(kp + i * wk) * (2 * kW4Group);
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
        v4f a = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(smem + xg + 16 * c);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(xv), dequant8(wd[c]), a, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(a[e], S, acc[e]);
        asm volatile("" ::: "memory");  // this stage's reads stay ahead of the load that refills it
    }

    if (wk > 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wred[(wave * 4 + e) * 64 + lane] = acc[e];
        __syncthreads();
        if (kp != 0) return;
        const int w0 = cg * wk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float sum = wred[(w0 * 4 + e) * 64 + lane];
            for (int w = 1; w < wk; ++w) sum += wred[((w0 + w) * 4 + e) * 64 + lane];
            acc[e] = sum;
        }
    }
    if (col >= n) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + 4 * gq + e;
        if (row < m) {
            if (y_bf16)
                static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(acc[e]);
            else
                static_cast<float *>(y)[row * n + col] = acc[e];
        }
    }
}

template <int D>
hipError_t launch_w4a16_ring(const W4Plan &p, int64_t m, int64_t n, int64_t k, const uint16_t *x,
                             const uint8_t *codes, const float *scales, void *y, bool y_bf16, hipStream_t stream) {
    // more than 64 KiB of dynamic LDS per block is opted into once per kernel
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&w4a16_ring_kernel<D>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)kW4MaxRingLds);
    if (attr != hipSuccess) return attr;
    const int64_t per_block = 16 * (p.waves / p.wk);
    const dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)((m + 15) / 16));
    const int x_lds = (int)(std::min<int64_t>(m, 16) * w4_xrow_bytes(k));
    hipLaunchKernelGGL((w4a16_ring_kernel<D>), grid, dim3(p.waves * 64), w4_lds_bytes(p, m, k), stream, m, n, k, x,
                       codes, scales, y, y_bf16 ? 1 : 0, p.wk, x_lds);
    return hipGetLastError();
}

template <int NT, int D, bool XL>
void launch_w4a16_t(const W4Plan &p, int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                    const float *scales, void *y, bool y_bf16, hipStream_t stream) {
    const int64_t per_block = 16 * NT * (p.waves / p.wk);
    const dim3 grid((unsigned)((n + per_block - 1) / per_block), (unsigned)((m + 15) / 16));
    const int x_lds = XL ? (int)(std::min<int64_t>(m, 16) * w4_xrow_bytes(k)) : 0;
    hipLaunchKernelGGL((w4a16_gemv_kernel<NT, D, XL, 16>), grid, dim3(p.waves * 64), w4_lds_bytes(p, m, k), stream,
                       m, n, k, x, codes, scales, y, y_bf16 ? 1 : 0, p.wk, x_lds);
}

}  // namespace

W4Plan plan_w4a16(int64_t m, int64_t n, int64_t k) {
    W4Plan p{};
    const int64_t groups = k / kW4Group;
    const int64_t tiles = (n + 15) / 16;
    const int64_t rows = std::min<int64_t>(m, 16);
    // LDS ring (one channel tile per wave): K split until about eight waves per SIMD exist in total (a wave's
    // own load rate is limited, so the waves in flight set the bandwidth), two stages per wave. Taken when the
    // staged activation rows stay small beside the codes a block streams (rows * wk <= waves: at most a
    // quarter of them) and everything fits in the CU's LDS. Measured on MI355X, 7B shapes at m = 1.
    p.tiles = 1;
    p.depth = 2;
    p.wk = 1;
    while (p.wk < 16 && tiles * p.wk < 8192 && p.wk < groups) p.wk *= 2;
    p.waves = std::max(8, p.wk);
    p.x_lds = true;
    p.ring = rows * p.wk <= p.waves;
    if (!p.ring) {
        // register stages: more channel tiles per wave when there are many, all eight waves splitting K,
        // activation operands from global memory unless the staged rows are few (m = 16 on the 7B shapes)
        p.tiles = tiles >= 2048 ? 4 : tiles >= 256 ? 2 : 1;
        p.waves = 8;
        p.wk = 8;
        p.depth = 1;
        p.x_lds = rows <= p.tiles;
    }
    const int fr = env_int("QR_W4_RING", -1), ft = env_int("QR_W4_TILES", 0), fw = env_int("QR_W4_WAVES", 0),
              fk = env_int("QR_W4_WK", 0), fd = env_int("QR_W4_DEPTH", 0), fx = env_int("QR_W4_XLDS", -1);
    if (fr >= 0) p.ring = fr != 0;
    if (ft == 1 || ft == 2 || ft == 4) p.tiles = ft;
    if (fw >= 1 && fw <= 16) p.waves = fw;
    if (fk >= 1) p.wk = fk;
    if (fd == 1 || fd == 2 || fd == 4 || fd == 8) p.depth = fd;
    if (fx >= 0) p.x_lds = fx != 0;
    if (p.wk > p.waves || p.waves % p.wk != 0) p.wk = p.waves;  // K parts must divide the waves
    if (p.ring) {
        p.x_lds = true;
        p.tiles = 1;
        if (p.depth < 2) p.depth = 2;
        if (w4_lds_bytes(p, m, k) > kW4MaxRingLds) p.ring = false;
    }
    if (!p.ring) {
        if (p.depth > 2) p.depth = 2;
        if (p.tiles == 4) p.depth = 1;  // four tiles with two stages would not fit the register file
        if (p.x_lds && w4_lds_bytes(p, m, k) > kW4MaxLds) p.x_lds = false;
    }
    return p;
}

size_t w4_lds_bytes(const W4Plan &p, int64_t m, int64_t k) {
    const size_t xb = p.x_lds ? (size_t)(std::min<int64_t>(m, 16) * w4_xrow_bytes(k)) : 0;
    if (p.ring)
        return xb + (size_t)p.waves * p.depth * kW4RingStage + (p.wk > 1 ? (size_t)p.waves * 4 * 64 * sizeof(float) : 0);
    return xb + (p.wk > 1 ? (size_t)p.waves * p.tiles * 4 * 64 * sizeof(float) : 0);
}

hipError_t launch_w4a16(const W4Plan &p, int64_t m, int64_t n, int64_t k, const uint16_t *x, const uint8_t *codes,
                        const float *scales, void *y, bool y_bf16, hipStream_t stream) {
    if (p.waves < 1 || p.waves > 16 || p.wk < 1 || p.waves % p.wk != 0) return hipErrorInvalidConfiguration;
    if (p.ring) {
        if (!p.x_lds || p.tiles != 1 || w4_lds_bytes(p, m, k) > kW4MaxRingLds) return hipErrorInvalidConfiguration;
        switch (p.depth) {
            case 2: return launch_w4a16_ring<2>(p, m, n, k, x, codes, scales, y, y_bf16, stream);
            case 4: return launch_w4a16_ring<4>(p, m, n, k, x, codes, scales, y, y_bf16, stream);
            case 8: return launch_w4a16_ring<8>(p, m, n, k, x, codes, scales, y, y_bf16, stream);
            default: return hipErrorInvalidConfiguration;
        }
    }
    if (w4_lds_bytes(p, m, k) > kW4MaxLds) return hipErrorInvalidConfiguration;
#define QR_W4_LAUNCH(NT, D, XL) launch_w4a16_t<NT, D, XL>(p, m, n, k, x, codes, scales, y, y_bf16, stream)
    const int key = p.tiles * 100 + p.depth * 10 + (p.x_lds ? 1 : 0);
    switch (key) {
        case 111: QR_W4_LAUNCH(1, 1, true); break;
        case 121: QR_W4_LAUNCH(1, 2, true); break;
        case 110: QR_W4_LAUNCH(1, 1, false); break;
        case 120: QR_W4_LAUNCH(1, 2, false); break;
        case 211: QR_W4_LAUNCH(2, 1, true); break;
        case 221: QR_W4_LAUNCH(2, 2, true); break;
        case 210: QR_W4_LAUNCH(2, 1, false); break;
        case 220: QR_W4_LAUNCH(2, 2, false); break;
        case 411: QR_W4_LAUNCH(4, 1, true); break;
        case 410: QR_W4_LAUNCH(4, 1, false); break;
        default: return hipErrorInvalidConfiguration;
    }
#undef QR_W4_LAUNCH
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
