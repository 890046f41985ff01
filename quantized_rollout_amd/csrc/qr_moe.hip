// qr_moe.hip -- the MoE glue around the grouped W8A8 linear: routing into per-expert token lists, the
// SiLU-gated product fused with the per-row quantization of the down projection's input, and the
// routing-weighted combine of the expert outputs.
//
// The expert FFN is that of the Qwen3-30B-A3B model the abstract of "QaRL: Rollout-Aligned Quantization-Aware
// RL ..." trains, with its linears in W8A8 as in QaRL section 3.1. The pages fix no routing rule, gate or
// combine; the library reads them as: each token takes its top_k largest logits (ties to the lower expert
// index), weighted by the softmax over those logits; h = silu(g) u over the fused gate/up output; the token's
// output is the weighted sum of its experts' down outputs.
//
// Everything that is decided on floating point (the bf16 rounding of h and of the combined output, the
// fp32 routing weights) is computed in fp64 and rounded once, so the results are those of the plain
// definition; the codes of h follow the activation quantizer step for step (IEEE fp32 division through the
// correctly rounded reciprocal form, round half to even, E4M3 nearest-even).
#include "qr_device.hpp"
#include "qr_internal.hpp"

namespace qr {
namespace {

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// ---------------------------------------------------------------------------------------------------------
// Routing, step 1: top-k of each token's logits and the softmax weights. One wavefront per token; lane l
// holds experts l, l + 64, ... as 64-bit keys (order-preserving bits of the logit, then the complement of
// the expert index, so the maximum key is the largest logit with ties to the lower index). k rounds of a
// wavefront maximum pick the choices; they are then stored in expert order.
// ---------------------------------------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int64_t T, int E, int k,
                                                         int32_t *__restrict__ topk_expert,
                                                         float *__restrict__ topk_weight) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefronts
    const float *l = logits + t * E;
    unsigned long long key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = 0;
        if (e < E) {
            float f = l[e];
            uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);  // -0 ties with +0
            const uint32_t fk = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            key[i] = ((unsigned long long)fk << 32) | (uint32_t)~(uint32_t)e;
        }
    }
    uint32_t taken = 0;
    int my_e = 0;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        unsigned long long best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (!((taken >> i) & 1u) && key[i] > best) best = key[i];
        best = wave_max_u64(best);
        const int e = (int)~(uint32_t)best;
        if ((e & 63) == lane) taken |= 1u << (e >> 6);
        if (j == lane) my_e = e;
    }
    // lanes 0..k-1 hold the choices in descending logit order; lane 0 has the largest logit
    const bool active = lane < k;
    const float my_l = active ? l[my_e] : 0.0f;
    int rank = 0;  // position in expert order
#pragma unroll 1
    for (int i = 0; i < k; ++i) {
        const int ei = __shfl(my_e, i, 64);
        rank += (active && ei < my_e) ? 1 : 0;
    }
    const double mx = (double)__shfl(my_l, 0, 64);
    const double ex = active ? exp((double)my_l - mx) : 0.0;
    double sum = 0.0;  // in expert order
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        const unsigned long long sel = __ballot(active && rank == r);
        sum += __shfl(ex, (int)__builtin_ctzll(sel), 64);
    }
    if (active) {
        topk_expert[t * k + rank] = my_e;
        topk_weight[t * k + rank] = (float)(ex / sum);
    }
}

// ---------------------------------------------------------------------------------------------------------
// Routing, step 2: the CSR lists (one workgroup of 8 wavefronts). Per-expert counts, their exclusive scan
// (expert_offsets), then the stable placement: token t's row for expert e is
//   offsets[e] + #{t' < t : t' chose e}
// computed chunk by chunk (512 tokens, one per thread): each wavefront ORs its lanes' bits into a 64-bit mask
// per expert, a thread per expert turns the masks into per-wavefront bases, and each choice adds the popcount
// of the lower lanes of its mask. All of it is order-independent, so the lists are deterministic.
// ---------------------------------------------------------------------------------------------------------
constexpr int kCsrThreads = 512;
constexpr int kCsrWaves = kCsrThreads / 64;
constexpr int kMaxExperts = 512;

__global__ __launch_bounds__(kCsrThreads) void route_csr_kernel(const int32_t *__restrict__ topk_expert,
                                                                const float *__restrict__ topk_weight, int64_t T,
                                                                int E, int k, int32_t *__restrict__ offsets,
                                                                int32_t *__restrict__ row_ids,
                                                                float *__restrict__ row_weights,
                                                                int32_t *__restrict__ pair_rows) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int off[kMaxExperts];
    __shared__ int carry[kMaxExperts];
    __shared__ int wsum[kCsrWaves];
    __shared__ unsigned long long mask[kCsrWaves][kMaxExperts];
    __shared__ int wbase[kCsrWaves][kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t pairs = T * k;

    for (int e = tid; e < E; e += kCsrThreads) {
        cnt[e] = 0;
        carry[e] = 0;
    }
    __syncthreads();
    for (int64_t p = tid; p < pairs; p += kCsrThreads) atomicAdd(&cnt[topk_expert[p]], 1);
    __syncthreads();

    // exclusive scan of cnt: wavefront w scans experts [64 w, 64 w + 64), then the wavefront totals
    {
        const int e = tid;
        const int c = e < E ? cnt[e] : 0;
        int incl = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (e < E) {
            off[e] = before + incl - c;
            offsets[e] = before + incl - c;
        }
        if (e == E - 1) offsets[E] = before + incl;
    }
    __syncthreads();

    for (int64_t t0 = 0; t0 < T; t0 += kCsrThreads) {
        for (int e = lane; e < E; e += 64) mask[wave][e] = 0;
        __syncthreads();
        const int64_t t = t0 + tid;
        const unsigned long long bit = 1ull << lane;
        if (t < T)
            for (int j = 0; j < k; ++j) atomicOr(&mask[wave][topk_expert[t * k + j]], bit);
        __syncthreads();
        for (int e = tid; e < E; e += kCsrThreads) {
            int run = carry[e];
#pragma unroll
            for (int w = 0; w < kCsrWaves; ++w) {
                wbase[w][e] = run;
                run += __popcll(mask[w][e]);
            }
            carry[e] = run;
        }
        __syncthreads();
        if (t < T) {
            for (int j = 0; j < k; ++j) {
                const int e = topk_expert[t * k + j];
                const int pos = off[e] + wbase[wave][e] + __popcll(mask[wave][e] & (bit - 1));
                row_ids[pos] = (int32_t)t;
                row_weights[pos] = topk_weight[t * k + j];
                pair_rows[t * k + j] = pos;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------------------
// h = bf16(silu(g) u) of the fused gate/up output y_gu [rows, 2I] (gate columns first), then the per-row
// absmax quantization of h (optionally of h diag(1/s)) for the down projection. One wavefront per row, four
// rows per workgroup, 4 elements (8 bytes of g and of u) per lane and chunk; up to kHold chunks per lane stay
// in registers between the absmax and the encoding, the rest are recomputed (the same value, bit for bit).
// ---------------------------------------------------------------------------------------------------------
constexpr int kHold = 4;

template <bool S>
__device__ __forceinline__ void silu_chunk(const uint16_t *__restrict__ g, const uint16_t *__restrict__ u, int64_t c,
                                           const float *__restrict__ s, float *hv, uint2 *hb) {
    const uint2 gp = *reinterpret_cast<const uint2 *>(g + 4 * c);
    const uint2 up = *reinterpret_cast<const uint2 *>(u + 4 * c);
    const float gf[4] = {bf16_lo(gp.x), bf16_hi(gp.x), bf16_lo(gp.y), bf16_hi(gp.y)};
    const float uf[4] = {bf16_lo(up.x), bf16_hi(up.x), bf16_lo(up.y), bf16_hi(up.y)};
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double gd = (double)gf[i];
        const double h = gd / (1.0 + exp(-gd)) * (double)uf[i];
        b[i] = f64_to_bf16(h);
        float v = __uint_as_float(b[i] << 16);
        if constexpr (S) {
            const float rs = 1.0f / s[4 * c + i];
            v = v * rs;
        }
        hv[i] = v;
    }
    if (hb != nullptr) *hb = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

template <int QT, bool S>
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(const uint16_t *__restrict__ y_gu, int64_t rows,
                                                             int64_t I, const float *__restrict__ s,
                                                             uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                             uint16_t *__restrict__ h_out) {
    constexpr float qmax = QMax<QT>::value;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // whole wavefronts
    const uint16_t *g = y_gu + row * 2 * I;
    const uint16_t *u = g + I;
    const int64_t nch = I / 4;

    float keep[kHold][4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        const int64_t c = lane + 64 * i;
        if (c < nch) {
            uint2 hb;
            silu_chunk<S>(g, u, c, s, keep[i], h_out != nullptr ? &hb : nullptr);
            if (h_out != nullptr) *reinterpret_cast<uint2 *>(h_out + row * I + 4 * c) = hb;
#pragma unroll
            for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(keep[i][j]));
        }
    }
    for (int64_t c = lane + 64 * kHold; c < nch; c += 64) {
        float hv[4];
        uint2 hb;
        silu_chunk<S>(g, u, c, s, hv, h_out != nullptr ? &hb : nullptr);
        if (h_out != nullptr) *reinterpret_cast<uint2 *>(h_out + row * I + 4 * c) = hb;
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(hv[j]));
    }
    amax = wave_max(amax);
    float Sc = amax / qmax;       // IEEE division
    if (!(Sc > 0.0f)) Sc = 1.0f;  // all-zero row, or a scale that underflows to zero
    const float r = 1.0f / Sc;
    const bool fast = Sc >= 0x1p-90f;
    if (lane == 0) scales[row] = Sc;

    uint8_t *dst = codes + row * I;
    auto emit = [&](const float *hv, int64_t c) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = fast ? div_by_scale(hv[j], Sc, r) : hv[j] / Sc;
            v[j] = fminf(fmaxf(x, -qmax), qmax);
        }
        *reinterpret_cast<uint32_t *>(dst + 4 * c) = encode_code4<QT>(v);
    };
#pragma unroll
    for (int i = 0; i < kHold; ++i) {
        const int64_t c = lane + 64 * i;
        if (c < nch) emit(keep[i], c);
    }
    for (int64_t c = lane + 64 * kHold; c < nch; c += 64) {
        float hv[4];
        silu_chunk<S>(g, u, c, s, hv, nullptr);
        emit(hv, c);
    }
}

// ---------------------------------------------------------------------------------------------------------
// out[t, :] = bf16(sum_j topk_weight[t, j] y_down[pair_rows[t, j], :]) in fp64, j ascending. One workgroup
// per token, 8 bf16 columns (16 bytes) per lane and step; a pair row outside [0, rows) adds nothing.
// ---------------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ y_down, int64_t rows,
                                                          const float *__restrict__ topk_weight,
                                                          const int32_t *__restrict__ pair_rows, int k, int64_t H,
                                                          uint16_t *__restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t nch = H / 8;
    for (int64_t c = threadIdx.x; c < nch; c += blockDim.x) {
        double acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            const int64_t pr = pair_rows[t * k + j];
            if (pr < 0 || pr >= rows) continue;
            const double w = (double)topk_weight[t * k + j];
            const uint4 v = *reinterpret_cast<const uint4 *>(y_down + pr * H + 8 * c);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += w * (double)bf16_lo(p[i]);
                acc[2 * i + 1] += w * (double)bf16_hi(p[i]);
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = (uint32_t)f64_to_bf16(acc[2 * i]) | ((uint32_t)f64_to_bf16(acc[2 * i + 1]) << 16);
        *reinterpret_cast<uint4 *>(out + t * H + 8 * c) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

int moe_max_experts() { return kMaxExperts; }

hipError_t launch_moe_route(const float *logits, int64_t T, int E, int k, int32_t *topk_expert, float *topk_weight,
                            int32_t *offsets, int32_t *row_ids, float *row_weights, int32_t *pair_rows,
                            hipStream_t stream) {
    if (T > 0) {
        const dim3 grid((unsigned)((T + 3) / 4));
#define QR_TOPK(EPL)                                                                                           \
    hipLaunchKernelGGL((route_topk_kernel<EPL>), grid, dim3(256), 0, stream, logits, T, E, k, topk_expert, \
                       topk_weight)
        if (E <= 64) {
            QR_TOPK(1);
        } else if (E <= 128) {
            QR_TOPK(2);
        } else if (E <= 256) {
            QR_TOPK(4);
        } else {
            QR_TOPK(8);
        }
#undef QR_TOPK
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // also for T = 0: the offsets (all zero) are still written
    hipLaunchKernelGGL(route_csr_kernel, dim3(1), dim3(kCsrThreads), 0, stream, topk_expert, topk_weight, T, E, k,
                       offsets, row_ids, row_weights, pair_rows);
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t *y_gu, int64_t rows, int64_t I, const float *s, int qtype,
                                 uint8_t *codes, float *scales, uint16_t *h_out, hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 3) / 4));
#define QR_SILU(QT, SS)                                                                                      \
    hipLaunchKernelGGL((silu_mul_quant_kernel<QT, SS>), grid, dim3(256), 0, stream, y_gu, rows, I, s, codes, scales, \
                       h_out)
    if (qtype == kInt8) {
        if (s != nullptr) QR_SILU(kInt8, true); else QR_SILU(kInt8, false);
    } else {
        if (s != nullptr) QR_SILU(kFp8, true); else QR_SILU(kFp8, false);
    }
#undef QR_SILU
    return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t *y_down, int64_t rows, const float *topk_weight,
                              const int32_t *pair_rows, int64_t T, int k, int64_t H, uint16_t *out,
                              hipStream_t stream) {
    const int64_t nch = H / 8;
    const int threads = nch >= 256 ? 256 : (int)((nch + 63) / 64) * 64;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)T), dim3(threads), 0, stream, y_down, rows, topk_weight,
                       pair_rows, k, H, out);
    return hipGetLastError();
}

}  // namespace qr
