// qr_linear.hip -- W8A8 linear (INT8 -> INT32, E4M3 -> FP32 on MFMA) with the dequantization epilogue.
//
// y[i,c] = acc[i,c] * x_scale[i] * w_scale[c], acc = sum_j xq[i,j] * wq[c,j]: the W8A8 product that quantized
// rollout runs at every decode step ("QuRL: Efficient Reinforcement Learning with Quantized Rollout",
// section 5; "QaRL: Rollout-Aligned Quantization-Aware RL ...", sections 2.2 and 3.1), with channel-wise
// weight scales and token-wise activation scales.
//
// Two kernels, chosen by the batch m:
//  * gemv_kernel (m <= 64): the decode regime, bound by streaming the n*k weight bytes from HBM. K-slice-major:
//    a block owns TB tiles of 16 output channels and all of K; wave w takes the 64U-byte K slices w, w + W, ...
//    For each slice it loads the activation slice once (coalesced, then moved into the MFMA layout with
//    ds_bpermute) and the slice of all TB weight tiles in one burst of 16-byte loads, then runs one MFMA per
//    (token tile, weight tile, 64-byte step). The waves' partial sums meet in LDS and are added in wave order
//    (deterministic, one launch, no cross-block synchronization); each wave finishes a share of the fragments
//    with the epilogue.
//  * m > 64: the LDS-ring MFMA GEMM of qr_gemm.hip.
#include "qr_device.hpp"
#include "qr_internal.hpp"

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

namespace qr {
namespace {

__device__ __forceinline__ void store_y(void *y, int64_t idx, float v, bool bf16) {
    if (bf16)
        static_cast<uint16_t *>(y)[idx] = f32_to_bf16(v);
    else
        static_cast<float *>(y)[idx] = v;
}

__device__ __forceinline__ void store_acc(void *acc_out, int64_t idx, int v) { static_cast<int *>(acc_out)[idx] = v; }
__device__ __forceinline__ void store_acc(void *acc_out, int64_t idx, float v) {
    static_cast<float *>(acc_out)[idx] = v;
}

__device__ __forceinline__ uint4 load16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ v4i as_v4i(const uint4 &a) { return v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w}; }
__device__ __forceinline__ v8i as_v8i(const uint4 &a, const uint4 &b) {
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// ---------------------------------------------------------------------------------------------------------
// Small-m GEMV
//
// A block owns TB tiles of 16 output channels (16 TB weight rows) and all of K. K is cut into slices of 64 U
// bytes; wave w takes slices w, w + W, ... For each slice it loads the activations once -- coalesced (lane l
// reads token row l >> 2, bytes 16 (l & 3) of each 64-byte block) and moved to the MFMA layout with ds_bpermute
// -- and keeps them in registers while the TB weight tiles stream past them, the next tile's loads in flight
// during the current tile's MFMAs. Activation traffic is therefore M K bytes per block rather than per tile.
//
// MFMA layout: lane (j, g) = (lane & 15, lane >> 4) supplies bytes [kb + 64 t + 16 g, +16) of weight row j of a
// tile (B operand, output channel j) and of token row j of a 16-token tile (A operand) for load t of a slice.
// INT8: one v_mfma_i32_16x16x64_i8 per load (K = 64 = the 4 lanes' 16 bytes). FP8: one
// v_mfma_scale_f32_16x16x128_f8f6f4 per pair of loads (32 bytes per lane). A and B use the same lane -> K map,
// so the dot products are those of the plain definition. Result C[i][c] sits in lane (c + 16 (i / 4)),
// element i % 4. Per-tile partials of all waves meet in LDS; every wave then sums a share of the 16x16
// fragments over the waves in wave order (deterministic) and applies the epilogue to them.
// ---------------------------------------------------------------------------------------------------------
// Activation input of the GEMV: codes and scales from the activation quantizer (kXCodes), or bfloat16 rows
// quantized inside the kernel (kXBf16, with X diag(1/s) for kXBf16S): in a prologue every block computes the
// per-token scales of its token rows and their codes, all lanes sharing the work, into LDS (after the
// reduction area), with the same IEEE steps as the activation quantizer (so the codes are the same bytes);
// the slice loop then reads its activation codes from LDS. For m <= kFuseRows only.
constexpr int kXCodes = 0, kXBf16 = 1, kXBf16S = 2;
constexpr int kFuseRows = 4;
constexpr int kPrefetchWaves = 8;  // most waves per block of the two-stage (prefetching) form

template <int QT, int MT, int U, int TB, int WMAX, int XM = kXCodes, bool PF = false, int KS = 1>
__global__ __launch_bounds__(WMAX * 64) void gemv_kernel(int64_t m, int64_t n, int64_t k, const uint8_t *__restrict__ xq,
                                                         const float *__restrict__ xs, const uint8_t *__restrict__ wq,
                                                         const float *__restrict__ ws, void *__restrict__ y,
                                                         int y_bf16, void *__restrict__ acc_out, int splits,
                                                         void *__restrict__ partial,
                                                         const uint16_t *__restrict__ xb = nullptr,
                                                         const float *__restrict__ xsv = nullptr) {
    typedef typename Acc<QT>::type acc_t;
    static_assert(QT == kInt8 || U % 2 == 0, "FP8 pairs load instructions");
    static_assert(XM == kXCodes || MT == 1, "in-kernel activation quantization for one token tile only");
    static_assert(KS == 1 || (MT == 1 && TB == 1 && !PF), "K parts inside the MFMA: one token tile, one weight tile");
    // KS > 1: K is cut into KS parts inside each MFMA. Lane row j of the weight operand is channel j / KS of a tile of
    // 16 / KS channels, over K part j % KS; row i of the activation operand is token i / KS over K part i % KS.
    // The products wanted are the blocks with equal parts, y[t][c] = sum_q C[t KS + q][c KS + q]: a tile covers
    // 16 / KS channels (KS times the workgroups on a few-channel linear) for at most 16 / KS tokens.
    constexpr int kCpt = 16 / KS;  // channels (and tokens) per tile
    const int64_t kq = k / KS;     // bytes of one K part (the host keeps k a multiple of 16 KS)
    extern __shared__ int32_t red[];  // [waves][TB][MT][4][64]
    const int waves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int64_t tile0 = (int64_t)blockIdx.x * TB;
    const int64_t m0 = (int64_t)blockIdx.y * (KS > 1 ? 16 / KS : 16 * MT);  // first token of this block
    constexpr int64_t kSlice = 64 * U;
    const int64_t slices = (kq + kSlice - 1) / kSlice;
    // split-K across blocks (blockIdx.z): this block's slices [lo, hi); with splits > 1 the raw sums go to
    // partial[split][m][n] and a separate reduction adds the splits in order and applies the epilogue
    const int64_t per_split = (slices + splits - 1) / splits;
    const int64_t lo = (int64_t)blockIdx.z * per_split;
    const int64_t hi = lo + per_split < slices ? lo + per_split : slices;

    // weight rows of this lane (rows past n re-read row n-1; those columns are never stored)
    const uint8_t *__restrict__ wrow[TB];
#pragma unroll
    for (int r = 0; r < TB; ++r) {
        const int64_t col = (tile0 + r) * kCpt + j / KS;
        wrow[r] = wq + (col < n ? col : n - 1) * k + (int64_t)(j % KS) * kq + 16 * g;
    }
    // coalesced activation loads: lane l reads token row (l >> 2) of each token tile, piece (l & 3)
    const int xr = lane >> 2, xp = lane & 3;
    const int xtok = xr / KS;                      // token of this lane's activation row (KS = 1: the row)
    const int64_t xkoff = (int64_t)(xr % KS) * kq;  // and its K part
    const int src_lane = 4 * j + g;  // the lane that loads what lane (j, g) needs
    // token rows past m re-read row m-1: they only feed output rows that are never stored
    const uint8_t *__restrict__ xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t r = m0 + mt * 16 + xtok;
        xrow[mt] = xq + (r < m ? r : m - 1) * k + xkoff + 16 * xp;
    }

    acc_t acc[TB][MT];
#pragma unroll
    for (int r = 0; r < TB; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[r][mt] = acc_t{0, 0, 0, 0};

    // in-kernel activation quantization: the scale of each token row (absmax of X diag(1/s) / qmax, IEEE
    // division, 1 when zero), then the codes of the token rows into LDS
    __shared__ float xq_scale[XM != kXCodes ? kFuseRows : 1];
    const int xrows = (int)(m - m0 < 16 ? m - m0 : 16);
    uint8_t *xlds = reinterpret_cast<uint8_t *>(red) + (size_t)waves * TB * MT * 1024;
    if constexpr (XM != kXCodes) {
        constexpr float qmax = QMax<QT>::value;
        auto x_elems = [&](int r, int64_t c, float *w) {  // 8 bfloat16 values of row r, chunk c, with 1/s applied
            const uint4 v = *reinterpret_cast<const uint4 *>(xb + (m0 + r) * k + 8 * c);
            const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[2 * i] = bf16_lo(p[i]);
                w[2 * i + 1] = bf16_hi(p[i]);
            }
            if constexpr (XM == kXBf16S) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float rs = 1.0f / xsv[8 * c + i];
                    w[i] = w[i] * rs;
                }
            }
        };
        __shared__ float xred[16][kFuseRows];
        float a[kFuseRows];
#pragma unroll
        for (int r = 0; r < kFuseRows; ++r) a[r] = 0.0f;
        for (int64_t c = threadIdx.x; c < k / 8; c += blockDim.x) {
#pragma unroll
            for (int r = 0; r < kFuseRows; ++r) {
                if (r < xrows) {
                    float w[8];
                    x_elems(r, c, w);
#pragma unroll
                    for (int i = 0; i < 8; ++i) a[r] = fmaxf(a[r], fabsf(w[i]));
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kFuseRows; ++r) {
            a[r] = wave_max(a[r]);
            if (lane == 0) xred[wave][r] = a[r];
        }
        __syncthreads();
        if (threadIdx.x < kFuseRows) {
            float amax = 0.0f;
            for (int w = 0; w < waves; ++w) amax = fmaxf(amax, xred[w][threadIdx.x]);
            float S = amax / qmax;  // IEEE division
            if (!(S > 0.0f)) S = 1.0f;
            xq_scale[threadIdx.x] = S;
        }
        __syncthreads();
        // the codes: 8 per thread and step, rows one after the other
        for (int r = 0; r < xrows; ++r) {
            const float S = xq_scale[r];
            const float R = 1.0f / S;
            const bool fast = S >= 0x1p-90f;
            for (int64_t c = threadIdx.x; c < k / 8; c += blockDim.x) {
                float w[8];
                x_elems(r, c, w);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float v = fast ? div_by_scale(w[i], S, R) : w[i] / S;
                    w[i] = fminf(fmaxf(v, -qmax), qmax);
                }
                *reinterpret_cast<uint2 *>(xlds + r * k + 8 * c) = make_uint2(encode_code4<QT>(w), encode_code4<QT>(w + 4));
            }
        }
        __syncthreads();
    }
    // 16 activation codes of this lane's token row at element j0 (global codes, or the block's LDS codes)
    auto x_codes16 = [&](const uint8_t *codes_at, int64_t j0) -> uint4 {
        if constexpr (XM == kXCodes) {
            return load16(codes_at);
        } else {
            const int row = xtok < xrows ? xtok : xrows - 1;
            return *reinterpret_cast<const uint4 *>(xlds + row * k + xkoff + j0);
        }
    };

    // Per slice, one burst: the slice's activations and all TB weight tiles are requested together, then the
    // activations are moved to the MFMA layout (in place) and the tiles' MFMAs run. Few registers per wave
    // keep many waves resident, and the resident waves hide each other's latency. Loads in full slices are
    // unconditional; in the partial last slice (k not a multiple of the slice) out-of-range bytes are zero.
    auto transpose = [&](uint4 (&xv)[MT][U]) {
#pragma unroll
        for (int t = 0; t < U; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                xv[mt][t].x = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)xv[mt][t].x);
                xv[mt][t].y = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)xv[mt][t].y);
                xv[mt][t].z = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)xv[mt][t].z);
                xv[mt][t].w = __builtin_amdgcn_ds_bpermute(src_lane * 4, (int)xv[mt][t].w);
            }
    };
    auto mma = [&](acc_t (&a)[MT], const uint4 (&xv)[MT][U], const uint4 (&wv)[U]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (QT == kInt8) {
#pragma unroll
                for (int t = 0; t < U; ++t)
                    a[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as_v4i(xv[mt][t]), as_v4i(wv[t]), a[mt], 0, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < U; t += 2)
                    // format 0 = E4M3 for both operands; scale exponents 127 = 2^0 (no block scaling)
                    a[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        as_v8i(xv[mt][t], xv[mt][t + 1]), as_v8i(wv[t], wv[t + 1]), a[mt], 0, 0, 0, 127, 0, 127);
            }
        }
    };
    const int64_t full = kq / kSlice;
    const int64_t full_hi = hi < full ? hi : full;
    auto load_slice = [&](int64_t sl, uint4 (&xv)[MT][U], uint4 (&wv)[TB][U]) {
        const int64_t kb = sl * kSlice;
#pragma unroll
        for (int t = 0; t < U; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xv[mt][t] = x_codes16(xrow[mt] + kb + 64 * t, kb + 64 * t + 16 * xp);
#pragma unroll
        for (int r = 0; r < TB; ++r)
#pragma unroll
            for (int t = 0; t < U; ++t) wv[r][t] = load16(wrow[r] + kb + 64 * t);
    };
    auto compute_slice = [&](uint4 (&xv)[MT][U], const uint4 (&wv)[TB][U]) {
        transpose(xv);
#pragma unroll
        for (int r = 0; r < TB; ++r) mma(acc[r], xv, wv[r]);
    };
    if constexpr (PF) {
        // two register stages: the next slice's loads are in flight while the current slice's MFMAs run, so a
        // wave with several slices waits for one memory round trip instead of one per slice (for blocks too
        // few to hide each other's latency: a short grid on a deep K)
        uint4 xa[MT][U], wa[TB][U], xb[MT][U], wb[TB][U];
        int64_t sl = lo + wave;
        if (sl < full_hi) load_slice(sl, xa, wa);
        while (sl < full_hi) {
            const int64_t s1 = sl + waves;
            if (s1 < full_hi) load_slice(s1, xb, wb);
            compute_slice(xa, wa);
            if (s1 >= full_hi) break;
            const int64_t s2 = s1 + waves;
            if (s2 < full_hi) load_slice(s2, xa, wa);
            compute_slice(xb, wb);
            sl = s2;
        }
    } else {
        for (int64_t sl = lo + wave; sl < full_hi; sl += waves) {
            uint4 xv[MT][U], wv[TB][U];
            load_slice(sl, xv, wv);
            compute_slice(xv, wv);
        }
    }
    if (full < slices && full >= lo && full < hi && wave == (full - lo) % waves) {  // the partial last slice
        const int64_t kb = full * kSlice;
        uint4 xv[MT][U], wv[TB][U];
#pragma unroll
        for (int t = 0; t < U; ++t) {
            const bool in = kb + 64 * t + 16 * xp < kq;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xv[mt][t] = in ? x_codes16(xrow[mt] + kb + 64 * t, kb + 64 * t + 16 * xp) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < TB; ++r)
#pragma unroll
            for (int t = 0; t < U; ++t) {
                const bool in = kb + 64 * t + 16 * g < kq;
                wv[r][t] = in ? load16(wrow[r] + kb + 64 * t) : make_uint4(0, 0, 0, 0);
            }
        transpose(xv);
#pragma unroll
        for (int r = 0; r < TB; ++r) mma(acc[r], xv, wv[r]);
    }

    // every wave publishes its partials; each wave then reduces a share of the fragments in wave order
    constexpr int kFrags = TB * MT;
    if (waves > 1) {
        int32_t *mine = red + (int64_t)wave * (kFrags * 256);
#pragma unroll
        for (int r = 0; r < TB; ++r)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int idx = (r * MT + mt) * 256 + i * 64 + lane;
                    if constexpr (QT == kInt8)
                        mine[idx] = acc[r][mt][i];
                    else
                        mine[idx] = __float_as_int(acc[r][mt][i]);
                }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < TB; ++r)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int f = r * MT + mt;
            if (waves > 1) {
                if (f % waves != wave) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int idx = f * 256 + i * 64 + lane;
                    if constexpr (QT == kInt8) {
                        int32_t sum = red[idx];
                        for (int w = 1; w < waves; ++w) sum += red[(int64_t)w * (kFrags * 256) + idx];
                        acc[r][mt][i] = sum;
                    } else {
                        float sum = __int_as_float(red[idx]);
                        for (int w = 1; w < waves; ++w) sum += __int_as_float(red[(int64_t)w * (kFrags * 256) + idx]);
                        acc[r][mt][i] = sum;
                    }
                }
            }
            if constexpr (KS > 1) {
                // the complete 16 x 16 fragment goes through this wave's own LDS area (after the reduction has
                // read it), then lane t kCpt + c adds the equal-part blocks C[t KS + q][c KS + q] over q in order
                // and applies the epilogue to token t, channel c of the tile
                int32_t *frag = red + (int64_t)wave * (kFrags * 256);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int idx = (4 * g + i) * 16 + j;  // C[4 g + i][j]
                    if constexpr (QT == kInt8)
                        frag[idx] = acc[r][mt][i];
                    else
                        frag[idx] = __float_as_int(acc[r][mt][i]);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's stores land before its reads
                const int tt = lane / kCpt, c = lane % kCpt;
                const int64_t row = m0 + tt, col = tile0 * kCpt + c;
                if (lane < kCpt * kCpt && row < m && col < n) {
                    typename std::remove_reference<decltype(acc[0][0][0])>::type a = 0;
                    for (int q = 0; q < KS; ++q) {
                        const int32_t v = frag[(tt * KS + q) * 16 + c * KS + q];
                        if constexpr (QT == kInt8)
                            a += v;
                        else
                            a += __int_as_float(v);
                    }
                    float sxv;
                    if constexpr (XM == kXCodes)
                        sxv = xs[row];
                    else
                        sxv = xq_scale[row - m0];
                    const float v = acc_to_f32(a) * sxv * ws[col];
                    store_y(y, row * n + col, v, y_bf16 != 0);
                    if (acc_out != nullptr) store_acc(acc_out, row * n + col, a);
                }
                continue;
            }
            const int64_t col = (tile0 + r) * 16 + j;
            if (splits > 1) {
                // raw sums of this split; the reduction applies the epilogue
                if (col >= n) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t row = m0 + mt * 16 + 4 * g + i;
                    if (row < m) store_acc(partial, ((int64_t)blockIdx.z * m + row) * n + col, acc[r][mt][i]);
                }
                continue;
            }
            // epilogue: y = acc * x_scale[row] * w_scale[col]; the scales are loaded together from clamped
            // indices (one round trip), then the stores are predicated
            const float sw = ws[col < n ? col : n - 1];
            float sx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + mt * 16 + 4 * g + i;
                if constexpr (XM == kXCodes)
                    sx[i] = xs[row < m ? row : m - 1];
                else
                    sx[i] = xq_scale[row < m ? row - m0 : xrows - 1];
            }
            if (col >= n) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + mt * 16 + 4 * g + i;
                if (row < m) {
                    const float v = acc_to_f32(acc[r][mt][i]) * sx[i] * sw;
                    store_y(y, row * n + col, v, y_bf16 != 0);
                    if (acc_out != nullptr) store_acc(acc_out, row * n + col, acc[r][mt][i]);
                }
            }
        }
}

template <int QT, int MT, int U, int TB, int WMAX>
void launch_gemv_t(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                   const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                   hipStream_t stream) {
    const int64_t m_blocks = (m + 16 * MT - 1) / (16 * MT);
    const dim3 grid((unsigned)((p.n_tiles + TB - 1) / TB), (unsigned)m_blocks, (unsigned)p.splits);
    const size_t lds = p.waves > 1 ? (size_t)p.waves * TB * MT * 256 * 4 : 0;
    // the two-stage form holds twice the registers: at most 8 waves per block (256 VGPRs each, no spills)
    constexpr int kPfWaves = WMAX < kPrefetchWaves ? WMAX : kPrefetchWaves;
    if (p.prefetch)
        hipLaunchKernelGGL((gemv_kernel<QT, MT, U, TB, kPfWaves, kXCodes, true>), grid, dim3(p.waves * 64), lds, stream,
                           m, n, k, xq, xs, wq, ws, y, y_bf16 ? 1 : 0, acc_out, p.splits, workspace);
    else
        hipLaunchKernelGGL((gemv_kernel<QT, MT, U, TB, WMAX>), grid, dim3(p.waves * 64), lds, stream, m, n, k, xq, xs,
                           wq, ws, y, y_bf16 ? 1 : 0, acc_out, p.splits, workspace);
    if (p.splits > 1) launch_splitk_reduce(QT, m, n, p.splits, workspace, xs, ws, y, y_bf16, acc_out, stream);
}

// (m_tiles, unroll, tiles per block, most waves per block); the planner further limits the waves so that the
// reduction's LDS, waves x TB x MT KiB, stays within 64 KiB.
#define QR_GEMV_VARIANTS(X) \
    X(1, 4, 1, 16) X(1, 4, 2, 16) X(1, 4, 4, 16) X(1, 8, 1, 16) X(1, 8, 2, 16) \
    X(2, 4, 1, 16) X(2, 4, 2, 16) X(2, 8, 1, 16) \
    X(4, 2, 1, 16) X(4, 2, 2, 16) X(4, 4, 1, 8)

// most waves per block of a variant, 0 if it does not exist
int gemv_variant_waves(int mt, int u, int tb) {
#define QR_GEMV_HAS(MT_, U_, TB_, W_) if (mt == MT_ && u == U_ && tb == TB_) return W_;
    QR_GEMV_VARIANTS(QR_GEMV_HAS)
#undef QR_GEMV_HAS
    return 0;
}

// the GEMV with K cut into S parts inside the MFMA (token blocks of 16 / S tokens, one weight tile of 16 / S
// channels per workgroup, no K split across workgroups)
template <int QT, int U, int S, int XM>
void launch_gemv_ksub_t(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                        const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, size_t lds,
                        const uint16_t *xb, const float *s, hipStream_t stream) {
    const dim3 grid((unsigned)p.n_tiles, (unsigned)((m + 16 / S - 1) / (16 / S)), 1u);
    hipLaunchKernelGGL((gemv_kernel<QT, 1, U, 1, 16, XM, false, S>), grid, dim3(p.waves * 64), lds, stream, m, n, k, xq,
                       xs, wq, ws, y, y_bf16 ? 1 : 0, acc_out, 1, nullptr, xb, s);
}

template <int QT, int XM>
bool launch_gemv_ksub(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                      const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, size_t lds,
                      const uint16_t *xb, const float *s, hipStream_t stream) {
#define QR_KSUB(U_, S_)                                                                                          \
    if (p.unroll == U_ && p.ksub == S_) {                                                                        \
        launch_gemv_ksub_t<QT, U_, S_, XM>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, lds, xb, s, stream); \
        return true;                                                                                             \
    }
    QR_KSUB(4, 2) QR_KSUB(4, 4) QR_KSUB(4, 8)
    if constexpr (XM == kXCodes) {
        QR_KSUB(8, 2) QR_KSUB(8, 4) QR_KSUB(8, 8)
    }
#undef QR_KSUB
    return false;
}

// false when the plan names no compiled variant (plan_linear only produces compiled ones; a caller that gets
// false reports hipErrorInvalidConfiguration instead of launching anything)
template <int QT>
bool launch_gemv_q(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                   const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                   hipStream_t stream) {
    if (p.ksub > 1)
        return launch_gemv_ksub<QT, kXCodes>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, (size_t)p.waves * 1024,
                                             nullptr, nullptr, stream);
#define QR_GEMV_CASE(MT_, U_, TB_, W_)                                                                          \
    if (p.m_tiles == MT_ && p.unroll == U_ && p.tiles == TB_) {                                                 \
        launch_gemv_t<QT, MT_, U_, TB_, W_>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream); \
        return true;                                                                                            \
    }
    QR_GEMV_VARIANTS(QR_GEMV_CASE)
#undef QR_GEMV_CASE
    return false;
}

// dynamic LDS of the GEMV with in-kernel activation quantization: the reduction area (always reserved: the codes
// sit after it) and the token rows' codes
size_t gemv_fused_lds_bytes(const LinearPlan &p, int64_t m, int64_t k) {
    return (size_t)p.waves * p.tiles * 1024 + (size_t)((m * k + 15) / 16 * 16);
}

// the GEMV with in-kernel activation quantization (bfloat16 x, optional X diag(1/s)); one token tile only
template <int QT, int U, int TB, int WMAX>
void launch_gemv_fused_t(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint16_t *xb, const float *s,
                         const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                         hipStream_t stream) {
    const dim3 grid((unsigned)((p.n_tiles + TB - 1) / TB), 1u, 1u);
    const size_t lds = gemv_fused_lds_bytes(p, m, k);
    if (s != nullptr)
        hipLaunchKernelGGL((gemv_kernel<QT, 1, U, TB, WMAX, kXBf16S>), grid, dim3(p.waves * 64), lds, stream, m, n, k,
                           nullptr, nullptr, wq, ws, y, y_bf16 ? 1 : 0, acc_out, 1, nullptr, xb, s);
    else
        hipLaunchKernelGGL((gemv_kernel<QT, 1, U, TB, WMAX, kXBf16>), grid, dim3(p.waves * 64), lds, stream, m, n, k,
                           nullptr, nullptr, wq, ws, y, y_bf16 ? 1 : 0, acc_out, 1, nullptr, xb, s);
}

template <int QT>
bool launch_gemv_fused_q(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint16_t *xb, const float *s,
                         const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                         hipStream_t stream) {
    if (p.ksub > 1) {
        const size_t lds = gemv_fused_lds_bytes(p, m, k);
        return s != nullptr ? launch_gemv_ksub<QT, kXBf16S>(p, m, n, k, nullptr, nullptr, wq, ws, y, y_bf16, acc_out,
                                                            lds, xb, s, stream)
                            : launch_gemv_ksub<QT, kXBf16>(p, m, n, k, nullptr, nullptr, wq, ws, y, y_bf16, acc_out,
                                                           lds, xb, s, stream);
    }
#define QR_GEMV_FUSED_CASE(MT_, U_, TB_, W_)                                                                    \
    if constexpr (MT_ == 1 && U_ == 4) {                                                                        \
        if (p.m_tiles == MT_ && p.unroll == U_ && p.tiles == TB_) {                                             \
            launch_gemv_fused_t<QT, U_, TB_, W_>(p, m, n, k, xb, s, wq, ws, y, y_bf16, acc_out, stream);        \
            return true;                                                                                        \
        }                                                                                                       \
    }
    QR_GEMV_VARIANTS(QR_GEMV_FUSED_CASE)
#undef QR_GEMV_FUSED_CASE
    return false;
}

}  // namespace

// Tuning overrides (forced kernel variants, split counts, tile sizes) and the plan trace are read from the
// environment only when QR_TUNE is set (non-empty, not "0") in the environment at the time the library is
// loaded; otherwise every plan is the automatic one and no variable is read, so a stray variable can change
// neither the kernels chosen nor the FP8 summation order.
static bool read_tune_switch() {
    const char *v = getenv("QR_TUNE");
    return v != nullptr && *v != '\0' && !(v[0] == '0' && v[1] == '\0');
}
static const bool g_tune = read_tune_switch();

bool tune_enabled() { return g_tune; }

int env_int(const char *name, int dflt) {
    if (!g_tune) return dflt;
    const char *v = getenv(name);
    if (v == nullptr || *v == '\0') return dflt;
    return atoi(v);
}

bool trace_enabled() { return g_tune && getenv("QR_TRACE") != nullptr; }

LinearPlan plan_linear(int qtype, int64_t m, int64_t n, int64_t k, int max_unroll, bool fused_quant) {
    (void)qtype;
    LinearPlan p{};
    const int force = env_int("QR_FORCE_VARIANT", -1);  // 0 = GEMV, 1 = tiled GEMM
    const bool gemv = force == 0 || (force != 1 && m <= 64);
    p.ws_bytes = 0;
    if (!gemv) {
        p.kind = 1;
        p.gemm = gemm_plan(m, n, k);
        p.ws_bytes = p.gemm.ws_bytes;
        return p;
    }
    p.kind = 0;
    p.m_tiles = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    p.n_tiles = (n + 15) / 16;
    // token tiles per workgroup: QR_GEMV_MT forces 1, 2 or 4 (fewer tiles: more token blocks, each reading the
    // weights). Two instead of four pay for 32 < m <= 64 on few tiles with a short K (measured on MI355X: 1.5B
    // qkv at m = 64 6.4 -> 5.6 us, o 6.4 -> 5.4; the gate/up is slower, the down unchanged)
    const int fmt = env_int("QR_GEMV_MT", 0);
    const bool gemv_overrides = env_int("QR_GEMV_UNROLL", 0) > 0 || env_int("QR_GEMV_TILES", 0) > 0 ||
                                env_int("QR_GEMV_WAVES", 0) > 0 || env_int("QR_GEMV_SPLITS", 0) > 0;
    if (fmt == 1 || fmt == 2 || fmt == 4)
        p.m_tiles = fmt;
    else if (fmt == 0 && !gemv_overrides && p.m_tiles == 4 && p.n_tiles < 160 && k <= 2048)
        p.m_tiles = 2;
    const int64_t m_blocks = (m + 16 * p.m_tiles - 1) / (16 * p.m_tiles);
    // slices of 256 bytes (128 for four token tiles) unless overridden
    int u = p.m_tiles == 4 ? 2 : 4;
    int tb = 1;
    int wave_cap = 0;  // 0 = the variant's maximum
    if (p.m_tiles == 1) {
        // one token tile (m <= 16): the activation slice is small, so each block takes one weight tile and
        // few wavefronts, 512-byte slices when K has at least three of them. Many small blocks keep more of
        // them resident per CU and shorten the last, partly filled round of blocks (measured on MI355X: 7B
        // gate/up at m = 1 from 31 to 26 us per call); only when there are few tiles (a short, deep K) do
        // more wavefronts per block, on 256-byte slices, pay.
        const bool few = p.n_tiles < 128;
        if (k >= 1536 && !few) u = 8;
        wave_cap = few ? 8 : 4;
        // past half a token tile, on many tiles, one wavefront streams all of K for its block: no partial sums
        // through LDS, and the most blocks resident per CU; on very many tiles two weight tiles per block also
        // share each activation slice (measured on MI355X, 7B gate/up, 2368 tiles, at m = 16: 34.4 us with one
        // tile on four wavefronts, 31.7 with two tiles, 29.0 with two tiles on one wavefront, 29.0-31.5 with one
        // tile on one wavefront; the 1.5B gate/up, 1120 tiles, at m = 16 with one tile on one wavefront: INT8
        // 9.2 -> 8.6 us, FP8 10.0 -> 8.4, at m = 9 INT8 8.5 -> 8.2; two tiles are slower there)
        if (m > 8 && p.n_tiles >= 2048 && gemv_variant_waves(1, u, 2) > 0) {
            tb = 2;
            wave_cap = 1;
        } else if (m > 8 && p.n_tiles >= 1024) {
            wave_cap = 1;
        }
    } else {
        // more tiles per block share each activation load (at m = 64 the activation slices a block reads
        // outweigh its weights); keep at least ~1000 blocks in flight
        const int64_t min_blocks = env_int("QR_GEMV_MIN_BLOCKS", 1024);
        for (int cand : {4, 2}) {
            if (gemv_variant_waves(p.m_tiles, u, cand) == 0) continue;
            if (((p.n_tiles + cand - 1) / cand) * m_blocks >= min_blocks) {
                tb = cand;
                break;
            }
        }
        if (p.m_tiles == 4) {
            // four token tiles (32 < m <= 64): with enough blocks, one wave each (no reduction, the most blocks
            // resident); with few, 256-byte slices over up to 8 waves (measured on MI355X: 1.5B gate/up at
            // m = 64 from 25 to 16 us, the few-tile 1.5B / 7B linears 5-15% faster)
            if (((p.n_tiles + tb - 1) / tb) * m_blocks >= 1024)
                wave_cap = 1;
            else if (tb == 1)
                u = 4;
        }
    }
    const int fu = env_int("QR_GEMV_UNROLL", 0), ft = env_int("QR_GEMV_TILES", 0);
    if ((fu > 0 || ft > 0) && gemv_variant_waves(p.m_tiles, fu > 0 ? fu : u, ft > 0 ? ft : tb) > 0) {
        u = fu > 0 ? fu : u;
        tb = ft > 0 ? ft : tb;
    }
    if (u > max_unroll && gemv_variant_waves(p.m_tiles, max_unroll, tb) > 0) u = max_unroll;
    // K cut into S parts inside the MFMA for one token tile of m <= 16 / S tokens: tiles of 16 / S channels, S
    // times the workgroups. A linear with fewer 16-channel tiles than about two per CU cannot stream at full rate
    // (one CU streams at most ~25 GB/s), and at m = 1 the MFMA's token rows are free to carry K parts instead.
    // Chosen at m = 1 from measurements on MI355X (graph replay, weights past the caches):
    //  - codes in: 8 parts below 512 tiles with k <= 8960 (1.5B down 8.8 -> 5.8 us, o 4.3 -> 3.4, 7B qkv
    //    7.6 -> 5.8, o 6.0 -> 5.2), 2 or 4 on many tiles (1.5B gate/up 8.2 -> 7.9 with k < 2048, 7B gate/up
    //    26.8 -> 24.5); one wavefront per workgroup with 8 parts on 128..511 tiles (below);
    //  - activation quantization inside the kernel (every workgroup repeats it): 2 parts below 256 tiles (1.5B
    //    qkv 6.4 -> 5.6 us, o 6.3 -> 5.5, down 11.4 -> 9.3; 7B o 9.2 -> 8.2), none otherwise.
    // QR_GEMV_KSUB forces S; other GEMV overrides turn the automatic choice off.
    p.ksub = 1;
    if (p.m_tiles == 1) {
        const int fk = env_int("QR_GEMV_KSUB", 0);
        const bool overrides = fu > 0 || ft > 0 || env_int("QR_GEMV_WAVES", 0) > 0 || env_int("QR_GEMV_SPLITS", 0) > 0;
        int ks = 1;
        bool blocks_ok = env_int("QR_GEMV_KSUB_BLOCKS", 0) > 0;  // several token blocks of 16 / S tokens
        if (fk == 2 || fk == 4 || fk == 8) {
            ks = fk;
        } else if (fk == 0 && !overrides && m == 1) {
            if (fused_quant) {
                ks = p.n_tiles < 256 ? 2 : 1;
            } else if (p.n_tiles >= 128 && p.n_tiles < 512) {
                // 8 parts with one wavefront per workgroup on 256-byte slices (measured on MI355X, the same box:
                // 7B down, k = 18944, 16.1 -> 14.7 us, qkv 6.07 -> 5.87, o 5.7 -> 5.44, the layer at m = 1 with
                // a2 65.6 -> 64.6 us; 1.5B qkv 4.0 -> 3.7; the fewest-tile 1.5B down is slower this way, and the
                // 7B gate/up with 8 parts on one wavefront was not faster on every box)
                ks = 8;
                u = 4;
                wave_cap = 1;
            } else if (k <= 8960) {
                ks = p.n_tiles < 512 ? 8 : (k >= 2048 ? 4 : 2);
            }
        } else if (fk == 0 && !overrides && !fused_quant && m > 8 && p.n_tiles < 160 && k <= 8960) {
            // two token blocks of 8 tokens, K in 2 parts: the weights are read twice (the second time mostly
            // from cache), which pays only on the fewest tiles (1.5B o at m = 16: 4.8 -> 4.1 us, down 10.2 ->
            // 9.7, qkv 4.4 -> 4.3; the 7B o and any many-tile linear are slower)
            ks = 2;
            blocks_ok = true;
        }
        while (ks > 1 && k % (16 * ks) != 0) ks /= 2;
        if (ks > 1 && (u == 4 || u == 8) && (m <= 16 / ks || blocks_ok)) {
            p.ksub = ks;
            tb = 1;
            p.n_tiles = (n + 16 / ks - 1) / (16 / ks);
        }
    }
    p.unroll = u;
    p.tiles = tb;
    const int64_t kpart = k / p.ksub;
    const int64_t slices = (kpart + 64 * u - 1) / (64 * u);
    // the reduction's LDS (waves x tb x m_tiles KiB) stays within 64 KiB
    int cap = gemv_variant_waves(p.m_tiles, u, tb);
    if (cap > 64 / (tb * p.m_tiles)) cap = 64 / (tb * p.m_tiles);
    if (wave_cap > 0 && cap > wave_cap && env_int("QR_GEMV_WAVES", 0) == 0) cap = wave_cap;
    // split K across blocks when four token tiles make each block long, the blocks would leave most CUs idle
    // and K is deep: two splits; the partial sums (splits x m x n x 4 bytes) go to the workspace and a separate
    // reduction adds them in split order. The reduction's launch costs more than it saves at m <= 32
    // (measured on MI355X: 1.5B down at m = 64 from 19.3 to 14.8 us; at m = 1 and 16 8.7 -> 9.6, 10.2 -> 10.5)
    const int64_t blocks = ((p.n_tiles + tb - 1) / tb) * m_blocks;
    int64_t splits = 1;
    const int64_t waves_cap = cap;
    if (p.m_tiles == 4 && blocks < 128 && slices >= 16) splits = 2;
    const int fs = env_int("QR_GEMV_SPLITS", 0);
    if (fs >= 1) splits = std::min<int64_t>(fs, slices);
    if (p.ksub > 1) splits = 1;
    const int64_t per_split = (slices + splits - 1) / splits;
    splits = (slices + per_split - 1) / per_split;  // no split without a slice
    int64_t waves = per_split < waves_cap ? per_split : waves_cap;
    const int forced_w = env_int("QR_GEMV_WAVES", 0);
    if (forced_w >= 1 && forced_w <= cap) waves = forced_w;
    p.waves = (int)(waves < 1 ? 1 : waves);
    p.splits = (int)splits;
    // two register stages for four token tiles on few blocks (32 < m <= 64, fewer than 1024 blocks): measured on
    // MI355X, 1.5B qkv / o at m = 64 from 7.2 to 6.4 us, down (two K splits) from 16.0 to 13.9 us; neutral or
    // slower at m <= 16 and on many-block plans, where other resident waves already hide the latency
    const int fpf = env_int("QR_GEMV_PREFETCH", -1);
    p.prefetch = fpf >= 0 ? fpf > 0 : (p.m_tiles == 4 && blocks < 1024);
    if (p.prefetch && p.waves > kPrefetchWaves) p.waves = kPrefetchWaves;
    p.ws_bytes = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * 4 : 0;
    return p;
}

LinearPlan plan_linear_bf16(int qtype, int64_t m, int64_t n, int64_t k) {
    // the in-kernel activation quantization holds a slice's activations as floats: at most 256-byte slices
    const LinearPlan p = plan_linear(qtype, m, n, k, 4, true);
    if (linear_bf16_fused(p, qtype, m, k)) return p;
    return plan_linear(qtype, m, n, k);
}

bool linear_bf16_fused(const LinearPlan &p, int qtype, int64_t m, int64_t k) {
    // Every workgroup quantizes the token rows itself, so the prologue is repeated per workgroup and only its
    // own latency is hidden by other workgroups. Measured on MI355X (graph replay, weights past the caches,
    // against the activation quantizer, about 3.6 us, followed by the linear on codes): at m = 1 it pays on at
    // most 256 workgroups (1.5B qkv, 256: 6.3 -> 5.8 us, o, 192: 6.1 -> 5.7), not on the 7B qkv (288: 8.4 against
    // 9.4 us) and o (448: 7.9 against 8.0), nor on the many of the 7B gate/up (2368), nor on the 7B down
    // (k = 18944, a long row in every workgroup), nor at m = 2 or 4.
    const int64_t max_m = env_int("QR_FUSE_MAX_M", 1);
    if (qtype == kFp8 && k > env_int("QR_FUSE_MAX_K_FP8", 8192)) return false;
    if (p.kind != 0 || p.m_tiles != 1 || p.splits != 1 || p.unroll != 4 || p.tiles < 1) return false;  // GEMV only
    const int64_t blocks = (p.n_tiles + p.tiles - 1) / p.tiles;
    return blocks <= env_int("QR_FUSE_MAX_BLOCKS", 256) && m <= std::min<int64_t>(max_m, kFuseRows) &&
           gemv_fused_lds_bytes(p, m, k) <= 65536;
}

size_t linear_bf16_workspace_bytes(const LinearPlan &p, int qtype, int64_t m, int64_t k) {
    if (linear_bf16_fused(p, qtype, m, k)) return 0;
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    return up((size_t)(m * k)) + up((size_t)m * 4) + p.ws_bytes;
}

hipError_t launch_linear_bf16(const LinearPlan &p, int qtype, int64_t m, int64_t n, int64_t k, const uint16_t *xb,
                              const float *s, const uint8_t *wq, const float *ws, void *y, bool y_bf16,
                              void *acc_out, void *workspace, hipStream_t stream) {
    if (linear_bf16_fused(p, qtype, m, k)) {
        const bool ok = qtype == kInt8 ? launch_gemv_fused_q<kInt8>(p, m, n, k, xb, s, wq, ws, y, y_bf16, acc_out, stream)
                                       : launch_gemv_fused_q<kFp8>(p, m, n, k, xb, s, wq, ws, y, y_bf16, acc_out, stream);
        if (!ok) return hipErrorInvalidConfiguration;
        return hipGetLastError();
    }
    // the activation quantizer into the workspace, then the linear on its codes
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    uint8_t *wsb = static_cast<uint8_t *>(workspace);
    uint8_t *xq = wsb;
    float *xs = reinterpret_cast<float *>(wsb + up((size_t)(m * k)));
    void *rest = wsb + up((size_t)(m * k)) + up((size_t)m * 4);
    hipError_t e = launch_quantize_rows(xb, true, m, k, s, s == nullptr ? kSNone : kSMulRecip, qtype, xq, xs, stream);
    if (e != hipSuccess) return e;
    return launch_linear(p, qtype, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, rest, stream);
}

hipError_t launch_linear(const LinearPlan &p, int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *xq,
                         const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                         void *workspace, hipStream_t stream) {
    if (p.kind == 0) {
        const bool ok = qtype == kInt8
                            ? launch_gemv_q<kInt8>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream)
                            : launch_gemv_q<kFp8>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
        if (!ok) return hipErrorInvalidConfiguration;
    } else {
        return launch_gemm(p.gemm, qtype, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
    }
    return hipGetLastError();
}

}  // namespace qr
