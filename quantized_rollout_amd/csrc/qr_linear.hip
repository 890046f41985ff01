// qr_linear.hip -- W8A8 linear (INT8 -> INT32, E4M3 -> FP32 on MFMA) with the dequantization epilogue.
//
// y[i,c] = acc[i,c] * x_scale[i] * w_scale[c], acc = sum_j xq[i,j] * wq[c,j]: the W8A8 product that quantized
// rollout runs at every decode step ("QuRL: Efficient Reinforcement Learning with Quantized Rollout",
// section 5; "QaRL: Rollout-Aligned Quantization-Aware RL ...", sections 2.2 and 3.1), with channel-wise
// weight scales and token-wise activation scales.
//
// Two kernels, chosen by the batch m:
//  * gemv_kernel (m <= 64): the decode regime, bound by streaming the n*k weight bytes from HBM. A wave owns
//    16 output channels and walks K in 256-byte steps, each lane loading 64 contiguous bytes of one weight row
//    (16 rows x 256 B per wave and step) plus the matching activation bytes, and issues MFMA 16x16 tiles over
//    up to four 16-token tiles. The waves of a block split the block's K range (reduced through LDS in a fixed
//    order); when the n tiles alone cannot fill 256 CUs, blocks also split K and the last block to finish a
//    tile sums the partials in split order and applies the epilogue (deterministic, one launch).
//  * gemm_kernel (m > 64): LDS-tiled MFMA GEMM, 128x128 output tiles, 128-byte K steps, double-buffered LDS.
#include "qr_device.hpp"
#include "qr_internal.hpp"

#include <stdlib.h>

namespace qr {
namespace {

constexpr int kStep = 256;  // K bytes per wave step in the GEMV

// Workspace layout of a split-K GEMV: [kMaxCounters uint32 arrival counters | partial tiles]. The counter
// region has the same place and size for every plan, and the last block of each tile resets its counter, so
// the region stays zero between calls whatever shapes ran before; the partials are scratch.
constexpr int64_t kMaxCounters = 65536;
constexpr size_t kCounterBytes = kMaxCounters * 4;

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

// Loads the 64 K bytes lane (j, g) contributes to one 256-byte step of row `row_ptr` (NULL = zero row).
__device__ __forceinline__ void load_step(uint4 *dst, const uint8_t *__restrict__ row_ptr, int64_t kb, int64_t k) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t off = kb + 16 * t;
        if (row_ptr != nullptr && off < k)
            dst[t] = *reinterpret_cast<const uint4 *>(row_ptr + off);
        else
            dst[t] = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------------------------------------
// Small-m GEMV with split-K
// ---------------------------------------------------------------------------------------------------------
template <int QT, int MT, int WPB>
__global__ __launch_bounds__(WPB * 64) void gemv_kernel(int64_t m, int64_t n, int64_t k,
                                                        const uint8_t *__restrict__ xq,
                                                        const float *__restrict__ xs,
                                                        const uint8_t *__restrict__ wq,
                                                        const float *__restrict__ ws, void *__restrict__ y,
                                                        int y_bf16, void *__restrict__ acc_out, int splits,
                                                        int64_t n_tiles, int32_t *__restrict__ partials,
                                                        uint32_t *__restrict__ counters) {
    typedef typename Acc<QT>::type acc_t;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int64_t tile = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t m0 = (int64_t)blockIdx.z * (16 * MT);

    const int64_t steps = (k + kStep - 1) / kStep;
    const int64_t per = (steps + splits - 1) / splits;
    const int64_t s_beg = (int64_t)split * per;
    const int64_t s_end = s_beg + per < steps ? s_beg + per : steps;

    const int64_t ncol = tile * 16 + j;
    const uint8_t *__restrict__ wrow = ncol < n ? wq + ncol * k : nullptr;
    const uint8_t *__restrict__ xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t r = m0 + mt * 16 + j;
        xrow[mt] = r < m ? xq + r * k : nullptr;
    }

    acc_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = acc_t{0, 0, 0, 0};

    int64_t st = s_beg + wave;
    if (st < s_end) {
        uint4 wcur[4], xcur[MT][4];
        load_step(wcur, wrow, st * kStep + g * 64, k);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load_step(xcur[mt], xrow[mt], st * kStep + g * 64, k);
        for (;;) {
            const int64_t nx = st + WPB;
            uint4 wnxt[4], xnxt[MT][4];
            if (nx < s_end) {
                load_step(wnxt, wrow, nx * kStep + g * 64, k);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) load_step(xnxt[mt], xrow[mt], nx * kStep + g * 64, k);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma_step(acc[mt], xcur[mt], wcur);
            if (nx >= s_end) break;
            st = nx;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                wcur[t] = wnxt[t];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xcur[mt][t] = xnxt[mt][t];
            }
        }
    }

    // intra-block reduction over the waves, in wave order
    if constexpr (WPB > 1) {
        __shared__ int32_t red[WPB - 1][MT][4][64];
        if (wave > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (QT == kInt8)
                        red[wave - 1][mt][r][lane] = acc[mt][r];
                    else
                        red[wave - 1][mt][r][lane] = __float_as_int(acc[mt][r]);
                }
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < WPB - 1; ++w)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (QT == kInt8)
                        acc[mt][r] += red[w][mt][r][lane];
                    else
                        acc[mt][r] += __int_as_float(red[w][mt][r][lane]);
                }
    }

    // inter-block split of K: publish the partial, the last block of the tile reduces in split order
    if (splits > 1) {
        const int64_t slot = (int64_t)blockIdx.z * n_tiles + tile;
        int32_t *__restrict__ mine = partials + (slot * splits + split) * (MT * 256);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (QT == kInt8)
                    mine[mt * 256 + r * 64 + lane] = acc[mt][r];
                else
                    mine[mt * 256 + r * 64 + lane] = __float_as_int(acc[mt][r]);
            }
        __threadfence();  // release the partial to the whole device (all XCDs)
        uint32_t old = 0;
        if (lane == 0) old = atomicAdd(counters + slot, 1u);
        old = __shfl(old, 0, 64);
        if (old != (uint32_t)(splits - 1)) return;
        __threadfence();  // acquire the other blocks' partials
        const int32_t *__restrict__ all = partials + slot * splits * (MT * 256);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int idx = mt * 256 + r * 64 + lane;
                if constexpr (QT == kInt8) {
                    int32_t sum = all[idx];
                    for (int s2 = 1; s2 < splits; ++s2) sum += all[s2 * (MT * 256) + idx];
                    acc[mt][r] = sum;
                } else {
                    float sum = __int_as_float(all[idx]);
                    for (int s2 = 1; s2 < splits; ++s2) sum += __int_as_float(all[s2 * (MT * 256) + idx]);
                    acc[mt][r] = sum;
                }
            }
        if (lane == 0) counters[slot] = 0u;  // leave the workspace zeroed for the next call
    }

    // epilogue: y = acc * x_scale[row] * w_scale[col]
    if (ncol < n) {
        const float sw = ws[ncol];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + mt * 16 + 4 * g + r;
                if (row < m) {
                    const float v = acc_to_f32(acc[mt][r]) * xs[row] * sw;
                    store_y(y, row * n + ncol, v, y_bf16 != 0);
                    if (acc_out != nullptr) store_acc(acc_out, row * n + ncol, acc[mt][r]);
                }
            }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Large-m LDS-tiled GEMM: 128 x 128 output tile per block of 4 waves (2 x 2), 64 x 64 per wave as 4 x 4
// MFMA 16x16 tiles, 128-byte K steps staged through double-buffered LDS (row stride padded to 144 bytes).
// ---------------------------------------------------------------------------------------------------------
constexpr int kBM = 128, kBN = 128, kBK = 128, kLds = kBK + 16;

template <int QT>
__global__ __launch_bounds__(256) void gemm_kernel(int64_t m, int64_t n, int64_t k, const uint8_t *__restrict__ xq,
                                                   const float *__restrict__ xs, const uint8_t *__restrict__ wq,
                                                   const float *__restrict__ ws, void *__restrict__ y, int y_bf16,
                                                   void *__restrict__ acc_out, int64_t tiles_n) {
    typedef typename Acc<QT>::type acc_t;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBM * kLds];  // [buffer][A/B][tile]

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int j = lane & 15, g = lane >> 4;
    const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    // global -> register staging: 128 rows x 128 B = 1024 chunks of 16 B per operand, 4 per thread
    auto gload = [&](uint4 *ra, uint4 *rb, int64_t k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i;
            const int row = c >> 3, col = (c & 7) * 16;
            const int64_t kk = k0 + col;
            const int64_t ar = m0 + row, br = n0 + row;
            ra[i] = (ar < m && kk < k) ? *reinterpret_cast<const uint4 *>(xq + ar * k + kk) : make_uint4(0, 0, 0, 0);
            rb[i] = (br < n && kk < k) ? *reinterpret_cast<const uint4 *>(wq + br * k + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf, const uint4 *ra, const uint4 *rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i;
            const int row = c >> 3, col = (c & 7) * 16;
            *reinterpret_cast<uint4 *>(&lds[buf][0][row * kLds + col]) = ra[i];
            *reinterpret_cast<uint4 *>(&lds[buf][1][row * kLds + col]) = rb[i];
        }
    };

    acc_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = acc_t{0, 0, 0, 0};

    const int64_t nsteps = (k + kBK - 1) / kBK;
    uint4 ra[4], rb[4];
    gload(ra, rb, 0);
    sstore(0, ra, rb);
    __syncthreads();
    for (int64_t s = 0; s < nsteps; ++s) {
        const int buf = (int)(s & 1);
        if (s + 1 < nsteps) gload(ra, rb, (s + 1) * kBK);
        // lane (j, g) reads 32 contiguous K bytes of row j of each 16-row sub-tile
        uint4 fa[4][2], fb[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint8_t *p = &lds[buf][0][(wm * 64 + a * 16 + j) * kLds + g * 32];
            fa[a][0] = *reinterpret_cast<const uint4 *>(p);
            fa[a][1] = *reinterpret_cast<const uint4 *>(p + 16);
            const uint8_t *q = &lds[buf][1][(wn * 64 + a * 16 + j) * kLds + g * 32];
            fb[a][0] = *reinterpret_cast<const uint4 *>(q);
            fb[a][1] = *reinterpret_cast<const uint4 *>(q + 16);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                if constexpr (QT == kInt8) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        v4i av = {(int)fa[a][h].x, (int)fa[a][h].y, (int)fa[a][h].z, (int)fa[a][h].w};
                        v4i bv = {(int)fb[b][h].x, (int)fb[b][h].y, (int)fb[b][h].z, (int)fb[b][h].w};
                        acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[a][b], 0, 0, 0);
                    }
                } else {
                    v8i av = {(int)fa[a][0].x, (int)fa[a][0].y, (int)fa[a][0].z, (int)fa[a][0].w,
                              (int)fa[a][1].x, (int)fa[a][1].y, (int)fa[a][1].z, (int)fa[a][1].w};
                    v8i bv = {(int)fb[b][0].x, (int)fb[b][0].y, (int)fb[b][0].z, (int)fb[b][0].w,
                              (int)fb[b][1].x, (int)fb[b][1].y, (int)fb[b][1].z, (int)fb[b][1].w};
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[a][b], 0, 0, 0, 127, 0,
                                                                                   127);
                }
            }
        if (s + 1 < nsteps) sstore(buf ^ 1, ra, rb);
        __syncthreads();
    }

#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t col = n0 + wn * 64 + b * 16 + j;
        if (col >= n) continue;
        const float sw = ws[col];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + a * 16 + 4 * g + r;
                if (row < m) {
                    const float v = acc_to_f32(acc[a][b][r]) * xs[row] * sw;
                    store_y(y, row * n + col, v, y_bf16 != 0);
                    if (acc_out != nullptr) store_acc(acc_out, row * n + col, acc[a][b][r]);
                }
            }
    }
}

template <int QT, int MT, int WPB>
void launch_gemv_t(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                   const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                   hipStream_t stream) {
    const int64_t m_blocks = (m + 16 * MT - 1) / (16 * MT);
    int32_t *partials = nullptr;
    uint32_t *counters = nullptr;
    if (p.splits > 1) {
        counters = static_cast<uint32_t *>(workspace);
        partials = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(workspace) + kCounterBytes);
    }
    const dim3 grid((unsigned)p.n_tiles, (unsigned)p.splits, (unsigned)m_blocks);
    hipLaunchKernelGGL((gemv_kernel<QT, MT, WPB>), grid, dim3(WPB * 64), 0, stream, m, n, k, xq, xs, wq, ws, y,
                       y_bf16 ? 1 : 0, acc_out, p.splits, p.n_tiles, partials, counters);
}

template <int QT>
void launch_gemv_q(const LinearPlan &p, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                   const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                   hipStream_t stream) {
#define QR_GEMV_CASE(MT_, W_)                                                                                   \
    if (p.m_tiles == MT_ && p.waves == W_) {                                                                    \
        launch_gemv_t<QT, MT_, W_>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);           \
        return;                                                                                                 \
    }
    QR_GEMV_CASE(1, 4)
    QR_GEMV_CASE(2, 4)
    QR_GEMV_CASE(4, 4)
    QR_GEMV_CASE(1, 8)
    QR_GEMV_CASE(2, 8)
    QR_GEMV_CASE(4, 8)
    QR_GEMV_CASE(1, 2)
    QR_GEMV_CASE(1, 1)
#undef QR_GEMV_CASE
    // plan_linear only produces the cases above
    abort();
}

}  // namespace

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    if (v == nullptr || *v == '\0') return dflt;
    return atoi(v);
}

LinearPlan plan_linear(int qtype, int64_t m, int64_t n, int64_t k) {
    (void)qtype;
    LinearPlan p{};
    const int force = env_int("QR_FORCE_VARIANT", -1);  // 0 = GEMV, 1 = tiled GEMM
    const bool gemv = force == 0 || (force != 1 && m <= 64);
    if (!gemv) {
        p.kind = 1;
        p.ws_bytes = 0;
        return p;
    }
    p.kind = 0;
    p.m_tiles = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    int waves = env_int("QR_GEMV_WAVES", 4);
    if (waves != 1 && waves != 2 && waves != 4 && waves != 8) waves = 4;
    if (p.m_tiles > 1 && waves == 2) waves = 4;
    if (p.m_tiles > 1 && waves == 1) waves = 4;
    p.waves = waves;
    p.n_tiles = (n + 15) / 16;
    const int64_t steps = (k + kStep - 1) / kStep;
    const int64_t m_blocks = (m + 16 * p.m_tiles - 1) / (16 * p.m_tiles);
    // enough blocks to keep every CU streaming; never more splits than K steps per wave allow
    const int64_t target = env_int("QR_GEMV_TARGET_BLOCKS", 1024);
    int64_t splits = (target + p.n_tiles * m_blocks - 1) / (p.n_tiles * m_blocks);
    const int64_t max_split = steps / p.waves > 0 ? steps / p.waves : 1;
    if (splits > max_split) splits = max_split;
    if (splits < 1) splits = 1;
    const int forced = env_int("QR_SPLITK", 0);
    if (forced > 0) splits = forced < steps ? forced : steps;
    if (splits > 65535) splits = 65535;
    // split-K needs one counter per output tile; they live in a fixed region at the start of the workspace
    if (m_blocks * p.n_tiles > kMaxCounters) splits = 1;
    p.splits = (int)splits;
    if (p.splits > 1) {
        p.ws_bytes = kCounterBytes + (size_t)(m_blocks * p.n_tiles) * (size_t)p.splits * (size_t)(p.m_tiles * 256) * 4;
    } else {
        p.ws_bytes = 0;
    }
    return p;
}

hipError_t launch_linear(const LinearPlan &p, int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *xq,
                         const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                         void *workspace, hipStream_t stream) {
    if (p.kind == 0) {
        if (qtype == kInt8)
            launch_gemv_q<kInt8>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
        else
            launch_gemv_q<kFp8>(p, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
    } else {
        const int64_t tiles_m = (m + kBM - 1) / kBM, tiles_n = (n + kBN - 1) / kBN;
        const dim3 grid((unsigned)(tiles_m * tiles_n));
        if (qtype == kInt8)
            hipLaunchKernelGGL((gemm_kernel<kInt8>), grid, dim3(256), 0, stream, m, n, k, xq, xs, wq, ws, y,
                               y_bf16 ? 1 : 0, acc_out, tiles_n);
        else
            hipLaunchKernelGGL((gemm_kernel<kFp8>), grid, dim3(256), 0, stream, m, n, k, xq, xs, wq, ws, y,
                               y_bf16 ? 1 : 0, acc_out, tiles_n);
    }
    return hipGetLastError();
}

}  // namespace qr
