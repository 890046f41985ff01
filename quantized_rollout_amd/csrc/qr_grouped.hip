// qr_grouped.hip -- grouped (MoE) W8A8 linear over per-expert token lists, and the changed-code counter.
//
// Grouped linear: the expert FFNs of a mixture-of-experts model (the Qwen3-30B-A3B model of "QaRL:
// Rollout-Aligned Quantization-Aware RL ...", abstract) run in W8A8 (QaRL section 3.1). Output rows are
// grouped by expert in CSR form; expert e owns rows [offsets[e], offsets[e+1]) and row j reads activation
// row row_ids[j]. With top-8 routing of 256 tokens over 128 experts an expert sees ~16 rows, so each expert's
// product is a decode-sized GEMV and every expert's weights are read once: the HBM traffic that bounds the call
// (QaRL section 3.1 notes MoE rollout is memory-bound). The kernel is K-slice-major, like the dense GEMV: a
// block owns TB 16-channel tiles of one expert and all of K; wave w takes the 64U-byte K slices w, w + W, ...,
// loads the slice of up to 32 gathered activation rows once (coalesced, then moved into the MFMA layout with
// ds_bpermute) and the slice of its TB weight tiles in one burst, and runs one MFMA per (token tile, weight
// tile, 64-byte step). The waves' partial sums meet in LDS and are added in wave order. An expert with more
// than 32 rows takes further passes over the same weight tiles (served from L2).
//
// Changed-code counter: how many published codes (and scales) differ between two quantizations of the same
// tensor ("QuRL: Efficient Reinforcement Learning with Quantized Rollout", section 4.3: an RL update is much
// smaller than the quantization error, so most codes do not move).
#include "qr_device.hpp"
#include "qr_internal.hpp"

#include <algorithm>

namespace qr {
namespace {

constexpr int kGroupedMT = 2;  // 16-row token tiles per pass

__device__ __forceinline__ uint4 gload16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ v4i gv4(const uint4 &a) { return v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w}; }
__device__ __forceinline__ v8i gv8(const uint4 &a, const uint4 &b) {
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int QT, int U, int TB, int WMAX>
__global__ __launch_bounds__(WMAX * 64) void grouped_kernel(
    int64_t n, int64_t k, const int32_t *__restrict__ offsets, const int32_t *__restrict__ row_ids,
    int64_t total_rows, int64_t x_rows, const uint8_t *__restrict__ xq, const float *__restrict__ xs,
    const uint8_t *__restrict__ wq, const float *__restrict__ ws, void *__restrict__ y, int y_bf16) {
    typedef typename Acc<QT>::type acc_t;
    constexpr int MT = kGroupedMT;
    static_assert(QT == kInt8 || U % 2 == 0, "FP8 pairs load instructions");
    extern __shared__ int32_t red[];  // [waves][TB][MT][4][64]
    const int waves = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int64_t e = blockIdx.y;
    const int64_t tile0 = (int64_t)blockIdx.x * TB;
    constexpr int64_t kSlice = 64 * U;
    const int64_t slices = (k + kSlice - 1) / kSlice;
    const int64_t full = k / kSlice;

    // the expert's rows (offsets are clamped into [0, total_rows]; an empty expert leaves the block at once)
    int64_t r0 = offsets[e], r1 = offsets[e + 1];
    r0 = r0 < 0 ? 0 : (r0 > total_rows ? total_rows : r0);
    r1 = r1 < 0 ? 0 : (r1 > total_rows ? total_rows : r1);
    if (r1 <= r0) return;

    // weight rows of this lane (channels past n re-read channel n-1; those columns are never stored)
    const uint8_t *__restrict__ wrow[TB];
#pragma unroll
    for (int r = 0; r < TB; ++r) {
        const int64_t col = (tile0 + r) * 16 + j;
        wrow[r] = wq + (e * n + (col < n ? col : n - 1)) * k + 16 * g;
    }
    // activation row of output row jr: row_ids[jr] (or jr), -1 when out of range (its outputs are zero)
    auto xrow_of = [&](int64_t jr) -> int64_t {
        const int64_t xr = row_ids != nullptr ? (int64_t)row_ids[jr] : jr;
        return (xr >= 0 && xr < x_rows) ? xr : -1;
    };
    const int xr_lane = lane >> 2, xp = lane & 3;  // coalesced activation loads: token row l / 4, piece l % 4
    const int src_lane = 4 * j + g;                 // the lane that loads what lane (j, g) needs

    for (int64_t c0 = r0; c0 < r1; c0 += 16 * MT) {
        const uint8_t *__restrict__ xrow[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t jr = c0 + mt * 16 + xr_lane;
            const int64_t xr = jr < r1 ? xrow_of(jr) : -1;
            // rows past the expert's list, or with an out-of-range id, read activation row 0 instead: they only
            // feed outputs that are never stored (or stored as zero)
            xrow[mt] = xq + (xr >= 0 ? xr : 0) * k + 16 * xp;
        }
        acc_t acc[TB][MT];
#pragma unroll
        for (int r = 0; r < TB; ++r)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[r][mt] = acc_t{0, 0, 0, 0};

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
                        a[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(gv4(xv[mt][t]), gv4(wv[t]), a[mt], 0, 0, 0);
                } else {
#pragma unroll
                    for (int t = 0; t < U; t += 2)
                        // format 0 = E4M3 for both operands; scale exponents 127 = 2^0 (no block scaling)
                        a[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            gv8(xv[mt][t], xv[mt][t + 1]), gv8(wv[t], wv[t + 1]), a[mt], 0, 0, 0, 127, 0, 127);
                }
            }
        };
        for (int64_t sl = wave; sl < full; sl += waves) {
            const int64_t kb = sl * kSlice;
            uint4 xv[MT][U], wv[TB][U];
#pragma unroll
            for (int t = 0; t < U; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xv[mt][t] = gload16(xrow[mt] + kb + 64 * t);
#pragma unroll
            for (int r = 0; r < TB; ++r)
#pragma unroll
                for (int t = 0; t < U; ++t) wv[r][t] = gload16(wrow[r] + kb + 64 * t);
            transpose(xv);
#pragma unroll
            for (int r = 0; r < TB; ++r) mma(acc[r], xv, wv[r]);
        }
        if (full < slices && wave == full % waves) {  // the partial last slice: bytes past k are zero
            const int64_t kb = full * kSlice;
            uint4 xv[MT][U], wv[TB][U];
#pragma unroll
            for (int t = 0; t < U; ++t) {
                const bool in = kb + 64 * t + 16 * xp < k;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    xv[mt][t] = in ? gload16(xrow[mt] + kb + 64 * t) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < TB; ++r)
#pragma unroll
                for (int t = 0; t < U; ++t) {
                    const bool in = kb + 64 * t + 16 * g < k;
                    wv[r][t] = in ? gload16(wrow[r] + kb + 64 * t) : make_uint4(0, 0, 0, 0);
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
                            for (int w = 1; w < waves; ++w)
                                sum += __int_as_float(red[(int64_t)w * (kFrags * 256) + idx]);
                            acc[r][mt][i] = sum;
                        }
                    }
                }
                // epilogue: y[jr, col] = acc * x_scale[row_ids[jr]] * w_scale[e, col]
                const int64_t col = (tile0 + r) * 16 + j;
                if (col >= n) continue;
                const float sw = ws[e * n + col];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t jr = c0 + mt * 16 + 4 * g + i;
                    if (jr >= r1) continue;
                    const int64_t xr = xrow_of(jr);
                    const float v = xr >= 0 ? acc_to_f32(acc[r][mt][i]) * xs[xr] * sw : 0.0f;
                    if (y_bf16)
                        static_cast<uint16_t *>(y)[jr * n + col] = f32_to_bf16(v);
                    else
                        static_cast<float *>(y)[jr * n + col] = v;
                }
            }
        if (waves > 1) __syncthreads();  // the next pass reuses the LDS
    }
}

// (slice steps U, weight tiles per block TB, maximum waves)
#define QR_GROUPED_VARIANTS(X) X(4, 1, 8) X(4, 2, 8) X(4, 4, 8) X(8, 1, 8) X(8, 2, 8) X(2, 2, 8)

template <int QT, int U, int TB, int WMAX>
void launch_grouped_t(int waves, int64_t num_experts, int64_t n, int64_t k, const int32_t *offsets,
                      const int32_t *row_ids, int64_t total_rows, int64_t x_rows, const uint8_t *xq,
                      const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16,
                      hipStream_t stream) {
    const int64_t n_tiles = (n + 15) / 16;
    const dim3 grid((unsigned)((n_tiles + TB - 1) / TB), (unsigned)num_experts);
    const size_t lds = waves > 1 ? (size_t)waves * TB * kGroupedMT * 256 * 4 : 0;
    hipLaunchKernelGGL((grouped_kernel<QT, U, TB, WMAX>), grid, dim3(waves * 64), lds, stream, n, k, offsets, row_ids,
                       total_rows, x_rows, xq, xs, wq, ws, y, y_bf16 ? 1 : 0);
}

// ---------------------------------------------------------------------------------------------------------
// changed-code counter
// ---------------------------------------------------------------------------------------------------------
__global__ void zero3_kernel(unsigned long long *out3) {
    if (threadIdx.x < 3) out3[threadIdx.x] = 0ull;
}

// One streaming pass over both code sets: each lane keeps kCountUnroll pairs of 16-byte loads in flight (grid-
// stride over 16-byte words), compares bytes four at a time, and the counts are summed over the workgroup and
// added with one 64-bit atomic per workgroup and count. The loads are non-temporal (each byte is read once, so it
// should not displace cached data). Measured on MI355X over two 1.31 GB code sets: 4 pairs in flight on 2048
// workgroups 550 us; 8 pairs, non-temporal, 768 workgroups of 256 lanes 415 us = 6.3 TB/s. With one atomic per
// wavefront the 233 M codes of a 7B layer took 129 us in one call and 303 us in four (one per linear): the
// atomics, not the loads, set the time.
constexpr int kCountUnroll = 8;
constexpr int kCountThreads = 1024;
constexpr int kCountBlocks = 256;

template <bool NT>
__device__ __forceinline__ uint4 count_load(const uint4 *p) {
    if constexpr (NT) {
        const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
        return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
    } else {
        return *p;
    }
}

template <int UNR, bool NT>
__global__ __launch_bounds__(kCountThreads) void count_kernel(const uint8_t *__restrict__ a, const uint8_t *__restrict__ b,
                                                    int64_t count, int fp8, const uint32_t *__restrict__ sa,
                                                    const uint32_t *__restrict__ sb, int64_t n_scales,
                                                    unsigned long long *__restrict__ out3) {
    unsigned long long nb = 0, nv = 0, ns = 0;
    const int64_t n16 = count / 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint4 *__restrict__ a4 = reinterpret_cast<const uint4 *>(a);
    const uint4 *__restrict__ b4 = reinterpret_cast<const uint4 *>(b);
    int64_t i = tid;
    for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
        uint4 x[UNR], z[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            x[u] = count_load<NT>(a4 + i + u * stride);
            z[u] = count_load<NT>(b4 + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            count_word(x[u].x, z[u].x, fp8 != 0, nb, nv);
            count_word(x[u].y, z[u].y, fp8 != 0, nb, nv);
            count_word(x[u].z, z[u].z, fp8 != 0, nb, nv);
            count_word(x[u].w, z[u].w, fp8 != 0, nb, nv);
        }
    }
    for (; i < n16; i += stride) {
        const uint4 x = a4[i], z = b4[i];
        count_word(x.x, z.x, fp8 != 0, nb, nv);
        count_word(x.y, z.y, fp8 != 0, nb, nv);
        count_word(x.z, z.z, fp8 != 0, nb, nv);
        count_word(x.w, z.w, fp8 != 0, nb, nv);
    }
    for (int64_t t = n16 * 16 + tid; t < count; t += stride) count_word(a[t], b[t], fp8 != 0, nb, nv);
    for (int64_t t = tid; t < n_scales; t += stride) ns += (sa[t] != sb[t]) ? 1ull : 0ull;

    // the workgroup's sums (wavefronts, then LDS), one atomic per counter and workgroup: atomics on the same three
    // words serialize (about 14 ns each on MI355X), so their number, not the streaming, bounded the count when
    // every wavefront added its own
    nb = wave_sum_u64(nb);
    nv = wave_sum_u64(nv);
    ns = wave_sum_u64(ns);
    __shared__ unsigned long long part[3][kCountThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = nb;
        part[1][threadIdx.x >> 6] = nv;
        part[2][threadIdx.x >> 6] = ns;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        unsigned long long v = 0;
        for (int w = 0; w < kCountThreads / 64; ++w) v += part[threadIdx.x][w];
        if (v) atomicAdd(out3 + threadIdx.x, v);
    }
}

}  // namespace

size_t grouped_workspace_bytes(int qtype, int64_t total_rows, int64_t n, int64_t k, int64_t num_experts) {
    (void)qtype;
    (void)total_rows;
    (void)n;
    (void)k;
    (void)num_experts;
    return 0;
}

hipError_t launch_grouped(int qtype, int64_t num_experts, int64_t n, int64_t k, const int32_t *offsets,
                          const int32_t *row_ids, int64_t total_rows, int64_t x_rows, const uint8_t *xq,
                          const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16,
                          hipStream_t stream) {
    // 128-byte K slices, two 16-channel tiles per block, about four slices per wave and at most four waves
    // (measured on MI355X for the 128-expert FP8 MoE linears: fewer, longer-running waves per block beat the
    // LDS reduction of many)
    int u = env_int("QR_GROUPED_UNROLL", 2), tb = env_int("QR_GROUPED_TILES", 2);
    bool known = false;
#define QR_GROUPED_KNOWN(U_, TB_, W_) known = known || (u == U_ && tb == TB_);
    QR_GROUPED_VARIANTS(QR_GROUPED_KNOWN)
#undef QR_GROUPED_KNOWN
    if (!known) {  // overrides that name no compiled variant fall back to the default
        u = 2;
        tb = 2;
    }
    const int64_t slices = (k + 64 * u - 1) / (64 * u);
    int waves = env_int("QR_GROUPED_WAVES", 0);
    if (waves < 1 || waves > 8) waves = (int)std::min<int64_t>(4, std::max<int64_t>(1, slices / 4));
    bool done = false;
#define QR_GROUPED_CASE(U_, TB_, W_)                                                                             \
    if (!done && u == U_ && tb == TB_) {                                                                         \
        if (qtype == kInt8)                                                                                      \
            launch_grouped_t<kInt8, U_, TB_, W_>(waves, num_experts, n, k, offsets, row_ids, total_rows, x_rows, \
                                                 xq, xs, wq, ws, y, y_bf16, stream);                             \
        else                                                                                                     \
            launch_grouped_t<kFp8, U_, TB_, W_>(waves, num_experts, n, k, offsets, row_ids, total_rows, x_rows,  \
                                                xq, xs, wq, ws, y, y_bf16, stream);                              \
        done = true;                                                                                             \
    }
    QR_GROUPED_VARIANTS(QR_GROUPED_CASE)
#undef QR_GROUPED_CASE
    return hipGetLastError();
}

hipError_t launch_count_changes(const uint8_t *a, const uint8_t *b, int64_t count, int qtype, const float *sa,
                                const float *sb, int64_t n_scales, int64_t *out3, hipStream_t stream) {
    unsigned long long *o = reinterpret_cast<unsigned long long *>(out3);
    hipLaunchKernelGGL(zero3_kernel, dim3(1), dim3(64), 0, stream, o);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // one 1024-lane workgroup per CU at most (16 wavefronts each), fewer for small inputs
    const int64_t work = count / 16 > n_scales ? count / 16 : n_scales;
    const int unr = env_int("QR_COUNT_UNROLL", kCountUnroll) == 4 ? 4 : kCountUnroll;
    const bool nt = env_int("QR_COUNT_NT", 1) > 0;
    int64_t blocks = (work + (int64_t)kCountThreads * unr - 1) / ((int64_t)kCountThreads * unr);
    const int64_t max_blocks = env_int("QR_COUNT_BLOCKS", kCountBlocks);
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
#define QR_COUNT(U_, NT_)                                                                                    \
    hipLaunchKernelGGL((count_kernel<U_, NT_>), dim3((unsigned)blocks), dim3(kCountThreads), 0, stream, a, b, count, \
                       qtype == kFp8 ? 1 : 0, reinterpret_cast<const uint32_t *>(sa),                      \
                       reinterpret_cast<const uint32_t *>(sb), n_scales, o)
    if (unr == 8) {
        if (nt) QR_COUNT(8, true); else QR_COUNT(8, false);
    } else {
        if (nt) QR_COUNT(4, true); else QR_COUNT(4, false);
    }
#undef QR_COUNT
    return hipGetLastError();
}


// ---------------------------------------------------------------------------------------------------------
// Token-list check (debug mode): one workgroup reads the offsets and row ids once and writes the OR of the
// failed conditions (see check_token_lists) to a device word that the host then copies back.
// ---------------------------------------------------------------------------------------------------------
__device__ int g_token_list_bits;

__global__ __launch_bounds__(1024) void token_list_check_kernel(const int32_t *__restrict__ offsets, int64_t num_experts,
                                                                const int32_t *__restrict__ row_ids, int64_t total_rows,
                                                                int64_t x_rows) {
    __shared__ int bits_all;
    const int t = threadIdx.x;
    if (t == 0) bits_all = 0;
    __syncthreads();
    int bits = 0;
    if (t == 0) {
        if (offsets[0] != 0) bits |= 1;
        if ((int64_t)offsets[num_experts] != total_rows) bits |= 2;
    }
    for (int64_t e = t; e < num_experts; e += blockDim.x)
        if (offsets[e + 1] < offsets[e]) bits |= 4;
    if (row_ids != nullptr)
        for (int64_t j = t; j < total_rows; j += blockDim.x) {
            const int32_t r = row_ids[j];
            if (r < 0 || (int64_t)r >= x_rows) bits |= 8;
        }
    if (bits != 0) atomicOr(&bits_all, bits);
    __syncthreads();
    if (t == 0) g_token_list_bits = bits_all;
}

hipError_t check_token_lists(const int32_t *offsets, int64_t num_experts, const int32_t *row_ids, int64_t total_rows,
                             int64_t x_rows, int *bits, hipStream_t stream) {
    hipLaunchKernelGGL(token_list_check_kernel, dim3(1), dim3(1024), 0, stream, offsets, num_experts, row_ids,
                       total_rows, x_rows);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = hipMemcpyFromSymbolAsync(bits, HIP_SYMBOL(g_token_list_bits), sizeof(int), 0, hipMemcpyDeviceToHost, stream);
    if (err != hipSuccess) return err;
    return hipStreamSynchronize(stream);
}

}  // namespace qr
