// qr_grouped.hip -- grouped (MoE) W8A8 linear over per-expert token lists, and the changed-code counter.
//
// Grouped linear: the expert FFNs of a mixture-of-experts model (the Qwen3-30B-A3B model of "QaRL:
// Rollout-Aligned Quantization-Aware RL ...", abstract) run in W8A8 (QaRL section 3.1). Output rows are
// grouped by expert in CSR form; expert e owns rows [offsets[e], offsets[e+1]) and row j reads activation
// row row_ids[j]. With top-8 routing of 256 tokens over 128 experts an expert sees ~16 rows, so the kernel
// is the GEMV of qr_linear.hip per expert: a wave owns 16 output channels of one expert and streams that
// expert's weight rows once per 32 gathered activation rows (two MFMA token tiles). Every expert's weights
// are read, which is the HBM traffic that bounds the call (QaRL section 3.1 notes MoE rollout is
// memory-bound). No split of K is needed: experts x channel tiles give >10k waves.
//
// Changed-code counter: how many published codes (and scales) differ between two quantizations of the same
// tensor ("QuRL: Efficient Reinforcement Learning with Quantized Rollout", section 4.3: an RL update is much
// smaller than the quantization error, so most codes do not move).
#include "qr_device.hpp"
#include "qr_internal.hpp"

namespace qr {
namespace {

constexpr int kStep = 256;
constexpr int kGroupedWaves = 4;
constexpr int kGroupedMT = 2;

__device__ __forceinline__ void load_step_g(uint4 *dst, const uint8_t *__restrict__ row_ptr, int64_t kb, int64_t k) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t off = kb + 16 * t;
        if (row_ptr != nullptr && off < k)
            dst[t] = *reinterpret_cast<const uint4 *>(row_ptr + off);
        else
            dst[t] = make_uint4(0, 0, 0, 0);
    }
}

template <int QT>
__global__ __launch_bounds__(kGroupedWaves * 64) void grouped_kernel(
    int64_t n, int64_t k, const int32_t *__restrict__ offsets, const int32_t *__restrict__ row_ids,
    int64_t total_rows, int64_t x_rows, const uint8_t *__restrict__ xq, const float *__restrict__ xs,
    const uint8_t *__restrict__ wq, const float *__restrict__ ws, void *__restrict__ y, int y_bf16) {
    typedef typename Acc<QT>::type acc_t;
    constexpr int MT = kGroupedMT;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int64_t e = blockIdx.y;
    const int64_t tile = (int64_t)blockIdx.x * kGroupedWaves + wave;
    const int64_t ncol = tile * 16 + j;
    if (tile * 16 >= n) return;

    int64_t r0 = offsets[e], r1 = offsets[e + 1];
    r0 = r0 < 0 ? 0 : (r0 > total_rows ? total_rows : r0);
    r1 = r1 < 0 ? 0 : (r1 > total_rows ? total_rows : r1);
    if (r1 <= r0) return;

    const uint8_t *__restrict__ wrow = ncol < n ? wq + (e * n + ncol) * k : nullptr;
    const float sw = ncol < n ? ws[e * n + ncol] : 0.0f;
    const int64_t steps = (k + kStep - 1) / kStep;

    for (int64_t mc = r0; mc < r1; mc += 16 * MT) {
        // activation rows this lane feeds into the two token tiles
        const uint8_t *__restrict__ xrow[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t jr = mc + mt * 16 + j;
            xrow[mt] = nullptr;
            if (jr < r1) {
                const int64_t xr = row_ids != nullptr ? (int64_t)row_ids[jr] : jr;
                if (xr >= 0 && xr < x_rows) xrow[mt] = xq + xr * k;
            }
        }
        acc_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = acc_t{0, 0, 0, 0};

        uint4 wcur[4], xcur[MT][4];
        load_step_g(wcur, wrow, g * 64, k);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load_step_g(xcur[mt], xrow[mt], g * 64, k);
        for (int64_t st = 0;; ++st) {
            uint4 wnxt[4], xnxt[MT][4];
            const bool more = st + 1 < steps;
            if (more) {
                load_step_g(wnxt, wrow, (st + 1) * kStep + g * 64, k);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) load_step_g(xnxt[mt], xrow[mt], (st + 1) * kStep + g * 64, k);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma_step(acc[mt], xcur[mt], wcur);
            if (!more) break;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                wcur[t] = wnxt[t];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xcur[mt][t] = xnxt[mt][t];
            }
        }

        if (ncol < n) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t jr = mc + mt * 16 + 4 * g + r;
                    if (jr >= r1) continue;
                    const int64_t xr = row_ids != nullptr ? (int64_t)row_ids[jr] : jr;
                    float v = 0.0f;
                    if (xr >= 0 && xr < x_rows) v = acc_to_f32(acc[mt][r]) * xs[xr] * sw;
                    if (y_bf16)
                        static_cast<uint16_t *>(y)[jr * n + ncol] = f32_to_bf16(v);
                    else
                        static_cast<float *>(y)[jr * n + ncol] = v;
                }
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// changed-code counter
// ---------------------------------------------------------------------------------------------------------
__global__ void zero3_kernel(unsigned long long *out3) {
    if (threadIdx.x < 3) out3[threadIdx.x] = 0ull;
}

// Bytes of a 32-bit word that are nonzero, as a mask with 0x80 in each such byte.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
    return (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
}

__device__ __forceinline__ void count_word(uint32_t a, uint32_t b, bool fp8, unsigned long long &nb,
                                           unsigned long long &nv) {
    const uint32_t diff = nonzero_bytes(a ^ b);
    const int d = __popc(diff);
    nb += d;
    if (fp8) {
        // +0 (0x00) and -0 (0x80) are one value: a byte pair whose magnitudes are both zero
        const uint32_t both_zero = ~nonzero_bytes((a | b) & 0x7F7F7F7Fu) & 0x80808080u;
        nv += d - __popc(diff & both_zero);
    } else {
        nv += d;
    }
}

// One streaming pass over both code sets: each lane keeps kCountUnroll pairs of 16-byte loads in flight (grid-
// stride over 16-byte words), compares bytes four at a time, and the counts are summed over the wave and added
// with one 64-bit atomic per wave and count.
constexpr int kCountUnroll = 4;

__global__ __launch_bounds__(256) void count_kernel(const uint8_t *__restrict__ a, const uint8_t *__restrict__ b,
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
    for (; i + (kCountUnroll - 1) * stride < n16; i += kCountUnroll * stride) {
        uint4 x[kCountUnroll], z[kCountUnroll];
#pragma unroll
        for (int u = 0; u < kCountUnroll; ++u) {
            x[u] = a4[i + u * stride];
            z[u] = b4[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < kCountUnroll; ++u) {
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

    nb = wave_sum_u64(nb);
    nv = wave_sum_u64(nv);
    ns = wave_sum_u64(ns);
    if ((threadIdx.x & 63) == 0) {
        if (nb) atomicAdd(out3 + 0, nb);
        if (nv) atomicAdd(out3 + 1, nv);
        if (ns) atomicAdd(out3 + 2, ns);
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
    const int64_t n_tiles = (n + 15) / 16;
    const dim3 grid((unsigned)((n_tiles + kGroupedWaves - 1) / kGroupedWaves), (unsigned)num_experts);
    if (qtype == kInt8)
        hipLaunchKernelGGL((grouped_kernel<kInt8>), grid, dim3(kGroupedWaves * 64), 0, stream, n, k, offsets,
                           row_ids, total_rows, x_rows, xq, xs, wq, ws, y, y_bf16 ? 1 : 0);
    else
        hipLaunchKernelGGL((grouped_kernel<kFp8>), grid, dim3(kGroupedWaves * 64), 0, stream, n, k, offsets,
                           row_ids, total_rows, x_rows, xq, xs, wq, ws, y, y_bf16 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_count_changes(const uint8_t *a, const uint8_t *b, int64_t count, int qtype, const float *sa,
                                const float *sb, int64_t n_scales, int64_t *out3, hipStream_t stream) {
    unsigned long long *o = reinterpret_cast<unsigned long long *>(out3);
    hipLaunchKernelGGL(zero3_kernel, dim3(1), dim3(64), 0, stream, o);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // enough 256-thread blocks for every CU to hold several (2048 = 256 CUs x 8), fewer for small inputs
    const int64_t work = count / 16 > n_scales ? count / 16 : n_scales;
    int64_t blocks = (work + 256 * kCountUnroll - 1) / (256 * kCountUnroll);
    const int64_t max_blocks = env_int("QR_COUNT_BLOCKS", 2048);
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, count,
                       qtype == kFp8 ? 1 : 0, reinterpret_cast<const uint32_t *>(sa),
                       reinterpret_cast<const uint32_t *>(sb), n_scales, o);
    return hipGetLastError();
}

}  // namespace qr
