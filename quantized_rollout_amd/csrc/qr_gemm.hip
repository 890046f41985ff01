// qr_gemm.hip -- the W8A8 linear for large batches: LDS-tiled MFMA GEMM (INT8 -> INT32, E4M3 -> FP32).
//
// y[i,c] = acc[i,c] * x_scale[i] * w_scale[c], acc = sum_j xq[i,j] * wq[c,j] -- the W8A8 product of quantized
// rollout ("QuRL: Efficient Reinforcement Learning with Quantized Rollout", section 5; "QaRL: Rollout-Aligned
// Quantization-Aware RL ...", sections 2.2 and 3.1) at the rollout batch sizes where the matrix cores, not HBM,
// bound the layer.
//
// Workgroup tile BM x BN of outputs, four wavefronts in a 2 x 2 arrangement, each owning a (BM/2) x (BN/2)
// register tile of 16x16 MFMA fragments (256 accumulators per lane at 256 x 256). K advances in 128-byte
// stages through two LDS buffers (rows padded to 144 bytes so that the sixteen rows a fragment read touches
// fall on distinct banks); the global loads of stage s+1 are in flight while stage s runs its MFMAs. Both
// operands are K-contiguous (codes in their canonical row-major layout), and a fragment read gives lane
// (j, g) 16 bytes of row j at K offset 16 g of each 64-byte half of the stage, the same for activations and
// weights, so the MFMA dot products are those of the plain definition. Workgroups are dispatched round-robin
// over the 8 XCDs; the tile order gives each XCD a contiguous run of tiles, token tiles fastest, so the
// workgroups that share a weight tile run on one XCD and share its L2.
#include "qr_device.hpp"
#include "qr_internal.hpp"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace qr {
namespace {

// f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N-1>): indices known at compile time, so
// register arrays (the accumulators) indexed by them stay in registers
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F &&f) {
    unroll_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int kBK = 128;            // K bytes per stage
constexpr int kRow = kBK + 16;      // padded LDS row stride

__device__ __forceinline__ v4i v4(const uint4 &a) { return v4i{(int)a.x, (int)a.y, (int)a.z, (int)a.w}; }
__device__ __forceinline__ v8i v8(const uint4 &a, const uint4 &b) {
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int QT, int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(int64_t m, int64_t n, int64_t k,
                                                            const uint8_t *__restrict__ xq,
                                                            const float *__restrict__ xs,
                                                            const uint8_t *__restrict__ wq,
                                                            const float *__restrict__ ws, void *__restrict__ y,
                                                            int y_bf16, void *__restrict__ acc_out, int tiles_m,
                                                            int tiles_n) {
    typedef typename Acc<QT>::type acc_t;
    constexpr int WM = BM / 2, WN = BN / 2;     // wave tile
    constexpr int FM = WM / 16, FN = WN / 16;   // 16x16 fragments per wave
    constexpr int CA = BM * kBK / 16 / 256;     // 16-byte chunks per thread per stage, activations
    constexpr int CB = BN * kBK / 16 / 256;     // weights
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * kRow];

    // tile order: each XCD (workgroup id mod 8) takes a contiguous run of the order, token tiles fastest
    const int total = tiles_m * tiles_n;
    const int per_xcd = (total + 7) / 8;
    const int order = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (order >= total) return;
    const int64_t m0 = (int64_t)(order % tiles_m) * BM;
    const int64_t n0 = (int64_t)(order / tiles_m) * BN;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int j = lane & 15, g = lane >> 4;

    // global -> LDS staging: chunk c of a stage is row c >> 3, bytes 16 (c & 7); rows past the end re-read the
    // last row (they only feed outputs that are never stored)
    const uint8_t *arow[CA];
    const uint8_t *brow[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int c = t + 256 * i;
        const int64_t r = m0 + (c >> 3);
        arow[i] = xq + (r < m ? r : m - 1) * k + 16 * (c & 7);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        const int c = t + 256 * i;
        const int64_t r = n0 + (c >> 3);
        brow[i] = wq + (r < n ? r : n - 1) * k + 16 * (c & 7);
    }
    uint4 ra[CA], rb[CB];
    auto gload = [&](int64_t k0) {  // a full stage: every load in range, none conditional
#pragma unroll
        for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const uint4 *>(arow[i] + k0);
#pragma unroll
        for (int i = 0; i < CB; ++i) rb[i] = *reinterpret_cast<const uint4 *>(brow[i] + k0);
    };
    auto gload_tail = [&](int64_t k0) {  // the partial last stage: bytes past k are zero
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = t + 256 * i;
            ra[i] = k0 + 16 * (c & 7) < k ? *reinterpret_cast<const uint4 *>(arow[i] + k0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = t + 256 * i;
            rb[i] = k0 + 16 * (c & 7) < k ? *reinterpret_cast<const uint4 *>(brow[i] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int c = t + 256 * i;
            *reinterpret_cast<uint4 *>(&lds[buf][(c >> 3) * kRow + 16 * (c & 7)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int c = t + 256 * i;
            *reinterpret_cast<uint4 *>(&lds[buf][(BM + (c >> 3)) * kRow + 16 * (c & 7)]) = rb[i];
        }
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = acc_t{0, 0, 0, 0};

    auto compute = [&](int buf) {
        const uint8_t *A = &lds[buf][(wm * WM + j) * kRow + 16 * g];
        const uint8_t *B = &lds[buf][(BM + wn * WN + j) * kRow + 16 * g];
        uint4 fa[FM][2], fb[FN][2];
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            fa[a][0] = *reinterpret_cast<const uint4 *>(A + a * 16 * kRow);
            fa[a][1] = *reinterpret_cast<const uint4 *>(A + a * 16 * kRow + 64);
        }
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            fb[b][0] = *reinterpret_cast<const uint4 *>(B + b * 16 * kRow);
            fb[b][1] = *reinterpret_cast<const uint4 *>(B + b * 16 * kRow + 64);
        }
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                if constexpr (QT == kInt8) {
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4(fa[a][0]), v4(fb[b][0]), acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4(fa[a][1]), v4(fb[b][1]), acc[a][b], 0, 0, 0);
                } else {
                    // format 0 = E4M3 for both operands; scale exponents 127 = 2^0 (no block scaling)
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        v8(fa[a][0], fa[a][1]), v8(fb[b][0], fb[b][1]), acc[a][b], 0, 0, 0, 127, 0, 127);
                }
            }
    };

    const int64_t full = k / kBK;
    const int64_t stages = (k + kBK - 1) / kBK;
    if (full > 0)
        gload(0);
    else
        gload_tail(0);
    sstore(0);
    __syncthreads();
    for (int64_t s = 0; s < stages; ++s) {
        const int buf = (int)(s & 1);
        const bool more = s + 1 < stages;
        if (s + 1 < full)
            gload((s + 1) * kBK);
        else if (more)
            gload_tail((s + 1) * kBK);
        compute(buf);
        if (more) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: y = acc * x_scale[row] * w_scale[col], the scales loaded together from clamped indices
    float sw[FN];
#pragma unroll
    for (int b = 0; b < FN; ++b) {
        const int64_t col = n0 + wn * WN + b * 16 + j;
        sw[b] = ws[col < n ? col : n - 1];
    }
    unroll<FM>([&](auto A) {
        constexpr int a = decltype(A)::value;
        float sx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = m0 + wm * WM + a * 16 + 4 * g + i;
            sx[i] = xs[row < m ? row : m - 1];
        }
        unroll<FN>([&](auto B) {
            constexpr int b = decltype(B)::value;
            const int64_t col = n0 + wn * WN + b * 16 + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + wm * WM + a * 16 + 4 * g + i;
                if (row < m && col < n) {
                    const float v = acc_to_f32(acc[a][b][i]) * sx[i] * sw[b];
                    if (y_bf16)
                        static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(v);
                    else
                        static_cast<float *>(y)[row * n + col] = v;
                    if (acc_out != nullptr) {
                        if constexpr (QT == kInt8)
                            static_cast<int32_t *>(acc_out)[row * n + col] = acc[a][b][i];
                        else
                            static_cast<float *>(acc_out)[row * n + col] = acc[a][b][i];
                    }
                }
            }
        });
    });
}

// ---------------------------------------------------------------------------------------------------------
// Ring-pipelined GEMM: BM x BN outputs per workgroup (BM = 256 or 128 activation rows, BN = 256, 128 or 64
// channels), wavefronts of 64 x 64 outputs each (2 x 2 fragments of the 32x32 MFMA: v_mfma_i32_32x32x32_i8,
// or v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit block scales), 64 accumulators per lane. K
// advances in 64-byte stages through a ring of four LDS buffers filled straight from memory by buffer loads
// with the LDS flag (no registers in between), up to three stages ahead of the MFMAs. A workgroup's loads are
// spread over all its wavefronts: the rate at which one wavefront's memory instructions are served is
// limited, so more wavefronts issuing them fetch more per CU. Each buffer holds the stage's BM activation rows
// then its BN weight rows, 64 bytes each, with
// logical 16-byte piece c of row r stored at physical piece c ^ ring_swizzle(r). The buffer resources bound
// the rows (rows past m or n load zeros) and the partial last stage points its out-of-range pieces past the
// end. A 32x32 fragment read gives lane l row (l & 31) and logical pieces (l >> 5) and 2 + (l >> 5) (INT8,
// two MFMAs of K = 32) or 2 (l >> 5) and 2 (l >> 5) + 1 (FP8, one MFMA of K = 64), the same for both
// operands, so the dot products are those of the plain definition. Result C[i][c] sits in lane
// (c + 32 (i / 4 mod 2)), register 4 (i / 8) + i mod 4.
// ---------------------------------------------------------------------------------------------------------
constexpr int kRingK = 64;   // K bytes per stage

// Tile of BM activation rows x BN channels: BM BN / 4096 wavefronts of 64 x 64 outputs in a (BM / 64) x (BN / 64)
// arrangement, each loading BM / waves activation rows and BN / waves weight rows (16 per load) of every stage.
// The narrow tiles are for few-row batches, where 256-channel tiles leave most CUs idle or need many K splits.
template <int BM, int BN>
struct Ring {
    static constexpr int kWaves = BM * BN / 4096;
    static constexpr int kWavesN = BN / 64;  // wavefronts across the channels
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBuf = (BM + BN) * kRingK;  // bytes per ring buffer
    static constexpr int kRowsA = BM / kWaves;       // activation rows loaded per wavefront
    static constexpr int kRowsB = BN / kWaves;       // weight rows loaded per wavefront
    static constexpr int kLoadsA = kRowsA / 16;
    static constexpr int kLoadsB = kRowsB / 16;
    static constexpr int kLoads = kLoadsA + kLoadsB;  // buffer loads per wavefront per stage
    static_assert(kRowsA % 16 == 0 && kRowsB % 16 == 0, "16 rows per load");
    // the bf16 epilogue stages each wavefront's 64 x 64 outputs (8 KiB) in the ring
    static_assert(kWaves * 8192 <= 4 * kBuf, "epilogue staging fits the ring");
};

typedef __attribute__((address_space(3))) void lds_void_t;

// piece permutation of a ring row (see above). A 16-byte-per-lane LDS read serves each half-wave as two
// groups of 16 lanes (split by the parity of lane bits 2..4), each group in one cycle over 64 four-byte banks;
// the lanes of a fragment read are 32 consecutive rows at one logical piece, so a group is conflict-free when
// its rows with equal (r mod 4) hold that piece at distinct physical pieces, which (r / 4) mod 4 provides.
__device__ __forceinline__ int ring_swizzle(int r) { return (r >> 2) & 3; }

template <int QT>
struct Acc32;
template <>
struct Acc32<kInt8> {
    typedef int __attribute__((ext_vector_type(16))) type;
};
template <>
struct Acc32<kFp8> {
    typedef float __attribute__((ext_vector_type(16))) type;
};

template <int QT, int BM, int BN>
__global__ __launch_bounds__((Ring<BM, BN>::kThreads), 1) void gemm_ring_kernel(
    int64_t m, int64_t n, int64_t k, const uint8_t *__restrict__ xq, const float *__restrict__ xs,
    const uint8_t *__restrict__ wq, const float *__restrict__ ws, void *__restrict__ y, int y_bf16,
    void *__restrict__ acc_out, int tiles_m, int tiles_n, int splits, int stages_per_split,
    void *__restrict__ partial, int dp_tiles) {
    typedef Ring<BM, BN> R;
    typedef typename Acc32<QT>::type acc_t;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * R::kBuf];  // local stage s in buffer s mod 4

    // work item order: each XCD (workgroup id mod 8) takes a contiguous run, split-major then token tiles
    // fastest, so the workgroups that share an operand slice run on one XCD and share its L2
    const int tiles = tiles_m * tiles_n;
    const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
    int split = 0, tile;
    bool to_partial;
    if (dp_tiles == 0) {
        const int total = tiles * splits;
        const int per_xcd = (total + 7) / 8;
        const int order = xcd * per_xcd + slot;
        if (order >= total) return;
        split = order / tiles;
        tile = order % tiles;
        to_partial = splits > 1;
    } else {
        // whole-K tiles first: each XCD's first dp_tiles / 8 workgroups, a contiguous run of tiles (whole CU
        // rounds, dp_tiles being a multiple of the CU count); then the K pieces of the remaining tiles, spread
        // evenly over the XCDs and dispatched as CUs free up
        const int dpx = dp_tiles / 8;
        if (slot < dpx) {
            tile = xcd * dpx + slot;
            to_partial = false;
        } else {
            const int rem = tiles - dp_tiles, pieces = rem * splits;
            const int p = xcd * ((pieces + 7) / 8) + (slot - dpx);
            if (p >= pieces) return;
            split = p / rem;
            tile = dp_tiles + p % rem;
            to_partial = true;
        }
    }
    const int64_t m0 = (int64_t)(tile % tiles_m) * BM;
    const int64_t n0 = (int64_t)(tile / tiles_m) * BN;
    const int64_t all_stages = (k + kRingK - 1) / kRingK;
    const int64_t st0 = to_partial ? (int64_t)split * stages_per_split : 0;
    const int64_t stages = to_partial ? std::min<int64_t>(stages_per_split, all_stages - st0)  // >= 1 by construction
                                      : all_stages;
    const int64_t full = k / kRingK;  // stages with every piece inside k

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / R::kWavesN, wn = wave % R::kWavesN;

    // buffer resources over the whole operands: rows past the end load zeros
    const v4i rsa = make_rsrc(xq, (uint32_t)(m * k));
    const v4i rsb = make_rsrc(wq, (uint32_t)(n * k));

    // stage loads, 16 rows per instruction; lane l writes physical piece l & 3 of row l / 4 of the block, which
    // holds logical piece (l & 3) ^ swz(row). Activation rows kRowsA wave ..; weight rows kRowsB wave ..
    uint32_t offa[R::kLoadsA];
    int lpa[R::kLoadsA];
#pragma unroll
    for (int q = 0; q < R::kLoadsA; ++q) {
        const int r = wave * R::kRowsA + q * 16 + (lane >> 2);
        lpa[q] = (lane & 3) ^ ring_swizzle(r);
        offa[q] = m0 + r < m ? (uint32_t)((m0 + r) * k + 16 * lpa[q]) : kOutOfRange;
    }
    uint32_t offb[R::kLoadsB];
    int lpb[R::kLoadsB];
#pragma unroll
    for (int q = 0; q < R::kLoadsB; ++q) {
        const int r = wave * R::kRowsB + q * 16 + (lane >> 2);
        lpb[q] = (lane & 3) ^ ring_swizzle(r);
        offb[q] = n0 + r < n ? (uint32_t)((n0 + r) * k + 16 * lpb[q]) : kOutOfRange;
    }
    auto issue = [&](int64_t gst, uint8_t *buf) {  // global stage gst into buffer buf
        const uint32_t k0 = (uint32_t)(gst * kRingK);
        const bool tail = gst >= full;
#pragma unroll
        for (int q = 0; q < R::kLoadsA; ++q) {
            const bool in = !tail || (int64_t)k0 + 16 * lpa[q] < k;
            dma16(rsa, lds_addr(buf + (wave * R::kRowsA + q * 16) * kRingK),
                  (in && offa[q] != kOutOfRange) ? offa[q] + k0 : kOutOfRange);
        }
#pragma unroll
        for (int q = 0; q < R::kLoadsB; ++q) {
            const bool in = !tail || (int64_t)k0 + 16 * lpb[q] < k;
            dma16(rsb, lds_addr(buf + (BM + wave * R::kRowsB + q * 16) * kRingK),
                  (in && offb[q] != kOutOfRange) ? offb[q] + k0 : kOutOfRange);
        }
    };

    acc_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = acc_t{};

    // fragment reads: lane row (l & 31), half h = l >> 5
    const int fr = lane & 31, h = lane >> 5;
    const int p0 = QT == kInt8 ? h : 2 * h, p1 = QT == kInt8 ? 2 + h : 2 * h + 1;
    struct Frags {
        uint4 a[2][2], b[2][2];
    };
    // read x of a stage (x = 0..7): A fragment x / 2 piece x % 2 for x < 4, then B fragment (x - 4) / 2
    auto read_one = [&](const uint8_t *buf, Frags &f, auto X) {
        constexpr int x = decltype(X)::value;
        if constexpr (x < 4) {
            const int r = wm * 64 + (x / 2) * 32 + fr;
            f.a[x / 2][x & 1] = *reinterpret_cast<const uint4 *>(buf + r * kRingK + 16 * (((x & 1) ? p1 : p0) ^ ring_swizzle(r)));
        } else {
            const int r = wn * 64 + ((x - 4) / 2) * 32 + fr;
            f.b[(x - 4) / 2][x & 1] =
                *reinterpret_cast<const uint4 *>(buf + (BM + r) * kRingK + 16 * (((x & 1) ? p1 : p0) ^ ring_swizzle(r)));
        }
    };
    // MFMA tile x (x = 0..3): fragments (x / 2, x % 2)
    auto mfma_one = [&](const Frags &f, auto X) {
        constexpr int x = decltype(X)::value, i = x / 2, j = x % 2;
        if constexpr (QT == kInt8) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4(f.a[i][0]), v4(f.b[j][0]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4(f.a[i][1]), v4(f.b[j][1]), acc[i][j], 0, 0, 0);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8(f.a[i][0], f.a[i][1]), v8(f.b[j][0], f.b[j][1]),
                                                                         acc[i][j], 0, 0, 0, 127, 0, 127);
        }
    };
    // wait until this wave's loads of a stage have landed (`later` = stages issued after it, 0..2) and its own
    // fragment reads are done; the barrier then makes every wave's loads of the stage visible and tells every
    // wave that all fragment reads issued before it are complete
    auto sync_stage = [&](int64_t later) {
        if (later >= 2)
            wait_vmcnt_lgkm0<2 * R::kLoads>();
        else if (later == 1)
            wait_vmcnt_lgkm0<R::kLoads>();
        else
            wait_vmcnt_lgkm0<0>();
        barrier_fenced();
    };
    auto buffer = [&](int64_t s) { return ring + (int)(s & 3) * R::kBuf; };
    // Pipeline: stage s + 3 is loaded while stage s runs. Each step waits for its own stage, refills the buffer
    // of stage s - 1 (which every wave has finished reading before the barrier of step s) with stage s + 3,
    // reads its fragments and runs its MFMAs; other wavefronts on the SIMD (or other workgroups on the CU, for
    // the small tiles) cover each one's fragment reads.
    Frags f;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (i < stages) issue(st0 + i, ring + i * R::kBuf);
    int64_t s = 0;
    for (; s + 3 < stages; ++s) {  // steady: two later stages in flight, one more issued here
        sync_stage(2);
        issue(st0 + s + 3, buffer(s + 3));
        unroll<8>([&](auto X) { read_one(buffer(s), f, X); });
        unroll<4>([&](auto X) { mfma_one(f, X); });
    }
    for (; s < stages; ++s) {  // the last (up to) three stages: nothing more to issue
        sync_stage(stages - s - 1);
        unroll<8>([&](auto X) { read_one(buffer(s), f, X); });
        unroll<4>([&](auto X) { mfma_one(f, X); });
    }
    wait_vmcnt<0>();  // no load may still be writing LDS when the wave ends

    const int64_t wrow0 = m0 + wm * 64, wcol0 = n0 + wn * 64;
    if (to_partial) {
        // split-K: this split's raw accumulators into its slice of the partial sums, [split][m][nb] over the
        // split columns n_lo .. n - 1 (all of n unless whole-K tiles come first)
        typedef typename std::conditional<QT == kInt8, int32_t, float>::type part_t;
        const int64_t n_lo = dp_tiles == 0 ? 0 : (int64_t)(dp_tiles / tiles_m) * BN, nb = n - n_lo;
        part_t *P = static_cast<part_t *>(partial) + (int64_t)split * m * nb;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t col = wcol0 + j * 32 + fr;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                    if (row < m && col < n) P[row * nb + (col - n_lo)] = acc[i][j][e];
                }
            }
        return;
    }

    // epilogue: y = acc * x_scale[row] * w_scale[col], the scales loaded together from clamped indices
    float sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = wcol0 + j * 32 + fr;
        sw[j] = ws[col < n ? col : n - 1];
    }
    // uniform over the workgroup (the barrier below is reached by every wavefront or by none)
    const bool fast = y_bf16 && acc_out == nullptr && (n % 8) == 0 && n0 + BN <= n;
    if (fast) {
        // bf16 tile through LDS: each wave converts its 64 x 64 outputs into its own 8 KiB of the ring (row
        // stride 128 bytes), then writes 16-byte row pieces with buffer stores (rows past m fall outside the
        // buffer and are dropped) instead of scattered 2-byte stores
        constexpr int kStride = 128;
        __syncthreads();  // every wave is done with the ring
        uint8_t *stage = ring + wave * (64 * kStride);
        unroll<2>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float sx[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                sx[e] = xs[row < m ? row : m - 1];
            }
            unroll<2>([&](auto J) {
                constexpr int j = decltype(J)::value;
#pragma unroll
                for (int e = 0; e < 16; e += 2) {  // rows r and r + 1 of the lane's column, one conversion
                    const int r = i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                    const uint32_t p = f32x2_to_bf16x2(acc_to_f32(acc[i][j][e]) * sx[e] * sw[j],
                                                       acc_to_f32(acc[i][j][e + 1]) * sx[e + 1] * sw[j]);
                    uint8_t *q = stage + r * kStride + (j * 32 + fr) * 2;
                    *reinterpret_cast<uint16_t *>(q) = (uint16_t)p;
                    *reinterpret_cast<uint16_t *>(q + kStride) = (uint16_t)(p >> 16);
                }
            });
        });
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(y, (short)0, (int)(m * n * 2), kBufferFlags);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = lane + 64 * q;  // 16-byte piece: row c / 8, columns 8 (c % 8) ..
            const int r = c >> 3, c8 = (c & 7) * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * kStride + c8 * 2);
            const int64_t row = wrow0 + r;
            const uint32_t off = row < m ? (uint32_t)((row * n + wcol0 + c8) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ry, off, 0, 0);
        }
        return;
    }
    unroll<2>([&](auto I) {
        constexpr int i = decltype(I)::value;
        float sx[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
            sx[e] = xs[row < m ? row : m - 1];
        }
        unroll<2>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const int64_t col = wcol0 + j * 32 + fr;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                if (row < m && col < n) {
                    const float v = acc_to_f32(acc[i][j][e]) * sx[e] * sw[j];
                    if (y_bf16)
                        static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(v);
                    else
                        static_cast<float *>(y)[row * n + col] = v;
                    if (acc_out != nullptr) {
                        if constexpr (QT == kInt8)
                            static_cast<int32_t *>(acc_out)[row * n + col] = acc[i][j][e];
                        else
                            static_cast<float *>(acc_out)[row * n + col] = acc[i][j][e];
                    }
                }
            }
        });
    });
}

// ---------------------------------------------------------------------------------------------------------
// Wide-wave GEMM: 256 x 256 outputs per workgroup and 2 x 2 wavefronts of 128 x 128
// outputs each (4 x 4 fragments of the 32x32 MFMA: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit
// block scales, or two v_mfma_i32_32x32x32_i8), 256 accumulators per lane. A wavefront's fragments of one
// 64-byte K step are 8 reads of 2 KiB for 16 MFMAs, half of what the ring kernel's 64 x 64 wavefronts read per
// MFMA, so the LDS carries less per operation. A second form (BN = 160, four wavefronts of 64 x 160 outputs) runs
// the columns past whole CU rounds of 256-wide tiles as one more round of narrower tiles, in a second launch.
// K (a multiple of 128 bytes) advances in 128-byte stages through two LDS buffers. Every thread loads its
// 16-byte pieces of stage s + 1 into registers (raw buffer loads: rows past m or n read as zero) while the MFMAs
// of stage s run, and writes them to the other buffer before the stage's barrier. A buffer holds the stage's 256
// activation rows and its 256 weight rows, 128 bytes each, with logical 16-byte piece c of row r stored at
// physical piece c ^ ((r / 2) mod 8): a fragment read (32 consecutive rows at one logical piece, served 16 lanes
// per cycle over 64 four-byte banks) and a row-major staging write then touch distinct banks. A fragment gives
// lane l row (l & 31) and, for the 64-byte step u of the stage, logical pieces 4 u + 2 (l >> 5) and
// 4 u + 2 (l >> 5) + 1 (FP8, one MFMA of K = 64) or 4 u + (l >> 5) and 4 u + 2 + (l >> 5) (INT8, two MFMAs of
// K = 32), the same for both operands, so the dot products are those of the plain definition. Work items
// (tiles, K splits, whole-K tiles then a split column band) are ordered per XCD as in the ring kernel.
// ---------------------------------------------------------------------------------------------------------
constexpr int kWideK = 128;     // K bytes per stage
constexpr int kWideN = 256;     // weight rows (output channels) per tile
constexpr int kWideBandN = 160; // output channels per tile of the band after whole rounds of 256-wide tiles
constexpr int kWideM = 256;     // activation rows per tile
constexpr int kWideThreads = 256;
constexpr int kWideBuf = (kWideM + kWideN) * kWideK;  // bytes per LDS stage buffer (64 KiB)
constexpr int kWideHalf = kWideM * kWideK;              // one operand's rows of a stage (32 KiB)
constexpr int kWideChunks = kWideM * kWideK / 16 / kWideThreads;  // 16-byte pieces per thread per operand (8)

__device__ __forceinline__ int wide_swizzle(int r) { return (r >> 1) & 7; }

template <int QT, int BN>
__global__ __launch_bounds__(kWideThreads, 1) void gemm_wide_kernel(
    int64_t m, int64_t n, int64_t k, const uint8_t *__restrict__ xq, const float *__restrict__ xs,
    const uint8_t *__restrict__ wq, const float *__restrict__ ws, void *__restrict__ y, int y_bf16,
    void *__restrict__ acc_out, int tiles_m, int tiles_n, int splits, int stages_per_split,
    void *__restrict__ partial, int dp_tiles, int64_t n_base) {
    typedef typename Acc32<QT>::type acc_t;
    // BN = 256: 2 x 2 wavefronts of 128 x 128 outputs; BN = 160 (a band of columns after whole rounds of 256-wide
    // tiles): 4 x 1 wavefronts of 64 x 160
    constexpr int WM = BN == kWideN ? 2 : 4, WN = 4 / WM;
    constexpr int WR = kWideM / WM, WC = BN / WN;               // outputs per wavefront
    constexpr int IA = WR / 32, JB = WC / 32;                   // 32 x 32 fragments per wavefront
    constexpr int CB = BN * kWideK / 16 / kWideThreads;         // weight staging pieces per thread
    constexpr int NS = kWideChunks + CB, NR = 2 * (IA + JB), NM = IA * JB;
    constexpr int NX = NS > NR ? (NS > NM ? NS : NM) : (NR > NM ? NR : NM);
    static_assert(WC % 32 == 0 && (BN * kWideK) % (16 * kWideThreads) == 0 && BN <= kWideN, "tile shape");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];  // two stage buffers of kWideBuf bytes

    // work item: the same order as the ring kernel (each XCD a contiguous run; whole-K tiles first)
    const int tiles = tiles_m * tiles_n;
    const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
    int split = 0, tile;
    bool to_partial;
    if (dp_tiles == 0) {
        const int total = tiles * splits;
        const int per_xcd = (total + 7) / 8;
        const int order = xcd * per_xcd + slot;
        if (order >= total) return;
        split = order / tiles;
        tile = order % tiles;
        to_partial = splits > 1;
    } else {
        const int dpx = dp_tiles / 8;
        if (slot < dpx) {
            tile = xcd * dpx + slot;
            to_partial = false;
        } else {
            const int rem = tiles - dp_tiles, pieces = rem * splits;
            const int p = xcd * ((pieces + 7) / 8) + (slot - dpx);
            if (p >= pieces) return;
            split = p / rem;
            tile = dp_tiles + p % rem;
            to_partial = true;
        }
    }
    const int64_t m0 = (int64_t)(tile % tiles_m) * kWideM;
    const int64_t n0 = n_base + (int64_t)(tile / tiles_m) * BN;
    const int64_t all_stages = (k + kWideK - 1) / kWideK;
    const int64_t st0 = to_partial ? (int64_t)split * stages_per_split : 0;
    const int64_t stages = to_partial ? std::min<int64_t>(stages_per_split, all_stages - st0) : all_stages;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // LDS: stage buffer b holds its activation rows at b * kWideHalf and its weight rows at kWideBuf + b * kWideHalf,
    // so that every access below is a register plus an immediate offset, and moving to the other buffer flips one
    // address bit (kWideHalf) of a few registers once per stage.
    // Staging: piece i of this thread is chunk t + 256 i of the stage, row (t / 8) + 32 i, logical piece t % 8;
    // the row's swizzle (r / 2) mod 8 does not depend on i, so piece i sits 32 rows (4 KiB) after piece 0.
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xq), (short)0,
                                                                         (int)(m * k), kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(wq), (short)0,
                                                                         (int)(n * k), kBufferFlags);
    const int srow = t >> 3, spiece = t & 7;
    const int lds0 = srow * kWideK + 16 * (spiece ^ wide_swizzle(srow));
    const int64_t rows_a = m - m0 - srow, rows_b = n - n0 - srow;  // piece i is in range while 32 i < rows
    // byte offsets of the pieces at K = 0, or kOutOfRange (past every operand) for rows outside the operand
    uint32_t va[kWideChunks], vb[CB];
#pragma unroll
    for (int i = 0; i < kWideChunks; ++i)
        va[i] = 32 * i < rows_a ? (uint32_t)((m0 + srow + 32 * i) * k + 16 * spiece) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < CB; ++i)
        vb[i] = 32 * i < rows_b ? (uint32_t)((n0 + srow + 32 * i) * k + 16 * spiece) : kOutOfRange;
    v4i ra[kWideChunks], rb[CB];
    // staging piece x of global stage gst (x < 8: activations, else weights). K is a whole number of stages here,
    // so the stage's K offset goes in the scalar offset, with no per-lane arithmetic; a row outside the operand
    // stays out of range with or without it.
    auto load_one = [&](int64_t gst, auto X) {
        constexpr int x = decltype(X)::value;
        const int k0 = (int)(gst * kWideK);
        if constexpr (x < 8)
            ra[x] = __builtin_amdgcn_raw_buffer_load_b128(rsa, va[x], k0, 0);
        else
            rb[x - 8] = __builtin_amdgcn_raw_buffer_load_b128(rsb, vb[x - 8], k0, 0);
    };
    // staging piece x into the buffer whose staging addresses are wa (activations) and wb (weights)
    auto store_one = [&](int wa, int wb, auto X) {
        constexpr int x = decltype(X)::value;
        if constexpr (x < 8)
            *reinterpret_cast<v4i *>(lds + wa + 4096 * x) = ra[x];
        else
            *reinterpret_cast<v4i *>(lds + wb + 4096 * (x - 8)) = rb[x - 8];
    };

    acc_t acc[IA][JB];
#pragma unroll
    for (int i = 0; i < IA; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = acc_t{};

    // one 64-byte step u of a stage: 16 fragment reads (lane row (l & 31), half h = l >> 5), 16 MFMA tiles; both
    // split into single instructions so that the pipeline below can interleave them with other memory operations
    const int fr = lane & 31, h = lane >> 5;
    const int q0 = QT == kInt8 ? h : 2 * h, q1 = QT == kInt8 ? 2 + h : 2 * h + 1;
    const int swz = wide_swizzle(fr);  // rows wm 128 + 32 i + fr and 128 wn + 32 j + fr share it
    // the lane's fragment addresses in buffer 0 for step u and piece parity p (the first or second 16 bytes)
    auto frag_a = [&](int u, int p) { return (wm * WR + fr) * kWideK + 16 * ((4 * u + (p ? q1 : q0)) ^ swz); };
    auto frag_b = [&](int u, int p) {
        return kWideBuf + (wn * WC + fr) * kWideK + 16 * ((4 * u + (p ? q1 : q0)) ^ swz);
    };
    struct Frags {
        uint4 a[IA][2], b[JB][2];
    };
    // read x (x = 0..15) at fragment addresses fa, fb: A fragment x / 2 piece x % 2 for x < 8, then B fragment
    // (x - 8) / 2 piece x % 2
    auto read_one = [&](const int (&fa)[2], const int (&fb)[2], Frags &f, auto X) {
        constexpr int x = decltype(X)::value;
        if constexpr (x < 2 * IA)
            f.a[x / 2][x & 1] = *reinterpret_cast<const uint4 *>(lds + fa[x & 1] + (x / 2) * 4096);
        else
            f.b[(x - 2 * IA) / 2][x & 1] = *reinterpret_cast<const uint4 *>(lds + fb[x & 1] + ((x - 2 * IA) / 2) * 4096);
    };
    // MFMA tile x of a step: fragments (x / 4, x % 4)
    auto mfma_one = [&](const Frags &f, auto X) {
        constexpr int x = decltype(X)::value, i = x / JB, j = x % JB;
        if constexpr (QT == kInt8) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4(f.a[i][0]), v4(f.b[j][0]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(v4(f.a[i][1]), v4(f.b[j][1]), acc[i][j], 0, 0, 0);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8(f.a[i][0], f.a[i][1]),
                                                                         v8(f.b[j][0], f.b[j][1]), acc[i][j], 0, 0,
                                                                         0, 127, 0, 127);
        }
    };

    // Pipeline (one wavefront per SIMD, so each wavefront hides its own latencies): stage s + 1 is in the staging
    // registers while stage s runs, and the fragments of one 64-byte step are read while the MFMAs of the other
    // run. Stage s runs in two phases around one barrier:
    //  A: the first step's 16 MFMA tiles, each followed by one of the second step's fragment reads, one write of
    //     the staged stage s + 1 into the other buffer (every wavefront finished reading it before the previous
    //     barrier) and one load of stage s + 2;
    //  the barrier (each wavefront's LDS accesses retired first): stage s's buffer is no longer read and stage
    //     s + 1's is written;
    //  B: the second step's 16 MFMA tiles, each followed by one of stage s + 1's first-step fragment reads.
    // The memory instructions thus issue while the matrix core is busy. Scheduling barriers between the groups
    // keep the compiler from regrouping them; the waits it inserts then cover one group's dependences only.
    // Addresses: c1a / c1b the current buffer's second-step fragments, n0a / n0b the next buffer's first-step
    // fragments, wa / wb the next buffer's staging pieces; all flip to the other buffer after each stage.
    int c1a[2] = {frag_a(1, 0), frag_a(1, 1)}, c1b[2] = {frag_b(1, 0), frag_b(1, 1)};
    int n0a[2] = {frag_a(0, 0) ^ kWideHalf, frag_a(0, 1) ^ kWideHalf};
    int n0b[2] = {frag_b(0, 0) ^ kWideHalf, frag_b(0, 1) ^ kWideHalf};
    int wa = lds0 ^ kWideHalf, wb = (kWideBuf + lds0) ^ kWideHalf;
    auto flip = [&]() {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            c1a[p] ^= kWideHalf;
            c1b[p] ^= kWideHalf;
            n0a[p] ^= kWideHalf;
            n0b[p] ^= kWideHalf;
        }
        wa ^= kWideHalf;
        wb ^= kWideHalf;
    };
    typedef std::integral_constant<bool, true> yes;
    typedef std::integral_constant<bool, false> no;
    Frags f0, f1;
    auto run_stage = [&](int64_t s, auto store_c, auto load_c, auto next_c) {
        constexpr bool kStore = decltype(store_c)::value, kLoad = decltype(load_c)::value,
                       kNext = decltype(next_c)::value;
        unroll<NX>([&](auto X) {
            constexpr int x = decltype(X)::value;
            if constexpr (x < NM) mfma_one(f0, X);
            if constexpr (x < NR) read_one(c1a, c1b, f1, X);
            if constexpr (kStore && x < NS) store_one(wa, wb, X);
            if constexpr (kLoad && x < NS) load_one(st0 + s + 2, X);
            __builtin_amdgcn_sched_barrier(0);
        });
        __syncthreads();
        unroll<NX>([&](auto X) {
            constexpr int x = decltype(X)::value;
            if constexpr (x < NM) mfma_one(f1, X);
            if constexpr (kNext && x < NR) read_one(n0a, n0b, f0, X);
            __builtin_amdgcn_sched_barrier(0);
        });
        flip();
    };
    unroll<NS>([&](auto X) { load_one(st0, X); });
    unroll<NS>([&](auto X) { store_one(lds0, kWideBuf + lds0, X); });
    if (stages > 1) unroll<NS>([&](auto X) { load_one(st0 + 1, X); });
    __syncthreads();
    {
        const int fa[2] = {frag_a(0, 0), frag_a(0, 1)}, fb[2] = {frag_b(0, 0), frag_b(0, 1)};
        unroll<NR>([&](auto X) { read_one(fa, fb, f0, X); });
    }
    int64_t s = 0;
    for (; s + 2 < stages; ++s) run_stage(s, yes{}, yes{}, yes{});  // steady state: stage s + 2 exists
    if (s + 1 < stages) {                                           // the last but one stage: nothing to load
        run_stage(s, yes{}, no{}, yes{});
        ++s;
    }
    run_stage(s, no{}, no{}, no{});  // the last stage
    __syncthreads();  // every fragment read is retired before the epilogue reuses the LDS

    const int64_t wrow0 = m0 + wm * WR, wcol0 = n0 + wn * WC;
    if (to_partial) {
        typedef typename std::conditional<QT == kInt8, int32_t, float>::type part_t;
        const int64_t n_lo = dp_tiles == 0 ? 0 : (int64_t)(dp_tiles / tiles_m) * BN, nb = n - n_lo;
        part_t *P = static_cast<part_t *>(partial) + (int64_t)split * m * nb;
#pragma unroll
        for (int i = 0; i < IA; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int64_t col = wcol0 + j * 32 + fr;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                    if (row < m && col < n) P[row * nb + (col - n_lo)] = acc[i][j][e];
                }
            }
        return;
    }

    // epilogue: y = acc * x_scale[row] * w_scale[col]
    float sw[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        const int64_t col = wcol0 + j * 32 + fr;
        sw[j] = ws[col < n ? col : n - 1];
    }
    const bool fast = y_bf16 && acc_out == nullptr && (n % 8) == 0 && n0 + BN <= n;  // uniform per workgroup
    if (fast) {
        // the wavefront's WR x WC bf16 outputs go through its own WR x 2 WC bytes of LDS (the last barrier of the
        // loop has retired every fragment read), then out as 16-byte row pieces with buffer stores (rows past m
        // fall outside the buffer and are dropped); a wavefront reads back only what it wrote
        constexpr int kStride = 2 * WC, kPieces = WC / 8;  // bytes and 16-byte pieces per staged row
        uint8_t *stage = lds + wave * (WR * kStride);
        unroll<IA>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float sx[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                sx[e] = xs[row < m ? row : m - 1];
            }
            unroll<JB>([&](auto J) {
                constexpr int j = decltype(J)::value;
#pragma unroll
                for (int e = 0; e < 16; e += 2) {  // rows r and r + 1 of the lane's column, one conversion
                    const int r = i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                    const uint32_t p = f32x2_to_bf16x2(acc_to_f32(acc[i][j][e]) * sx[e] * sw[j],
                                                       acc_to_f32(acc[i][j][e + 1]) * sx[e + 1] * sw[j]);
                    uint8_t *q = stage + r * kStride + (j * 32 + fr) * 2;
                    *reinterpret_cast<uint16_t *>(q) = (uint16_t)p;
                    *reinterpret_cast<uint16_t *>(q + kStride) = (uint16_t)(p >> 16);
                }
            });
        });
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(y, (short)0, (int)(m * n * 2), kBufferFlags);
#pragma unroll
        for (int q = 0; q < WR * kPieces / 64; ++q) {
            const int c = lane + 64 * q;  // 16-byte piece: row c / kPieces, columns 8 (c % kPieces) ..
            const int r = c / kPieces, c8 = (c % kPieces) * 8;
            const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * kStride + c8 * 2);
            const int64_t row = wrow0 + r;
            const uint32_t off = row < m ? (uint32_t)((row * n + wcol0 + c8) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ry, off, 0, 0);
        }
        return;
    }
    unroll<IA>([&](auto I) {
        constexpr int i = decltype(I)::value;
        float sx[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
            sx[e] = xs[row < m ? row : m - 1];
        }
        unroll<JB>([&](auto J) {
            constexpr int j = decltype(J)::value;
            const int64_t col = wcol0 + j * 32 + fr;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = wrow0 + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                if (row < m && col < n) {
                    const float v = acc_to_f32(acc[i][j][e]) * sx[e] * sw[j];
                    if (y_bf16)
                        static_cast<uint16_t *>(y)[row * n + col] = f32_to_bf16(v);
                    else
                        static_cast<float *>(y)[row * n + col] = v;
                    if (acc_out != nullptr) {
                        if constexpr (QT == kInt8)
                            static_cast<int32_t *>(acc_out)[row * n + col] = acc[i][j][e];
                        else
                            static_cast<float *>(acc_out)[row * n + col] = acc[i][j][e];
                    }
                }
            }
        });
    });
}

// Split-K: acc = the partial sums of the splits added in split order (exact for INT32; a fixed order for FP32,
// so repeated calls agree bit for bit), then the epilogue y = acc * x_scale[row] * w_scale[col]. The partial
// sums cover the columns n_lo .. n - 1 ([split][m][nb], nb = n - n_lo). Four consecutive outputs per thread
// when nb is a multiple of 4, one otherwise.
template <int QT, int VEC>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int64_t m, int64_t n, int64_t n_lo, int splits,
                                                            const void *__restrict__ partial,
                                                            const float *__restrict__ xs,
                                                            const float *__restrict__ ws, void *__restrict__ y,
                                                            int y_bf16, void *__restrict__ acc_out) {
    typedef typename std::conditional<QT == kInt8, int32_t, float>::type part_t;
    const int64_t nb = n - n_lo;
    const int64_t total = m * nb;
    const part_t *P = static_cast<const part_t *>(partial);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * VEC;
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC; base < total; base += stride) {
        part_t a[VEC];
        if constexpr (VEC == 4) {
            typedef part_t vec_t __attribute__((ext_vector_type(4)));
            auto ld = [&](int sp) {  // read once: non-temporal
                return __builtin_nontemporal_load(reinterpret_cast<const vec_t *>(P + (int64_t)sp * total + base));
            };
            vec_t v = ld(0);
            a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
            int sp = 1;
            for (; sp + 4 <= splits; sp += 4) {  // four loads in flight, then added in split order
                const vec_t v1 = ld(sp), v2 = ld(sp + 1), v3 = ld(sp + 2), v4 = ld(sp + 3);
                a[0] += v1.x; a[1] += v1.y; a[2] += v1.z; a[3] += v1.w;
                a[0] += v2.x; a[1] += v2.y; a[2] += v2.z; a[3] += v2.w;
                a[0] += v3.x; a[1] += v3.y; a[2] += v3.z; a[3] += v3.w;
                a[0] += v4.x; a[1] += v4.y; a[2] += v4.z; a[3] += v4.w;
            }
            for (; sp < splits; ++sp) {
                v = ld(sp);
                a[0] += v.x; a[1] += v.y; a[2] += v.z; a[3] += v.w;
            }
        } else {
            a[0] = P[base];
            for (int sp = 1; sp < splits; ++sp) a[0] += P[(int64_t)sp * total + base];
        }
        const int64_t row = base / nb, col = n_lo + (base - row * nb);
        const float sx = xs[row];
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = acc_to_f32(a[e]) * sx * ws[col + e];
        const int64_t idx = row * n + col;
        if constexpr (VEC == 4) {
            // n and col are multiples of 4 here (nb and n_lo are), so one 8- or 16-byte store per output type
            if (y_bf16) {
                const uint2 o = {f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3])};
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(y) + idx) = o;
            } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(y) + idx) = float4{v[0], v[1], v[2], v[3]};
            }
            if (acc_out != nullptr) {
                typedef part_t vec_t __attribute__((ext_vector_type(4)));
                *reinterpret_cast<vec_t *>(static_cast<part_t *>(acc_out) + idx) = vec_t{a[0], a[1], a[2], a[3]};
            }
        } else {
            if (y_bf16)
                static_cast<uint16_t *>(y)[idx] = f32_to_bf16(v[0]);
            else
                static_cast<float *>(y)[idx] = v[0];
            if (acc_out != nullptr) static_cast<part_t *>(acc_out)[idx] = a[0];
        }
    }
}

template <int QT, int BM, int BN>
hipError_t launch_ring(const GemmPlan &g, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                       const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                       hipStream_t stream) {
    typedef Ring<BM, BN> R;
    const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
    int grid;
    if (g.dp_tiles == 0) {
        grid = ((tiles_m * tiles_n * g.splits + 7) / 8) * 8;
    } else {
        const int pieces = (tiles_m * tiles_n - g.dp_tiles) * g.splits;
        grid = 8 * (g.dp_tiles / 8 + (pieces + 7) / 8);
    }
    hipLaunchKernelGGL((gemm_ring_kernel<QT, BM, BN>), dim3(grid), dim3(R::kThreads), 0, stream, m, n, k, xq, xs,
                       wq, ws, y, y_bf16 ? 1 : 0, acc_out, tiles_m, tiles_n, g.splits, g.stages_per_split,
                       workspace, g.dp_tiles);
    if (g.splits > 1)
        launch_splitk_reduce(QT, m, n, g.splits, workspace, xs, ws, y, y_bf16, acc_out, stream, g.n_lo);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_wide(const GemmPlan &g, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                       const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                       hipStream_t stream) {
    // more than 64 KiB of dynamic LDS per workgroup is opted into once per kernel
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_wide_kernel<QT, kWideN>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kWideBuf);
    static const hipError_t attr_b = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&gemm_wide_kernel<QT, kWideBandN>), hipFuncAttributeMaxDynamicSharedMemorySize,
        2 * kWideBuf);
    if (attr != hipSuccess) return attr;
    if (attr_b != hipSuccess) return attr_b;
    if (k % kWideK != 0) return hipErrorInvalidValue;  // the kernel's loads take whole 128-byte stages
    const int tiles_m = (int)((m + kWideM - 1) / kWideM);
    const int64_t n_main = g.band ? g.band_n0 : n;  // columns of the 256-wide tiles
    if (g.band && (g.splits != 1 || g.dp_tiles != 0 || n_main % kWideN != 0)) return hipErrorInvalidValue;
    const int tiles_n = (int)((n_main + kWideN - 1) / kWideN);
    if (tiles_n > 0) {
        int grid;
        if (g.dp_tiles == 0) {
            grid = ((tiles_m * tiles_n * g.splits + 7) / 8) * 8;
        } else {
            const int pieces = (tiles_m * tiles_n - g.dp_tiles) * g.splits;
            grid = 8 * (g.dp_tiles / 8 + (pieces + 7) / 8);
        }
        hipLaunchKernelGGL((gemm_wide_kernel<QT, kWideN>), dim3(grid), dim3(kWideThreads), 2 * kWideBuf, stream, m, n,
                           k, xq, xs, wq, ws, y, y_bf16 ? 1 : 0, acc_out, tiles_m, tiles_n, g.splits,
                           g.stages_per_split, workspace, g.dp_tiles, (int64_t)0);
    }
    if (g.band) {  // the remaining columns as one round of 256 x kWideBandN tiles over all of K
        const int tiles_b = (int)((n - n_main + kWideBandN - 1) / kWideBandN);
        const int grid = ((tiles_m * tiles_b + 7) / 8) * 8;
        hipLaunchKernelGGL((gemm_wide_kernel<QT, kWideBandN>), dim3(grid), dim3(kWideThreads), 2 * kWideBuf, stream,
                           m, n, k, xq, xs, wq, ws, y, y_bf16 ? 1 : 0, acc_out, tiles_m, tiles_b, 1,
                           (int)((k + kWideK - 1) / kWideK), workspace, 0, n_main);
    }
    if (g.splits > 1)
        launch_splitk_reduce(QT, m, n, g.splits, workspace, xs, ws, y, y_bf16, acc_out, stream, g.n_lo);
    return hipGetLastError();
}

template <int QT, int BM, int BN>
hipError_t launch_t(int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs, const uint8_t *wq,
                    const float *ws, void *y, bool y_bf16, void *acc_out, hipStream_t stream) {
    const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int grid = ((total + 7) / 8) * 8;
    hipLaunchKernelGGL((gemm_tiled_kernel<QT, BM, BN>), dim3(grid), dim3(256), 0, stream, m, n, k, xq, xs, wq, ws, y,
                       y_bf16 ? 1 : 0, acc_out, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_q(const GemmPlan &g, int64_t m, int64_t n, int64_t k, const uint8_t *xq, const float *xs,
                    const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out, void *workspace,
                    hipStream_t stream) {
    switch (g.tile) {
        case kGemmRing:
#define QR_RING(BM_, BN_) launch_ring<QT, BM_, BN_>(g, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream)
            if (g.bm == 128) {
                if (g.bn == 64) return QR_RING(128, 64);
                if (g.bn == 128) return QR_RING(128, 128);
                return QR_RING(128, 256);
            }
            if (g.bn == 64) return QR_RING(256, 64);
            if (g.bn == 128) return QR_RING(256, 128);
            return QR_RING(256, 256);
#undef QR_RING
        case kGemmWide:
            return launch_wide<QT>(g, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
        case 1: return launch_t<QT, 256, 128>(m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, stream);
        case 2: return launch_t<QT, 128, 256>(m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, stream);
        default: return launch_t<QT, 128, 128>(m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, stream);
    }
}

}  // namespace

bool gemm_ring_fits(int64_t m, int64_t n, int64_t k) {
    // every buffer offset of the ring kernel (operands, bf16 output) stays below 2^31
    const int64_t lim = (int64_t)1 << 31;
    return m * k < lim && n * k < lim && m * n * 2 < lim;
}

GemmPlan gemm_plan(int64_t m, int64_t n, int64_t k) {
    GemmPlan g{};
    g.splits = 1;
    auto count = [&](int bm, int bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
    const int forced = env_int("QR_GEMM_TILE", -1);
    const bool ring = gemm_ring_fits(m, n, k) && !(forced >= 1 && forced <= 3);
    if (!ring) {
        if (forced >= 1 && forced <= 3)
            g.tile = forced;
        else
            g.tile = count(256, 128) >= 256 ? 1 : (count(128, 256) >= 256 ? 2 : 3);
        return g;
    }
    // The wide-wave kernel where measured faster than the ring (MI355X, 7B-shaped FP8 linears, weights past the
    // caches): batches above 128 rows with at least 128 output tiles of 256 x 256 or a deep K (gate/up at m = 512
    // 98 -> 92 us and at m = 2048 282 -> 267 us, down 56 -> 54 and 149 -> 133 us, qkv at m = 2048 47 -> 45 us);
    // the ring kernel elsewhere (its 128-row tiles at small batches, and few-tile shapes split over K: qkv and o at
    // m = 512 29 / 27 us against 36 / 33, o at m = 2048 39 against 44 us)
    const bool wide_pays = m > 128 && (count(kWideM, kWideN) >= 128 || k >= 8192);
    g.tile = (forced == kGemmWide || (forced < 0 && wide_pays)) && k % kWideK == 0 ? kGemmWide : kGemmRing;
    // Cost model, fitted to the 7B-shaped FP8 linears at m = 128, 512, 2048 on MI355X: a workgroup takes about
    // 0.65 us per 64 bytes of K with 128 activation rows per tile and 0.83 us with 256; workgroups beyond the
    // 256 CUs run in further rounds; a split adds its partial sums (written and read back, about 5 TB/s) and
    // the reduction launch (about 5 us). The cheapest (rows per tile, splits) wins; splits keep >= 256 bytes of K.
    const int stage_bytes = g.tile == kGemmWide ? kWideK : kRingK;
    const int64_t min_stages = 256 / stage_bytes;
    const int64_t stages = (k + stage_bytes - 1) / stage_bytes;
    const double per64 = (double)stage_bytes / 64.0;
    const int fbm = env_int("QR_GEMM_BM", 0);
    const int fbn = env_int("QR_GEMM_BN", 0);
    const int fs = env_int("QR_GEMM_SPLITS", 0);
    const int64_t forced_sp = fs >= 1 ? std::min<int64_t>(fs, stages) : 0;
    g.bm = (m <= 128 && g.tile != kGemmWide) ? 128 : 256;
    g.bn = 256;
    g.stages_per_split = (int)stages;
    // microseconds per 64 bytes of K of one workgroup, by tile (rows, channels). The narrow ring tiles are
    // scaled from one-round measurements (MI355X, FP8, one 4096-deep tile per CU: 0.47 / 0.64 / 0.88 us for 128 x
    // 64 / 128 / 256, 0.56 / 0.85 / 1.16 us for 256 x 64 / 128 / 256) by the ratio of the fitted 256-channel
    // costs to their one-round figures. They pay where 256-channel tiles leave CUs idle or need many K splits:
    // the 7B qkv and o at m = 128 (21.9 -> 18.1, 21.0 -> 16.7 us) and m = 512 (29.3 -> 24.8, 27.9 -> 24.4 us).
    auto stage_us = [&](int bm, int bn) -> double {
        if (g.tile == kGemmWide) return 0.83;
        if (bn == 256) return bm == 128 ? 0.65 : 0.83;
        if (bn == 128) return bm == 128 ? 0.47 : 0.61;
        return bm == 128 ? 0.35 : 0.40;
    };
    auto tile_ok = [&](int bm, int bn) {
        if ((fbm == 128 || fbm == 256) && fbm != bm) return false;
        if ((fbn == 64 || fbn == 128 || fbn == 256) && fbn != bn) return false;
        if (g.tile == kGemmWide) return bm == kWideM && bn == kWideN;
        return true;
    };
    double best = 1e30;
    for (int bm : {128, 256})
        for (int bn : {256, 128, 64}) {
            if (!tile_ok(bm, bn)) continue;
            const int64_t tiles = count(bm, bn);
            for (int64_t sp = forced_sp ? forced_sp : 1; sp <= (forced_sp ? forced_sp : 16); ++sp) {
                if (!forced_sp && sp > 1 && (stages + sp - 1) / sp < min_stages) break;
                const int64_t sps = (stages + sp - 1) / sp;
                const int64_t used = (stages + sps - 1) / sps;  // no split without a stage
                const int64_t rounds = (tiles * used + 255) / 256;
                double t = (double)rounds * (double)sps * stage_us(bm, bn) * per64;
                if (used > 1) t += 5.0 + (double)used * (double)m * (double)n * 8.0 / 5.0e6;
                if (t < best) {
                    best = t;
                    g.bm = bm;
                    g.bn = bn;
                    g.stages_per_split = (int)sps;
                    g.splits = (int)used;
                }
            }
        }
    // Whole rounds of tiles over all of K, then the remaining tiles (a band of output columns) split over K
    // so that their pieces fill one more round: for tile counts just past a multiple of the CU count (the 7B
    // gate/up at m = 512: 296 tiles of 256 x 256), where the last round would otherwise run few tiles over all
    // of K. Needs the round to hold whole columns of tiles (round mod token tiles = 0).
    const int round = std::max(8, env_int("QR_GEMM_ROUND", 256) / 8 * 8);
    const int fh = env_int("QR_GEMM_HYB", -1);  // -1 automatic, 0 never, >= 2 that many splits where possible
    if (fh != 0 && !(fs >= 1)) {
        for (int bm : {128, 256})
            for (int bn : {256, 128, 64}) {
            if (!tile_ok(bm, bn)) continue;
            const int64_t tm = (m + bm - 1) / bm, tiles = count(bm, bn);
            if (tiles <= round || round % tm != 0 || tiles % round == 0) continue;
            const int64_t dp = tiles / round * round, rem = tiles - dp;
            const int64_t n_lo = dp / tm * bn;
            for (int64_t sp = fh >= 2 ? fh : 2; sp <= (fh >= 2 ? fh : 16); ++sp) {
                const int64_t sps = (stages + sp - 1) / sp;
                const int64_t used = (stages + sps - 1) / sps;
                if (used < 2) break;
                if (fh < 2 && (sps < min_stages || rem * used > round)) continue;
                const double c = stage_us(bm, bn) * per64;
                const double t = (double)(dp / round) * (double)stages * c + (double)((rem * used + round - 1) / round) *
                                 (double)sps * c + 5.0 + (double)used * (double)m * (double)(n - n_lo) * 8.0 / 5.0e6;
                if (fh >= 2 || t < best) {
                    best = fh >= 2 ? -1.0 : t;
                    g.bm = bm;
                    g.bn = bn;
                    g.stages_per_split = (int)sps;
                    g.splits = (int)used;
                    g.dp_tiles = (int)dp;
                    g.n_lo = n_lo;
                }
            }
        }
    }
    // The wide kernel over all of K in whole rounds of 256-wide tiles, then the remaining columns as one round of
    // 256 x 160 tiles in a second launch (the columns from band_n0). The cost model takes a band round at 0.7 of
    // a full one, fitted on MI355X (7B FP8, graph replay, weights past the caches: gate/up at m = 2048 254 ->
    // 251 us, qkv 42.0 -> 40.5, o 36.2 (ring) -> 32.9, gate/up at m = 512 90.7 (split band) -> 87.2; the
    // deep-K down and the few-tile qkv and o at m = 512 stay on their plans).
    // At 64 < m <= 128 (one token tile, the ring kernel's 128-row tiles otherwise) only a band that fills at
    // least three quarters of a round over a K of at least 2048 bytes, where the cost model's factor does not
    // hold (7B gate/up at m = 128, FP8: 45.2 -> 41.4 us, INT8 47 -> 44; the 1.5B gate/up, 112 band tiles over
    // K = 1536: 15.1 -> 18.6, not taken).
    const int fband = env_int("QR_GEMM_BAND", -1);  // -1 by the cost model, 0 never, 1 wherever it applies
    const bool band_forced_off = fband == 0 || fs > 1 || fh >= 2 || (forced >= 0 && forced != kGemmWide) ||
                                 (fbn != 0 && fbn != kWideN) || (fbm != 0 && fbm != kWideM);
    if (!band_forced_off && (m > 64 || fband == 1) && k % kWideK == 0) {
        const int64_t tm = (m + kWideM - 1) / kWideM, tiles = count(kWideM, kWideN);
        if (tiles % round != 0 && round % tm == 0) {
            const int64_t n0b = tiles / round * round / tm * kWideN;
            const int64_t band_tiles = tm * ((n - n0b + kWideBandN - 1) / kWideBandN);
            const int64_t wstages = (k + kWideK - 1) / kWideK;
            const double c = 0.83 * (double)kWideK / 64.0 * (double)wstages;  // one round of 256-wide tiles
            const double t = (double)(tiles / round) * c + 0.7 * c;
            const bool small_ok = m > 128 || (4 * band_tiles >= 3 * round && k >= 2048);
            if (n0b < n && band_tiles <= round && (fband == 1 || (small_ok && t < best))) {
                g = GemmPlan{};
                g.tile = kGemmWide;
                g.bm = kWideM;
                g.bn = kWideN;
                g.splits = 1;
                g.stages_per_split = (int)wstages;
                g.band = true;
                g.band_n0 = n0b;
            }
        }
    }
    g.ws_bytes = g.splits > 1 ? (size_t)g.splits * (size_t)m * (size_t)(n - g.n_lo) * 4 : 0;
    return g;
}

void launch_splitk_reduce(int qtype, int64_t m, int64_t n, int splits, const void *partial, const float *xs,
                          const float *ws, void *y, bool y_bf16, void *acc_out, hipStream_t stream, int64_t n_lo) {
    const int64_t total_out = m * (n - n_lo);
    const bool vec = ((n - n_lo) % 4) == 0;
    const int64_t items = vec ? total_out / 4 : total_out;
    const int blocks = (int)std::min<int64_t>((items + 255) / 256, 65536);  // about one item per thread
#define QR_REDUCE(QT, V)                                                                                       \
    hipLaunchKernelGGL((splitk_reduce_kernel<QT, V>), dim3(blocks), dim3(256), 0, stream, m, n, n_lo, splits, partial, \
                       xs, ws, y, y_bf16 ? 1 : 0, acc_out)
    if (qtype == kInt8) {
        if (vec) QR_REDUCE(kInt8, 4); else QR_REDUCE(kInt8, 1);
    } else {
        if (vec) QR_REDUCE(kFp8, 4); else QR_REDUCE(kFp8, 1);
    }
#undef QR_REDUCE
}

hipError_t launch_gemm(const GemmPlan &g, int qtype, int64_t m, int64_t n, int64_t k, const uint8_t *xq,
                       const float *xs, const uint8_t *wq, const float *ws, void *y, bool y_bf16, void *acc_out,
                       void *workspace, hipStream_t stream) {
    if (qtype == kInt8) return launch_q<kInt8>(g, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
    return launch_q<kFp8>(g, m, n, k, xq, xs, wq, ws, y, y_bf16, acc_out, workspace, stream);
}

}  // namespace qr
