// qr_device.hpp -- device-side helpers shared by the gfx950 kernels of libqr.so.
//
// Codecs, the per-row division, wavefront reductions and MFMA wrappers. gfx950 (CDNA4) only: wave64,
// v_mfma_i32_16x16x64_i8 for INT8 and v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit scales) for FP8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kInt8 = 0;
constexpr int kFp8 = 1;

// ---------------------------------------------------------------------------------------------------------
// bfloat16 <-> fp32
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bfloat16 bits, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 -> bfloat16 bits in one hardware conversion (v_cvt_pk_bf16_f32: round to nearest even, the same bits
// as f32_to_bf16 for finite values): a in the low half, b in the high half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, b2_t));
}

// double -> bfloat16 bits with one rounding (nearest even). The conversion to fp32 is made round-to-odd
// (truncate, then set the last bit when inexact); rounding that 24-bit value to nearest even at 8 bits then
// equals the direct rounding because 24 >= 8 + 2 (S. Boldo, G. Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", IEEE Trans. Computers 57(4), 2008).
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(d)) u -= 1u;  // the neighbour toward zero (sign and magnitude bits)
        f = __uint_as_float(u | 1u);
    }
    return f32_to_bf16(f);
}

// ---------------------------------------------------------------------------------------------------------
// Correctly rounded w / S for a whole row with one reciprocal.
//
// r = RN(1/S) is computed once per row with IEEE division. Then q = RN(w*r) is within one ulp of w/S, the
// remainder e = w - q*S is exact when formed by one fused multiply-add, and RN(q + e*r) is the correctly
// rounded quotient (P. Markstein, "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990; also Muller et al., Handbook of Floating-Point Arithmetic,
// section on division with an FMA). The theorem needs the remainder to stay in the normal range, so callers
// use it only for rows whose scale S is at least 2^-90; smaller rows take the IEEE division.
// For w = -0 the last step returns +0 (fma(+0, r, -0) = +0), so the quotient takes the sign of w, which is
// the sign of w / S for S > 0 (FP8 codes keep the sign of zero).
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float div_by_scale(float w, float S, float r) {
    float q = w * r;
    float e = __builtin_fmaf(-q, S, w);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), w);
}

// ---------------------------------------------------------------------------------------------------------
// Code encoders. Inputs are already clamped to [-qmax, qmax].
// ---------------------------------------------------------------------------------------------------------

// INT8: round half to even (v_rndne_f32), then the exact integer conversion.
__device__ __forceinline__ uint32_t encode_int8(float v) {
    return (uint32_t)(int32_t)__builtin_rintf(v) & 0xFFu;
}

// FP8 E4M3FN, nearest value with ties to the even mantissa, sign of zero kept. |v| <= 448.
// The gfx950 conversion v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even under the default rounding mode)
// gives exactly these codes: on the MI355X it was compared with a bit-level encoder (rounding the 23-bit fp32
// mantissa to 3 bits, subnormal targets by an fp32 addition of 2^14) on every fp32 bit pattern clamped to
// [-448, 448], and agreed on all 4278190082 non-NaN ones; that encoder agreed with the reference on every
// rounding case (sign, exponent, the kept mantissa bits, the round bit and the sticky bits).
__device__ __forceinline__ uint32_t encode_e4m3(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}

template <int QT>
__device__ __forceinline__ uint32_t encode_code(float v) {
    if constexpr (QT == kInt8) {
        return encode_int8(v);
    } else {
        return encode_e4m3(v);
    }
}

// four codes packed into a word, v[0] in the low byte (FP8: two pack-conversions of two values each)
template <int QT>
__device__ __forceinline__ uint32_t encode_code4(const float *v) {
    if constexpr (QT == kInt8) {
        return encode_int8(v[0]) | (encode_int8(v[1]) << 8) | (encode_int8(v[2]) << 16) | (encode_int8(v[3]) << 24);
    } else {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    }
}

template <int QT>
struct QMax;
template <>
struct QMax<kInt8> {
    static constexpr float value = 127.0f;
};
template <>
struct QMax<kFp8> {
    static constexpr float value = 448.0f;
};

// ---------------------------------------------------------------------------------------------------------
// Wavefront reductions (wave64).
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------------------------------------
// MFMA on 64-byte K chunks.
//
// Both operands use the same lane map: lane l supplies row (l & 15) of its operand (an activation row for A,
// a weight row = output channel for B) and 16 (INT8) or 32 (FP8) consecutive K bytes chosen by (l >> 4).
// Because A and B are addressed identically, the K permutation inside one instruction does not change the
// dot products. The 16x16 result C[i][j] sits in lane (j + 16 * (i / 4)), element (i % 4).
//
// mma_k64(acc, a[4], b[4]): acc += A(16 x 256) * B(256 x 16)^T using four 64-byte K sub-chunks per lane.
// ---------------------------------------------------------------------------------------------------------
template <int QT>
struct Acc;
template <>
struct Acc<kInt8> {
    typedef v4i type;
};
template <>
struct Acc<kFp8> {
    typedef v4f type;
};

__device__ __forceinline__ void mma_step(v4i &acc, const uint4 *a, const uint4 *b) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        v4i av = {(int)a[t].x, (int)a[t].y, (int)a[t].z, (int)a[t].w};
        v4i bv = {(int)b[t].x, (int)b[t].y, (int)b[t].z, (int)b[t].w};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ void mma_step(v4f &acc, const uint4 *a, const uint4 *b) {
#pragma unroll
    for (int t = 0; t < 4; t += 2) {
        v8i av = {(int)a[t].x, (int)a[t].y, (int)a[t].z, (int)a[t].w,
                  (int)a[t + 1].x, (int)a[t + 1].y, (int)a[t + 1].z, (int)a[t + 1].w};
        v8i bv = {(int)b[t].x, (int)b[t].y, (int)b[t].z, (int)b[t].w,
                  (int)b[t + 1].x, (int)b[t + 1].y, (int)b[t + 1].z, (int)b[t + 1].w};
        // format 0 = E4M3 for both operands; scale exponents 127 = 2^0 (no block scaling)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
    }
}

__device__ __forceinline__ float acc_to_f32(int a) { return (float)a; }
__device__ __forceinline__ float acc_to_f32(float a) { return a; }

// ---------------------------------------------------------------------------------------------------------
// Changed-code counting, four code bytes at a time
// ---------------------------------------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------------------------------------
// Buffer loads straight into LDS (the compiler does not track them: kernels count them with vmcnt themselves)
// ---------------------------------------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;          // raw buffer descriptor word 3 (32-bit untyped data)
constexpr uint32_t kOutOfRange = 0x80000000u;      // a buffer offset past every operand (they stay below 2 GiB)

// One 16-byte-per-lane buffer load straight into LDS: lane l's 16 bytes land at lds_base + 16 l. Issued as
// assembly so that the compiler neither tracks it nor inserts its own waits for the LDS it writes: the kernel
// counts these loads itself (vmcnt) and orders them with the workgroup barrier. M0 (the LDS base register)
// is restored afterwards.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_base, uint32_t voffset) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voffset), "s"(rsrc)
        : "memory");
}

// Raw buffer descriptor (32-bit untyped elements, no stride): base, num_records bytes; loads at offsets
// >= num_records return zero.
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(b & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = kBufferFlags;
    return r;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
// LDS address of a wave-uniform pointer, as a scalar
__device__ __forceinline__ uint32_t lds_addr(uint8_t *p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)(lds_u8_t *)p);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt with the vector-memory counter at N and the LDS counter at zero
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// workgroup barrier that the compiler may not move memory accesses across (the loads into LDS it cannot see
// are ordered by it)
__device__ __forceinline__ void barrier_fenced() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One 4-byte-per-lane buffer load straight into LDS: lane l's 4 bytes land at lds_base + 4 l (as dma16).
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds_base, uint32_t voffset) {
    int saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(voffset), "s"(rsrc)
        : "memory");
}

}  // namespace qr
