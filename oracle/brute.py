"""Exact-arithmetic brute force of the quantized-actor linear, for tiny inputs (test infrastructure only).

Every value is a ``fractions.Fraction``; each fp32 operation of the method is modelled as the exact result
followed by one explicit rounding to the nearest binary32 value (ties to even), written here from the IEEE 754
definition. The FP8 code set is enumerated from the floating-point format of "QuRL: Efficient Reinforcement
Learning with Quantized Rollout", section 3, Eq. (2), with 4 exponent and 3 mantissa bits (OCP E4M3FN: bias 7,
no infinity, 0x7F/0xFF NaN). Nothing here calls the C oracle; tests compare the two.
"""
from fractions import Fraction
import math
import struct

QMAX = {0: 127, 1: 448}  # INT8, FP8


def f32_value(x: float) -> Fraction:
    """Exact value of a Python float that holds an fp32 number."""
    return Fraction(x)


def _floor_log2(a: Fraction) -> int:
    """Largest e with 2^e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_f32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value, ties to even (24-bit significand, smallest
    normal 2^-126, subnormal quantum 2^-149). Overflow is not modelled (the path never approaches it)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 23)
    n = round(a / quantum)  # Fraction.__round__ rounds half to even
    return sign * n * quantum


def round_bf16_signed_sqrt(sign: int, v2: Fraction) -> Fraction:
    """The bfloat16 value nearest to sign * sqrt(v2) for a rational v2 >= 0, ties to even (8-bit significand,
    smallest normal 2^-126, subnormal quantum 2^-133), decided by exact comparisons of squares, so no square
    root is ever rounded. Overflow is not modelled."""
    if v2 == 0:
        return Fraction(0)
    e = max(_floor_log2(v2) // 2, -126)  # 2^(2e) <= v2 < 2^(2e + 2): the binade of sqrt(v2)
    quantum = Fraction(2) ** (e - 7)
    t = v2 / quantum ** 2  # (sqrt(v2) / quantum)^2
    n = math.isqrt(t.numerator // t.denominator)  # floor(sqrt(t))
    mid2 = Fraction(2 * n + 1, 2) ** 2
    if t > mid2 or (t == mid2 and n % 2 == 1):
        n += 1
    return sign * n * quantum


def rmsnorm_row(x, gamma, eps):
    """RMSNorm of one row, exactly rounded: bf16(x_j gamma_j / sqrt(sum x^2 / K + eps)) for Python floats that
    hold bfloat16 (x) and fp32 (gamma, eps) values; 0 where x_j gamma_j = 0 or the radicand is 0."""
    xs = [f32_value(v) for v in x]
    D = sum(v * v for v in xs) / len(xs) + f32_value(eps)
    out = []
    for v, g in zip(xs, gamma):
        p = v * f32_value(g)
        out.append(Fraction(0) if p == 0 or D == 0 else round_bf16_signed_sqrt(1 if p > 0 else -1, p * p / D))
    return out


def neg_zero_sign(x: float) -> bool:
    """True for a negative number or -0.0."""
    return struct.pack(">f", x)[0] & 0x80 != 0


def e4m3_values():
    """Exact values of the 127 non-negative finite E4M3 codes 0x00..0x7E, by Eq. (2)."""
    out = []
    for c in range(127):
        E, F = (c >> 3) & 15, c & 7
        if E == 0:
            out.append(Fraction(F, 8) * Fraction(2) ** -6)
        else:
            out.append((1 + Fraction(F, 8)) * Fraction(2) ** (E - 7))
    return out


_E4M3 = e4m3_values()


def e4m3_decode(code: int) -> Fraction:
    mag = _E4M3[code & 0x7F]
    return -mag if code & 0x80 else mag


def e4m3_encode(v: Fraction, negative: bool) -> int:
    """Nearest code to |v| <= 448 by scanning every magnitude; ties to the even code; sign bit from
    ``negative`` (so -0 encodes as 0x80)."""
    a = abs(v)
    best, best_d = None, None
    for c, val in enumerate(_E4M3):
        d = abs(val - a)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if negative else 0)


def quantize_row(row, qtype, s=None, recip=False):
    """Quantize one row of fp32 values (Python floats). ``s`` optional invariant scale; ``recip`` selects
    x * fl32(1/s) (activations) instead of w * s (weights). Returns (codes, scale as Fraction)."""
    qmax = QMAX[qtype]
    wp = []
    neg = []
    for j, x in enumerate(row):
        v = f32_value(x)
        is_neg = neg_zero_sign(x)
        if s is not None:
            sj = f32_value(s[j])
            factor = round_f32(1 / sj) if recip else sj
            v = round_f32(v * factor)
            is_neg = is_neg != (factor < 0)
        wp.append(v)
        neg.append(is_neg if v == 0 else v < 0)
    a = max((abs(v) for v in wp), default=Fraction(0))
    S = round_f32(a / qmax)
    if S == 0:  # all-zero row, or a scale that underflows: replaced by 1
        S = Fraction(1)
    codes = []
    for v, is_neg in zip(wp, neg):
        q = round_f32(v / S)
        q = max(-qmax, min(qmax, q))
        if qtype == 0:
            codes.append(int(round(q)) & 0xFF)
        else:
            codes.append(e4m3_encode(q, is_neg))
    return codes, S


def code_value(code: int, qtype: int) -> Fraction:
    code = int(code)
    if qtype == 0:
        return Fraction(code - 256 if code >= 128 else code)
    return e4m3_decode(code)


def linear(qtype, x_codes, x_scales, w_codes, w_scales):
    """Exact accumulators and exact outputs: acc[m][n] = sum_k x*w (codes decoded exactly) and
    y = acc * S_x[m] * S_w[n], all as Fractions."""
    acc, y = [], []
    for i, xr in enumerate(x_codes):
        ar, yr = [], []
        for c, wr in enumerate(w_codes):
            a = sum((code_value(p, qtype) * code_value(q, qtype) for p, q in zip(xr, wr)), Fraction(0))
            ar.append(a)
            yr.append(a * Fraction(x_scales[i]) * Fraction(w_scales[c]))
        acc.append(ar)
        y.append(yr)
    return acc, y


# ---- next row: W4A16 ------------------------------------------------------------------------------------
def quantize_w4_row(row, group, s=None):
    """Group-wise symmetric INT4 codes of one row of fp32 values (Python floats): per group of ``group``
    channels, S = fl32(max|w'| / 7) (1 when zero), q = nearest integer of fl32(w' / S), ties to even, clamped
    to [-7, 7]; w' = fl32(w * s_j) with an invariant scale. Returns (list of ints, list of Fraction scales)."""
    qs, scales = [], []
    for g0 in range(0, len(row), group):
        wp = []
        for j in range(g0, g0 + group):
            v = f32_value(row[j])
            if s is not None:
                v = round_f32(v * f32_value(s[j]))
            wp.append(v)
        S = round_f32(max(abs(v) for v in wp) / 7)
        if S == 0:
            S = Fraction(1)
        scales.append(S)
        for v in wp:
            q = round_f32(v / S)
            q = max(Fraction(-7), min(Fraction(7), q))
            qs.append(int(round(q)))
    return qs, scales


def w4a16_linear(x_rows, w_codes, w_scales, group):
    """Exact y[m][n] = sum_g S[n][g] * sum_{j in g} x[m][j] * q[n][j] (x given as exact values), as Fractions."""
    y = []
    for xr in x_rows:
        yr = []
        for qr, sr in zip(w_codes, w_scales):
            acc = Fraction(0)
            for g, S in enumerate(sr):
                acc += S * sum((Fraction(xr[j]) * qr[j] for j in range(g * group, (g + 1) * group)), Fraction(0))
            yr.append(acc)
        y.append(yr)
    return y
