"""Pins of the oracle's per-row absmax quantizer (weights and activations) against exact brute force,
closed-form worked cases, invariants and the round-trip error bound. CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from oracle import core as O
from quantized_rollout_amd import synth

QT = [O.INT8, O.FP8]


def _decode(codes, qtype):
    if qtype == O.INT8:
        return codes.view(np.int8).astype(np.float64)
    return O.e4m3_decode(codes)


def _rand_rows(rng, rows, k, scale=1.0):
    return (rng.standard_normal((rows, k)) * scale).astype(np.float32)


@pytest.mark.parametrize("qtype", QT)
@pytest.mark.parametrize("mode", ["none", "w", "x"])
def test_quantizer_matches_exact_brute_force(qtype, mode):
    rng = np.random.default_rng(10 + qtype)
    x = _rand_rows(rng, 6, 16, 0.02)
    x[1, 3] *= 20          # an outlier channel
    x[2] = 0.0             # all-zero row
    x[3, :8] = -x[3, :8]   # mixed signs
    x[4, 5] = -0.0
    s = rng.uniform(0.5, 2.0, 16).astype(np.float32) if mode != "none" else None
    s_mode = {"none": None, "w": O.S_MUL, "x": O.S_MUL_RECIP}[mode]
    codes, scales = O.quantize_rows(x, qtype, s=s, s_mode=s_mode)
    for r in range(x.shape[0]):
        bc, bs = brute.quantize_row([float(v) for v in x[r]], qtype,
                                    None if s is None else [float(v) for v in s], recip=(mode == "x"))
        assert Fraction(float(scales[r])) == bs, (r, scales[r], bs)
        assert list(codes[r]) == bc, (r, list(codes[r]), bc)


@pytest.mark.parametrize("qtype", QT)
def test_quantizer_near_ties_match_brute_force(qtype):
    """Values placed on and one ulp around rounding boundaries of w / S, where a wrong division or a wrong
    tie rule would change a code."""
    qmax = O.QMAX[qtype]
    rng = np.random.default_rng(20 + qtype)
    rows = []
    for _ in range(4):
        amax = np.float32(rng.uniform(0.01, 0.05))
        S = np.float32(amax / np.float32(qmax))
        row = [amax]
        if qtype == O.INT8:
            targets = [j + 0.5 for j in range(-5, 5)]
        else:
            mags = O.e4m3_decode(np.arange(126, dtype=np.uint8))
            targets = list((mags[10:20] + mags[11:21]) / 2)
        for t in targets:
            base = np.float32(np.float64(t) * np.float64(S))
            row += [base, np.nextafter(base, np.float32(1)), np.nextafter(base, np.float32(-1))]
        rows.append(row[:31] + [np.float32(0)] * (32 - len(row[:31])))
    x = np.array(rows, np.float32)
    codes, scales = O.quantize_rows(x, qtype)
    for r in range(x.shape[0]):
        bc, bs = brute.quantize_row([float(v) for v in x[r]], qtype)
        assert Fraction(float(scales[r])) == bs
        assert list(codes[r]) == bc


@pytest.mark.parametrize("qtype", QT)
def test_bf16_input_equals_widened_fp32(qtype):
    rng = np.random.default_rng(3)
    x = _rand_rows(rng, 5, 48, 0.02)
    xb = synth.f32_to_bf16_bits(x)
    c1, s1 = O.quantize_rows(xb, qtype)
    c2, s2 = O.quantize_rows(synth.bf16_bits_to_f32(xb), qtype)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_worked_case_unit_scale_int8():
    """A row whose largest magnitude is exactly 127 has S = 127/127 = 1, so the codes are the values
    rounded half-to-even: 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, 0.49 -> 0, -126.5 -> -126."""
    row = np.array([[127.0, 2.5, 3.5, -2.5, 0.49, -126.5, 1.0, -127.0] + [0.0] * 8], np.float32)
    codes, scales = O.quantize_rows(row, O.INT8)
    assert scales[0] == 1.0
    assert list(codes[0].view(np.int8)[:8]) == [127, 2, 4, -2, 0, -126, 1, -127]


def test_worked_case_unit_scale_fp8():
    """Largest magnitude 448 gives S = 1; the codes are then the E4M3 encodings of the values."""
    row = np.array([[448.0, 1.0, -1.5, 240.0, 250.0, 2.0 ** -9, -(2.0 ** -10), 0.0] + [0.0] * 8], np.float32)
    codes, scales = O.quantize_rows(row, O.FP8)
    assert scales[0] == 1.0
    # 250 lies between 240 (0x77) and 256 (0x78), nearer to 256; 2^-10 is a tie between 0 and 2^-9 -> 0
    assert list(codes[0][:8]) == [0x7E, 0x38, 0xBC, 0x77, 0x78, 0x01, 0x80, 0x00]


@pytest.mark.parametrize("qtype", QT)
def test_integer_multiples_of_scale_round_trip(qtype):
    """w = S * j for representable codes j: dequantization returns w exactly."""
    S = np.float32(2.0 ** -7)
    if qtype == O.INT8:
        j = np.array([127, -127, 5, -64, 0, 33, 100, -1] * 2, np.float64)
    else:
        j = O.e4m3_decode(np.array([0x7E, 0xFE, 0x38, 0x01, 0x4C, 0xC4, 0x20, 0x00] * 2, np.uint8))
    w = (j * float(S)).astype(np.float32)[None, :]
    codes, scales = O.quantize_rows(w, qtype)
    assert scales[0] == S
    assert np.array_equal(_decode(codes[0], qtype) * float(S), w[0].astype(np.float64))


@pytest.mark.parametrize("qtype", QT)
def test_invariants_max_code_sign_symmetry_monotone(qtype):
    rng = np.random.default_rng(4)
    x = _rand_rows(rng, 32, 64, 0.02)
    codes, scales = O.quantize_rows(x, qtype)
    vals = _decode(codes, qtype)
    qmax = O.QMAX[qtype]
    # a nonzero row reaches the largest code
    assert np.all(np.abs(vals).max(axis=1) == qmax)
    # Q(-W) = -Q(W): the sign bit flips (INT8: two's-complement negation), scales unchanged
    cn, sn = O.quantize_rows(-x, qtype)
    assert np.array_equal(sn, scales)
    if qtype == O.INT8:
        assert np.array_equal(cn.view(np.int8), -codes.view(np.int8))
    else:
        assert np.array_equal(cn, codes ^ 0x80)
    # codes are monotone in the value within a row
    for r in range(x.shape[0]):
        order = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(vals[r][order]) >= 0)


@pytest.mark.parametrize("qtype", QT)
def test_all_zero_row(qtype):
    codes, scales = O.quantize_rows(np.zeros((2, 32), np.float32), qtype)
    assert np.all(scales == 1.0) and np.all(codes == 0)


@pytest.mark.parametrize("qtype", QT)
def test_underflowing_scale_is_replaced_by_one(qtype):
    """A row of fp32 subnormals whose max / qmax rounds to 0 gets S = 1: codes are signed zeros (FP8) or 0
    (INT8), matching the exact brute force; a row just large enough for a nonzero S keeps it."""
    tiny = np.float32(2.0 ** -149)
    row = (np.array([3, -3, 1, -1, 0, 2, -2, 3] * 2, np.float32) * tiny)[None, :]
    codes, scales = O.quantize_rows(row, qtype)
    assert scales[0] == 1.0
    if qtype == O.INT8:
        assert np.all(codes == 0)
    else:
        assert list(codes[0][:8]) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x00, 0x80, 0x00]
    bc, bs = brute.quantize_row([float(v) for v in row[0]], qtype)
    assert bs == 1 and list(codes[0]) == bc
    big = (np.float32(2.0 ** -120) * np.arange(1, 17, dtype=np.float32))[None, :]
    c2, s2 = O.quantize_rows(big, qtype)
    assert s2[0] != 1.0 and s2[0] > 0


@pytest.mark.parametrize("qtype", QT)
@pytest.mark.parametrize("with_s", [False, True])
def test_round_trip_error_bound(qtype, with_s):
    """INT8: |S q - w'| <= S/2 (plus fp32 slack); FP8: at most half an E4M3 step of v = w'/S, i.e.
    S * max(|v| * 2^-4, 2^-10) (QuRL section 4.3: quantization error ~ |theta| / 2^b)."""
    rng = np.random.default_rng(5)
    x = _rand_rows(rng, 64, 256, 0.02)
    x[:, 7] *= 20
    s = rng.uniform(0.5, 2.0, 256).astype(np.float32) if with_s else None
    codes, scales = O.quantize_rows(x, qtype, s=s)
    wp = x.astype(np.float64) if s is None else (x * s).astype(np.float32).astype(np.float64)
    S = scales.astype(np.float64)[:, None]
    err = np.abs(_decode(codes, qtype) * S - wp)
    slack = 4 * np.abs(wp) * 2.0 ** -24
    if qtype == O.INT8:
        assert np.all(err <= S / 2 + slack)
    else:
        v = np.abs(wp) / S
        assert np.all(err <= S * np.maximum(v * 2.0 ** -4, 2.0 ** -10) + slack)


@pytest.mark.parametrize("qtype", QT)
def test_power_of_two_invariant_scale_is_exact(qtype):
    """A uniform s = 2^j commutes with every rounding: weights give identical codes and S * 2^j,
    activations identical codes and S * 2^-j."""
    rng = np.random.default_rng(6)
    x = _rand_rows(rng, 16, 64, 0.02)
    c0, s0 = O.quantize_rows(x, qtype)
    for j in (-3, 1, 4):
        s = np.full(64, 2.0 ** j, np.float32)
        cw, sw = O.quantize_rows(x, qtype, s=s, s_mode=O.S_MUL)
        assert np.array_equal(cw, c0) and np.array_equal(sw, (s0 * np.float32(2.0 ** j)))
        cx, sx = O.quantize_rows(x, qtype, s=s, s_mode=O.S_MUL_RECIP)
        assert np.array_equal(cx, c0) and np.array_equal(sx, (s0 * np.float32(2.0 ** -j)))


def _transform_bound_check(qtype, X, W, s_w, s_x):
    """The oracle's quantized product of X diag(1/s_x) and W diag(s_w) against the exact X W^T: returns the
    largest |y - (X W^T)[i,c]| / bound over all outputs, where bound is the closed-form quantization error of
    the transformed operands (P3 per element, plus the fp32 rounding of the transformed values)."""
    xc, xs = O.quantize_rows(X, qtype, s=s_x, s_mode=O.S_MUL_RECIP)
    wc, ws = O.quantize_rows(W, qtype, s=s_w, s_mode=O.S_MUL)
    _, _, acc = O.linear(qtype, xc, xs, wc, ws, O.F32)
    xp = X.astype(np.float64) / s_x.astype(np.float64)   # the exact transformed operands
    wp = W.astype(np.float64) * s_w.astype(np.float64)

    def delta(v, S):
        if qtype == O.INT8:
            return np.full_like(v, 0.5) * S[:, None]
        return np.maximum(np.abs(v / S[:, None]) * 2.0 ** -4, 2.0 ** -10) * S[:, None]

    dx, dw = delta(xp, xs.astype(np.float64)), delta(wp, ws.astype(np.float64))
    worst = 0.0
    for i in range(X.shape[0]):
        for c in range(W.shape[0]):
            exact = sum(Fraction(float(X[i, j])) * Fraction(float(W[c, j])) for j in range(X.shape[1]))
            y = Fraction(float(acc[i, c])) * Fraction(float(xs[i])) * Fraction(float(ws[c]))
            bound = float(np.sum(np.abs(xp[i]) * dw[c] + np.abs(wp[c]) * dx[i] + dx[i] * dw[c]))
            bound += float(np.sum(np.abs(xp[i] * wp[c]))) * 2.0 ** -21  # fp32 rounding of x / s and w s
            worst = max(worst, abs(float(y - exact)) / bound)
    return worst


@pytest.mark.parametrize("qtype", QT)
def test_unquantized_product_invariant_under_transform(qtype):
    """X W^T = (X diag(1/s)) (W diag(s))^T exactly (QuRL section 4.3), in rational arithmetic; and the oracle's
    quantized product with the transform folded into both quantizers stays within the closed-form quantization
    error of the transformed operands from that exact product. The same s on the wrong side (W diag(1/s)) is far
    outside the bound."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 32)).astype(np.float32)
    X[:, 5] *= np.float32(20)
    W = (rng.standard_normal((4, 32)) * 0.02).astype(np.float32)
    s = rng.uniform(0.5, 2, 32).astype(np.float32)
    for i in range(3):
        for c in range(4):
            lhs = sum(Fraction(float(X[i, j])) * Fraction(float(W[c, j])) for j in range(32))
            rhs = sum((Fraction(float(X[i, j])) / Fraction(float(s[j]))) *
                      (Fraction(float(W[c, j])) * Fraction(float(s[j]))) for j in range(32))
            assert lhs == rhs
    assert _transform_bound_check(qtype, X, W, s, s) <= 1.0
    assert _transform_bound_check(qtype, X, W, (1.0 / s).astype(np.float32), s) > 1.0


def test_int8_range_is_symmetric():
    """-128 is never produced (codes stay in [-127, 127], so |acc| <= k * 127^2)."""
    rng = np.random.default_rng(8)
    x = _rand_rows(rng, 64, 128)
    codes, _ = O.quantize_rows(x, O.INT8)
    assert codes.view(np.int8).min() >= -127
