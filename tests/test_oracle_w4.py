"""Pins of the W4A16 oracle (the next row after the W8A8 path: group-wise INT4 weights, bfloat16 activations,
"QaRL: Rollout-Aligned Quantization-Aware RL ...", section 3.1 with the integer Quant of section 2.2).

Against: the exact-arithmetic brute force (independent code), the round-trip bound of the integer quantizer,
invariants (a code of magnitude 7 in every nonzero group, sign symmetry, power-of-two invariant scale), the
nibble packing written out by hand, and closed forms of the product."""
import numpy as np

from oracle import brute as B
from oracle import core as O

G = O.W4_GROUP


def _bf16(x):
    """bfloat16 bit patterns of fp32 values (round to nearest even) and their exact values."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


def test_codes_and_scales_match_exact_arithmetic():
    rng = np.random.default_rng(40)
    for trial in range(3):
        w = (rng.standard_normal((3, 2 * G)) * 0.02).astype(np.float32)
        w[0, :G] *= np.float32(1e-3)  # a group of small values
        s = rng.uniform(0.5, 2.0, 2 * G).astype(np.float32) if trial == 2 else None
        codes, scales = O.quantize_w4(w, s=s)
        q = O.unpack_w4(codes)
        for r in range(3):
            bq, bs = B.quantize_w4_row([float(v) for v in w[r]], G, None if s is None else [float(v) for v in s])
            assert list(q[r]) == bq
            assert [float(v) for v in scales[r]] == [float(v) for v in bs]


def test_round_trip_bound_and_a_full_scale_code_per_group():
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((16, 4 * G)) * 0.02).astype(np.float32)
    w[3, G:2 * G] = 0.0  # an all-zero group: scale 1, codes 0
    codes, scales = O.quantize_w4(w)
    q = O.unpack_w4(codes).astype(np.float64)
    S = np.repeat(scales.astype(np.float64), G, axis=1)
    err = np.abs(S * q - w)
    assert (err <= S * 0.5 * (1 + 2.0 ** -20)).all()
    for r in range(16):
        for g in range(4):
            blk = q[r, g * G:(g + 1) * G]
            if (w[r, g * G:(g + 1) * G] != 0).any():
                assert np.abs(blk).max() == 7
            else:
                assert scales[r, g] == 1.0 and not blk.any()
    assert np.abs(q).max() <= 7


def test_sign_symmetry_and_power_of_two_invariant_scale():
    rng = np.random.default_rng(42)
    w = (rng.standard_normal((4, 2 * G)) * 0.02).astype(np.float32)
    c, s = O.quantize_w4(w)
    cn, sn = O.quantize_w4(-w)
    assert np.array_equal(O.unpack_w4(cn), -O.unpack_w4(c)) and np.array_equal(sn, s)
    c2, s2 = O.quantize_w4(w, s=np.full(2 * G, 4.0, np.float32))
    assert np.array_equal(c2, c) and np.array_equal(s2, s * np.float32(4.0))


def test_nibble_packing_by_hand():
    # group values S0 * j with max |j| = 7: S = fl32(7 S0 / 7) = S0 exactly for S0 = 0.5, so q = j
    j = np.array(([-7, -6, 5, 7, 0, -1, 3, -8 + 1] * (G // 8)), np.float32)
    codes, scales = O.quantize_w4((j * np.float32(0.5))[None, :])
    assert scales[0, 0] == 0.5
    # sign and magnitude: channel 0 (-7 = 0b1111) in the low nibble, channel 1 (-6 = 0b1110) in the high
    # nibble, ..., -1 = 0b1001; zero is 0000 (never the negative zero 1000)
    assert list(codes[0, :4]) == [0xEF, 0x75, 0x90, 0xF3]
    z, _ = O.quantize_w4(np.concatenate([np.full(G // 2, -1e-9, np.float32), np.full(G // 2, 1.0, np.float32)])[None])
    assert (z[0, :G // 4] == 0).all() and (z[0, G // 4:] == 0x77).all()


def test_bf16_input_equals_its_fp32_value():
    rng = np.random.default_rng(43)
    bits, vals = _bf16(rng.standard_normal((5, G)) * 0.02)
    assert all(np.array_equal(a, b) for a, b in zip(O.quantize_w4(bits), O.quantize_w4(vals)))


def test_linear_matches_exact_sum_and_closed_form():
    rng = np.random.default_rng(44)
    m, n, k = 3, 4, 2 * G
    xb, xv = _bf16(rng.standard_normal((m, k)))
    codes, scales = O.quantize_w4((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    y, y64 = O.w4a16_linear(xb, codes, scales)
    q = O.unpack_w4(codes)
    ref = B.w4a16_linear([[float(v) for v in r] for r in xv], [list(map(int, r)) for r in q],
                         [[B.f32_value(float(v)) for v in r] for r in scales], G)
    for i in range(m):
        for c in range(n):
            assert abs(y64[i, c] - float(ref[i][c])) <= 1e-12 * max(1.0, abs(float(ref[i][c])))
    # bfloat16 output: one rounding of the exact value
    assert np.array_equal(y, np.vectorize(O.round_to_bf16, otypes=[np.uint16])(y64))
    # closed form: x = 1, every code 7 (a positive constant row) -> y = 7 * G * sum of the row's scales
    wc, ws = O.quantize_w4(np.full((2, k), 0.01, np.float32))
    assert (O.unpack_w4(wc) == 7).all()
    ones, _ = _bf16(np.ones((1, k)))
    _, y1 = O.w4a16_linear(ones, wc, ws)
    assert np.allclose(y1[0], 7 * G * ws.astype(np.float64).sum(axis=1), rtol=0, atol=0)
