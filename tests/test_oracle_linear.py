"""Pins of the oracle's W8A8 linear, grouped linear and changed-code count: textbook special cases,
exact brute force on tiny inputs, closed forms and error bounds. CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from oracle import core as O
from quantized_rollout_amd import synth

QT = [O.INT8, O.FP8]


def _codes_int8(a):
    return np.asarray(a, np.int8).view(np.uint8)


def _bf16_to_f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def test_int8_all_max_rows_give_closed_form():
    for k in (16, 256, 18944):
        x = _codes_int8(np.full((2, k), 127))
        w = _codes_int8(np.full((3, k), -127))
        _, acc, _ = O.linear(O.INT8, x, np.ones(2, np.float32), w, np.ones(3, np.float32), O.F32)
        assert np.all(acc == -16129 * k)
    # k = 18944 (the 7B down projection): 305,547,776 fits in int32
    assert 16129 * 18944 == 305547776


def test_int8_alternating_and_one_hot():
    k = 64
    alt = np.array([127 if j % 2 == 0 else -127 for j in range(k)])
    ones = np.full(k, 127)
    x = _codes_int8(np.stack([alt, ones]))
    w = _codes_int8(np.stack([ones, np.zeros(k, int)]))
    _, acc, _ = O.linear(O.INT8, x, np.ones(2, np.float32), w, np.ones(2, np.float32), O.F32)
    assert acc[0, 0] == 0 and acc[1, 0] == 127 * 127 * k and np.all(acc[:, 1] == 0)
    onehot_x = np.zeros((1, k), int)
    onehot_x[0, 37] = -3
    wr = np.arange(k) % 255 - 127
    _, acc, _ = O.linear(O.INT8, _codes_int8(onehot_x), np.ones(1, np.float32), _codes_int8(wr[None, :]),
                         np.ones(1, np.float32), O.F32)
    assert acc[0, 0] == -3 * wr[37]


def test_fp8_all_max_rows_closed_form():
    """All-448 codes: acc = 448^2 * k = 200704 * k, exactly representable."""
    for k in (16, 3584, 18944):
        x = np.full((1, k), 0x7E, np.uint8)
        w = np.full((2, k), 0xFE, np.uint8)
        y, _, acc = O.linear(O.FP8, x, np.ones(1, np.float32), w, np.ones(2, np.float32), O.F32)
        assert np.all(acc == -200704.0 * k)
        assert np.all(y == np.float32(-200704.0 * k))
    assert 200704 * 18944 == 2 ** 21 * 1813


@pytest.mark.parametrize("qtype", QT)
def test_linear_matches_exact_brute_force(qtype):
    rng = np.random.default_rng(30 + qtype)
    for (m, n, k) in [(1, 1, 16), (3, 4, 16), (4, 2, 32), (2, 3, 48)]:
        x = rng.standard_normal((m, k)).astype(np.float32)
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        xc, xs = O.quantize_rows(x, qtype)
        wc, ws = O.quantize_rows(w, qtype)
        y32, acc_i, acc_f = O.linear(qtype, xc, xs, wc, ws, O.F32)
        ybf, _, _ = O.linear(qtype, xc, xs, wc, ws, O.BF16)
        bacc, by = brute.linear(qtype, [list(r) for r in xc], [float(v) for v in xs],
                                [list(r) for r in wc], [float(v) for v in ws])
        for i in range(m):
            for c in range(n):
                assert Fraction(float(acc_f[i, c])) == bacc[i][c]
                if qtype == O.INT8:
                    assert int(acc_i[i, c]) == bacc[i][c]
                # y: one rounding of the (fp64) product: within an fp32 / bf16 half-ulp of the exact value
                exact = float(by[i][c])
                assert abs(float(y32[i, c]) - exact) <= abs(exact) * 2.0 ** -24 * 1.0001
                assert abs(_bf16_to_f64(ybf[i, c]) - exact) <= abs(exact) * 2.0 ** -8 * 1.0001


@pytest.mark.parametrize("qtype", QT)
def test_quantized_product_error_bound(qtype):
    """|y - x.w| <= sum_j (|x_j| dw_j + |w_j| dx_j + dx_j dw_j) with dx, dw the per-element round-trip
    bounds; the outlier channel makes the per-token scale large, as in the toy workload."""
    rng = np.random.default_rng(40)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    x[:, [3, 50, 100, 200]] *= 20
    w = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    xc, xs = O.quantize_rows(x, qtype)
    wc, ws = O.quantize_rows(w, qtype)
    y, _, _ = O.linear(qtype, xc, xs, wc, ws, O.F32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    if qtype == O.INT8:
        dx = np.broadcast_to(xs[:, None] / 2, x.shape).astype(np.float64)
        dw = np.broadcast_to(ws[:, None] / 2, w.shape).astype(np.float64)
    else:
        dx = xs[:, None] * np.maximum(np.abs(x) / xs[:, None] * 2.0 ** -4, 2.0 ** -10)
        dw = ws[:, None] * np.maximum(np.abs(w) / ws[:, None] * 2.0 ** -4, 2.0 ** -10)
    bound = np.abs(x) @ dw.T + dx @ np.abs(w).T + dx @ dw.T
    assert np.all(np.abs(y - ref) <= bound * 1.001 + 1e-6)


def test_int8_batch_prefix_invariance():
    rng = np.random.default_rng(41)
    xc = rng.integers(-127, 128, (8, 64)).astype(np.int8).view(np.uint8)
    wc = rng.integers(-127, 128, (5, 64)).astype(np.int8).view(np.uint8)
    xs = rng.uniform(0.01, 1, 8).astype(np.float32)
    ws = rng.uniform(0.01, 1, 5).astype(np.float32)
    yfull, accfull, _ = O.linear(O.INT8, xc, xs, wc, ws)
    for m in (1, 3, 7):
        y, acc, _ = O.linear(O.INT8, xc[:m], xs[:m], wc, ws)
        assert np.array_equal(acc, accfull[:m]) and np.array_equal(y, yfull[:m])


@pytest.mark.parametrize("qtype", QT)
def test_grouped_special_cases(qtype):
    rng = np.random.default_rng(50)
    k, n, E, T = 32, 8, 4, 6
    xc, xs = O.quantize_rows(rng.standard_normal((T, k)).astype(np.float32), qtype)
    wc = np.empty((E, n, k), np.uint8)
    ws = np.empty((E, n), np.float32)
    for e in range(E):
        wc[e], ws[e] = O.quantize_rows((rng.standard_normal((n, k)) * 0.02).astype(np.float32), qtype)
    # E = 1 with identity rows equals the plain linear
    y1 = O.grouped_linear(qtype, np.array([0, T], np.int32), None, xc, xs, wc[:1], ws[:1])
    y0, _, _ = O.linear(qtype, xc, xs, wc[0], ws[0])
    assert np.array_equal(y1, y0)
    # token lists with an empty expert; each expert's rows equal the linear on the gathered rows
    offsets = np.array([0, 3, 3, 7, 9], np.int32)
    row_ids = np.array([0, 2, 5, 1, 2, 3, 4, 0, 5], np.int32)
    y = O.grouped_linear(qtype, offsets, row_ids, xc, xs, wc, ws)
    assert y.shape == (9, n)
    for e in range(E):
        rows = row_ids[offsets[e]:offsets[e + 1]]
        if rows.size == 0:
            continue
        ye, _, _ = O.linear(qtype, xc[rows], xs[rows], wc[e], ws[e])
        assert np.array_equal(y[offsets[e]:offsets[e + 1]], ye)
    with pytest.raises(ValueError):
        O.grouped_linear(qtype, np.array([0, 3, 2, 7, 9], np.int32), row_ids, xc, xs, wc, ws)


def test_route_top_k_lists():
    rng = np.random.default_rng(51)
    logits = rng.standard_normal((16, 8)).astype(np.float32)
    logits[0, :] = 0.5  # all tied: the lowest expert indices win
    off, rows = synth.route_top_k(logits, 3)
    assert off[0] == 0 and off[-1] == 16 * 3 and np.all(np.diff(off) >= 0)
    for e in range(8):
        toks = rows[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)
        for t in toks:
            assert (logits[t] > logits[t, e]).sum() < 3
    assert set(e for e in range(8) if 0 in rows[off[e]:off[e + 1]]) == {0, 1, 2}


@pytest.mark.parametrize("qtype", QT)
def test_count_code_changes(qtype):
    rng = np.random.default_rng(60)
    w = (rng.standard_normal((64, 128)) * 0.02).astype(np.float32)
    w2 = (w + rng.standard_normal(w.shape) * 1e-4).astype(np.float32)
    a, sa = O.quantize_rows(w, qtype)
    b, sb = O.quantize_rows(w2, qtype)
    assert list(O.count_code_changes(a, a, qtype, sa, sa)) == [0, 0, 0]
    got = O.count_code_changes(a, b, qtype, sa, sb)
    assert got[0] == int(np.sum(a != b)) and got[0] > 0
    assert got[2] == int(np.sum(sa.view(np.uint32) != sb.view(np.uint32)))
    if qtype == O.INT8:
        assert got[1] == got[0]
    # FP8 +0 vs -0: one byte differs, no value differs
    z = np.array([0x00, 0x80, 0x38, 0x38], np.uint8)
    z2 = np.array([0x80, 0x00, 0x38, 0xB8], np.uint8)
    assert list(O.count_code_changes(z, z2, O.FP8)) == [3, 1, 0]


@pytest.mark.parametrize("qtype", QT)
def test_abs_sum_matches_brute_force(qtype):
    """The sum of |x_j w_j| (the scale of the fp32 summation bound that gates FP8 accumulators) against exact
    rational arithmetic over every code byte, on tiny random inputs."""
    rng = np.random.default_rng(90 + qtype)
    for m, n, k in ((1, 1, 16), (3, 4, 32), (2, 5, 48)):
        if qtype == O.INT8:
            x = _codes_int8(rng.integers(-127, 128, (m, k)))
            w = _codes_int8(rng.integers(-127, 128, (n, k)))
        else:
            x = rng.integers(0, 256, (m, k)).astype(np.uint8)
            w = rng.integers(0, 256, (n, k)).astype(np.uint8)
            x[(x & 0x7F) == 0x7F] = 0x01  # no NaN codes
            w[(w & 0x7F) == 0x7F] = 0x81
        got = O.linear_abs_sum(qtype, x, w)
        for i in range(m):
            for c in range(n):
                want = sum(abs(brute.code_value(int(x[i, j]), qtype) * brute.code_value(int(w[c, j]), qtype))
                           for j in range(k))
                assert Fraction(float(got[i, c])) == want, (m, n, k, i, c)


@pytest.mark.parametrize("qtype", QT)
def test_abs_sum_closed_forms(qtype):
    """Equal to |acc| when every product has one sign (all-max rows: 127^2 k or 448^2 k); at least |acc| and
    strictly more when signs mix (alternating signs: acc = 0, abs sum = qmax^2 k)."""
    k = 256
    hi, lo = (0x7F, 0x81) if qtype == O.INT8 else (0x7E, 0xFE)  # +qmax, -qmax
    q2 = 127 * 127 if qtype == O.INT8 else 448 * 448
    x = np.stack([np.full(k, hi, np.uint8), np.array([hi if j % 2 == 0 else lo for j in range(k)], np.uint8)])
    w = np.full((1, k), lo, np.uint8)
    a = O.linear_abs_sum(qtype, x, w)
    _, _, acc = O.linear(qtype, x, np.ones(2, np.float32), w, np.ones(1, np.float32), O.F32)
    assert a[0, 0] == q2 * k and acc[0, 0] == -q2 * k
    assert a[1, 0] == q2 * k and acc[1, 0] == 0


def _pow2_code(e, neg=False):
    c = ((e + 7) << 3) if e >= -6 else (1 << (e + 9))
    return c | (0x80 if neg else 0)


def test_fp8_mfma_truncation_tolerance():
    """The tolerance of FP8 accumulators on the matrix cores (measured on gfx950: products added inside one
    instruction are aligned to the largest exponent sum and truncated 13 bits below it): cases the probes of the
    hardware fixed, and the bound's own invariants."""
    k = 512

    def row(entries):
        a = np.zeros((1, k), np.uint8)
        b = np.zeros((1, k), np.uint8)
        for j, ea, eb, neg in entries:
            a[0, j], b[0, j] = _pow2_code(ea, neg), _pow2_code(eb)
        return a, b

    T = lambda e: O.fp8_mfma_truncation(*row(e))[0, 0]  # noqa: E731
    assert T([(0, 4, 4, False)]) == 0.0                                   # one product: exact
    assert T([(0, 4, 4, False), (1, -5, -5, False)]) == 2.0 ** -10        # 2^8 + 2^-10: dropped (probe: lost)
    assert T([(0, 4, 4, False), (1, -5, -5, True)]) == 2.0 ** -10         # the same below zero
    assert T([(0, 4, 4, False), (1, -2, -3, False)]) == 0.0               # 2^-5 = 13 below 2^8: kept (probe: kept)
    assert T([(0, 4, 4, False), (1, -3, -3, False)]) == 2.0 ** -6         # 2^-6: dropped (probe: lost)
    assert T([(0, 4, 4, False), (500, -5, -5, False)]) == 0.0             # far apart: never in one instruction
    # 2^8 with fifteen 2^-6 after it: at most all fifteen dropped (probe: the seven in its 8-block were)
    assert T([(0, 4, 4, False)] + [(j, -3, -3, False) for j in range(1, 16)]) == 15 * 2.0 ** -6
    # all-448 rows: every product on the grid, the accumulator exact (the closed form checked on the GPU)
    x = np.full((2, k), 0x7E, np.uint8)
    w = np.full((3, k), 0xFE, np.uint8)
    assert not O.fp8_mfma_truncation(x, w).any()
    # random codes: 0 <= T <= sum |p|
    rng = np.random.default_rng(95)
    x = rng.integers(0, 256, (4, 1040)).astype(np.uint8)
    w = rng.integers(0, 256, (5, 1040)).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x38
    w[(w & 0x7F) == 0x7F] = 0x38
    t = O.fp8_mfma_truncation(x, w)
    assert (t >= 0).all() and (t <= O.linear_abs_sum(O.FP8, x, w)).all() and t.max() > 0
