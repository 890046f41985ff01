"""Pins of the requantize + diff oracle (the next row after the W8A8 path: one publish of W + dW, [QaRL] 3.1's
per-step publish of low-bit weights, compared against the previous publish as in [QuRL] 4.3).

Against: hand-worked codes on either side of a rounding boundary, a scale change, the FP8 signed zero (a byte
change that is no value change), per-row counts recomputed with numpy from the codes alone, and the
identity with the pinned a1 quantizer and a5 count."""
import numpy as np
import pytest

from oracle import core as O


def _publish(w, q, prev=None, s=None):
    if prev is None:
        c, sc = O.quantize_rows(w, q, s=s)
        return c, sc
    return O.requantize_weights(w, q, prev[0], prev[1], s=s)


def _numpy_counts(prev_c, new_c, prev_s, new_s):
    """Per-row (bytes, values, scale) changes from the code bytes alone: E4M3FN is one-to-one on the finite
    values except +0 / -0 (0x00 / 0x80), and INT8 codes are two's complement."""
    diff = prev_c != new_c
    both_zero = ((prev_c & 0x7F) == 0) & ((new_c & 0x7F) == 0)
    return diff, both_zero, prev_s.view(np.uint32) != new_s.view(np.uint32)


def test_unchanged_weights_change_nothing():
    rng = np.random.default_rng(60)
    w = (rng.standard_normal((7, 96)) * 0.02).astype(np.float32)
    for q in (O.INT8, O.FP8):
        prev = _publish(w, q)
        c, sc, rc, out3 = _publish(w, q, prev)
        assert np.array_equal(c, prev[0]) and np.array_equal(sc, prev[1])
        assert not rc.any() and not out3.any()


def test_int8_code_crosses_a_rounding_boundary_by_hand():
    # S = fl32(63.5 / 127) = 0.5 exactly; 5.245 / 0.5 = 10.49 -> code 10, 5.255 / 0.5 = 10.51 -> code 11
    row = np.zeros(32, np.float32)
    row[0] = 63.5
    row[5] = 5.245
    row[9] = 5.24
    prev = _publish(row[None], O.INT8)
    assert prev[1][0] == 0.5 and prev[0][0, 5] == 10 and prev[0][0, 9] == 10
    new = row.copy()
    new[5] = 5.255  # crosses 10.5
    new[9] = 5.20   # 10.4: stays 10
    c, sc, rc, out3 = _publish(new[None], O.INT8, prev)
    assert c[0, 5] == 11 and c[0, 9] == 10 and sc[0] == 0.5
    assert rc.tolist() == [[1, 1, 0]] and out3.tolist() == [1, 1, 0]


def test_scale_change_counts_the_row_once():
    rng = np.random.default_rng(61)
    w = (rng.standard_normal((3, 64)) * 0.02).astype(np.float32)
    w[:, 0] = 0.05  # the row maximum
    prev = _publish(w, O.INT8)
    new = w.copy()
    new[1, 0] = 0.06  # row 1's scale changes, and with it most of its codes
    c, sc, rc, out3 = _publish(new, O.INT8, prev)
    diff, _, sdiff = _numpy_counts(prev[0], c, prev[1], sc)
    assert rc[:, 2].tolist() == [0, 1, 0] and sdiff.tolist() == [False, True, False]
    assert rc[:, 0].tolist() == diff.sum(axis=1).tolist() and rc[1, 0] > 32
    assert rc[0, 0] == 0 and rc[2, 0] == 0


def test_fp8_signed_zero_is_a_byte_change_but_not_a_value_change():
    # S = fl32(448 / 448) = 1; -1e-9 rounds to -0 (0x80), +1e-9 to +0 (0x00)
    row = np.zeros(16, np.float32)
    row[0] = 448.0
    row[3] = -1e-9
    prev = _publish(row[None], O.FP8)
    assert prev[0][0, 3] == 0x80
    new = row.copy()
    new[3] = 1e-9
    c, sc, rc, out3 = _publish(new[None], O.FP8, prev)
    assert c[0, 3] == 0x00
    assert rc.tolist() == [[1, 0, 0]] and out3.tolist() == [1, 0, 0]


@pytest.mark.parametrize("q", [O.INT8, O.FP8])
@pytest.mark.parametrize("bf16", [False, True])
def test_small_update_matches_numpy_counts_and_the_a1_a5_composition(q, bf16):
    rng = np.random.default_rng(62 + q + 2 * bf16)
    w = (rng.standard_normal((9, 256)) * 0.02).astype(np.float32)
    dw = (rng.standard_normal((9, 256)) * 1e-4).astype(np.float32)
    s = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    if bf16:
        to = lambda a: ((a.view(np.uint32).astype(np.uint64) + 0x7FFF + ((a.view(np.uint32) >> 16) & 1)) >> 16
                        ).astype(np.uint16)
        w_in, w2_in = to(w), to(w + dw)
    else:
        w_in, w2_in = w, w + dw
    prev = _publish(w_in, q, s=s)
    c, sc, rc, out3 = _publish(w2_in, q, prev, s=s)
    # the codes and scales are the a1 quantizer's
    ca, sa = O.quantize_rows(w2_in, q, s=s)
    assert np.array_equal(c, ca) and np.array_equal(sc, sa)
    # per-row counts from the bytes alone
    diff, both_zero, sdiff = _numpy_counts(prev[0], c, prev[1], sc)
    assert rc[:, 0].tolist() == diff.sum(axis=1).tolist()
    assert rc[:, 1].tolist() == (diff & ~both_zero).sum(axis=1).tolist()
    assert rc[:, 2].tolist() == sdiff.astype(int).tolist()
    assert out3.tolist() == rc.sum(axis=0).tolist()
    # and the whole-tensor triple is the a5 count of the two publishes
    assert out3.tolist() == O.count_code_changes(prev[0], c, q, prev[1], sc).tolist()
    assert 0 < out3[0] < c.size  # a small update changes some codes, not all
