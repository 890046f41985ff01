"""Pins of the MoE glue oracle (the next row around the grouped W8A8 linear of the MoE FFN: routing, the
SiLU-gated product, the routing-weighted combine).

Against: the host routing of the input generator (independent code), the routing's invariants (choices in
expert order, rows grouped by expert with tokens ascending, softmax weights summing to one, equal logits giving
equal weights), closed forms of silu(g) u, and the combine of single-expert routes and equal rows."""
import math

import numpy as np

from oracle import core as O
from quantized_rollout_amd import synth


def _bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_bits(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_route_matches_the_host_routing_and_its_invariants():
    rng = np.random.default_rng(70)
    for T, E, k in ((16, 8, 3), (64, 128, 8), (5, 32, 1)):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        logits[0, :] = 0.25  # all tied: the lowest expert indices win
        if T > 1:
            logits[1, 3] = logits[1, 5] = logits[1].max() + 1.0  # a tie at the top
        r = O.moe_route(logits, k)
        off, rows = synth.route_top_k(logits, k)
        assert np.array_equal(r["offsets"], off) and np.array_equal(r["row_ids"], rows)
        assert (np.diff(r["topk_expert"], axis=1) > 0).all()
        assert list(r["topk_expert"][0]) == list(range(k))
        for t in range(T):
            for j in range(k):
                row, e = r["pair_rows"][t, j], r["topk_expert"][t, j]
                assert r["row_ids"][row] == t and r["offsets"][e] <= row < r["offsets"][e + 1]
                assert r["row_weights"][row] == r["topk_weight"][t, j]
        assert np.allclose(r["topk_weight"].astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
        assert np.allclose(r["topk_weight"][0], 1.0 / k, atol=1e-7)  # equal logits, equal weights
        # a larger logit never gets a smaller weight
        for t in range(T):
            l = logits[t, r["topk_expert"][t]]
            w = r["topk_weight"][t]
            assert all(w[a] >= w[b] for a in range(k) for b in range(k) if l[a] > l[b])


def test_route_two_experts_closed_form():
    logits = np.array([[1.0, 3.0, -2.0]], np.float32)
    r = O.moe_route(logits, 2)
    assert list(r["topk_expert"][0]) == [0, 1]
    w0 = 1.0 / (1.0 + math.exp(2.0))
    assert np.allclose(r["topk_weight"][0], [w0, 1.0 - w0], rtol=0, atol=6e-8)


def test_silu_mul_closed_forms():
    g = np.array([0.0, 1.5, 30.0, -30.0, math.log(3.0), 2.0, -1.0, 4.0], np.float32)
    u = np.array([3.0, 0.0, 1.0, 5.0, 1.0, -2.0, 1.0, 0.5], np.float32)
    y = _bf16_bits(np.concatenate([g, u])[None, :])
    h = _bf16_value(O.silu_mul(y))[0]
    gb, ub = _bf16_value(_bf16_bits(g)), _bf16_value(_bf16_bits(u))
    assert h[0] == 0.0 and h[1] == 0.0                   # silu(0) = 0; u = 0
    assert h[2] == 30.0                                   # silu(30) = 30 (1 - 9.4e-14): rounds to 30
    assert -1e-10 < h[3] < 0.0                            # silu(-30) * 5 = -1.4e-11
    assert h[4] == _bf16_value(_bf16_bits(np.float32(0.75 * float(gb[4]) * float(ub[4]))))  # sigmoid(ln 3) = 3/4
    # silu(g) - silu(-g) = g: the rows (2, u) and (-2, u) differ by 2 u before rounding
    y2 = _bf16_bits(np.array([[2.0, -2.0, 1.0, 1.0]], np.float32))
    hp, hn = _bf16_value(O.silu_mul(y2))[0]
    assert abs((float(hp) - float(hn)) - 2.0) <= 2 * 2.0 ** -7 * 2.0


def test_combine_single_routes_and_equal_rows():
    rng = np.random.default_rng(71)
    y = _bf16_bits(rng.standard_normal((6, 40)).astype(np.float32))
    # k = 1 with weight 1: each token's output is its row
    out = O.moe_combine(y, np.ones((6, 1), np.float32), np.arange(6, dtype=np.int32)[::-1].reshape(6, 1).copy())
    assert np.array_equal(out, y[::-1])
    # two equal rows, weights 1/4 and 3/4: the row itself
    y2 = np.concatenate([y[:1], y[:1]])
    out2 = O.moe_combine(y2, np.array([[0.25, 0.75]], np.float32), np.array([[0, 1]], np.int32))
    assert np.array_equal(out2[0], y[0])


# A hand-worked combine: T = 2 tokens, k = 3 choices, H = 4 channels, six distinct expert-output rows and
# distinct weights. Every value and weight is dyadic, so each sum is exact and its bfloat16 bits are written
# out by hand below.
_Y_ROWS = np.array([[1, 2, -4, 8],          # row 0
                    [16, -1, 0.5, 3],       # row 1
                    [-2, 6, 10, 0.25],      # row 2
                    [4, -8, 2, 1],          # row 3
                    [0, 1, -3, 12],         # row 4
                    [-6, 0.5, 7, -1]],      # row 5
                   np.float32)
_PAIR_ROWS = np.array([[3, 0, 5], [1, 4, 2]], np.int32)          # [t][j]
_WEIGHTS = np.array([[0.5, 0.25, 0.25], [0.125, 0.375, 0.5]], np.float32)
# token 0: 0.5 row3 + 0.25 row0 + 0.25 row5 = [0.75, -3.375, 1.75, 2.25]
# token 1: 0.125 row1 + 0.375 row4 + 0.5 row2 = [1, 3.25, 3.9375, 5]
_EXPECTED_BITS = np.array([[0x3F40, 0xC058, 0x3FE0, 0x4010],
                           [0x3F80, 0x4050, 0x407C, 0x40A0]], np.uint16)


def test_combine_hand_worked_two_tokens_three_choices():
    out = O.moe_combine(_bf16_bits(_Y_ROWS), _WEIGHTS, _PAIR_ROWS)
    assert np.array_equal(out, _EXPECTED_BITS), [[hex(v) for v in r] for r in out]


def test_combine_pairs_each_weight_with_its_own_row():
    """Swapping two pair rows of token 0 (weights unchanged) changes its output to the hand value
    0.5 row0 + 0.25 row3 + 0.25 row5 = [0, -0.875, 0.25, 4]; token 1 is untouched. A layout slip ([j][t]
    instead of [t][j]) or a weight paired with another choice's row would give neither expected output."""
    pr = _PAIR_ROWS.copy()
    pr[0, 0], pr[0, 1] = pr[0, 1], pr[0, 0]
    out = O.moe_combine(_bf16_bits(_Y_ROWS), _WEIGHTS, pr)
    assert np.array_equal(out[0], np.array([0x0000, 0xBF60, 0x3E80, 0x4080], np.uint16)), [hex(v) for v in out[0]]
    assert np.array_equal(out[1], _EXPECTED_BITS[1])
    # the [j][t] reading of the same buffer pairs token 0's weights with rows 3, 0, 5 of another shape
    wrong = O.moe_combine(_bf16_bits(_Y_ROWS), _WEIGHTS, _PAIR_ROWS.T.copy().reshape(2, 3))
    assert not np.array_equal(wrong, _EXPECTED_BITS)


def test_combine_rounds_once():
    """1 + 2^-8 + 2^-20 rounds once to bfloat16 1 + 2^-7 (0x3F81); rounding the partial sum 1 + 2^-8 first
    (a tie, to even: 1.0) would give 0x3F80."""
    y = _bf16_bits(np.array([[2.0], [2.0 ** -6], [2.0 ** -18]], np.float32))
    out = O.moe_combine(y, np.array([[0.5, 0.25, 0.25]], np.float32), np.array([[0, 1, 2]], np.int32))
    assert out[0, 0] == 0x3F81


def test_combine_skips_pair_rows_outside_the_rows():
    """A pair row outside [0, R) adds nothing (the library's contract for an inconsistent pair list)."""
    pr = _PAIR_ROWS.copy()
    pr[1, 1] = 6      # past the last row: token 1 loses 0.375 row4 -> [1, 2.875, 5.0625, 0.5]
    pr[0, 2] = -1     # token 0 loses 0.25 row5 -> [2.25, -3.5, 0, 2.5]
    out = O.moe_combine(_bf16_bits(_Y_ROWS), _WEIGHTS, pr)
    assert np.array_equal(out, np.array([[0x4010, 0xC060, 0x0000, 0x4020],
                                         [0x3F80, 0x4038, 0x40A2, 0x3F00]], np.uint16)), out
