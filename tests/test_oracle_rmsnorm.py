"""Pins of the RMSNorm producer oracle (the next row that fuses the token-wise activation quantizer into the
producer of a linear's input).

Against: the exact-rational RMSNorm of ``oracle/brute.py`` (rounding decided by comparing squares, no square
root), closed forms (rows of one magnitude, a single non-zero entry, zero rows), the scale invariance of the
normalization, and the library RMSNorm of PyTorch in float64. The producer's codes are the token-wise
quantizer's codes of h, checked against the exact quantizer of ``oracle/brute.py``."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import core as O


def _bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf16_bits(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _row(rng, K, scale):
    x = rng.standard_normal(K) * scale
    if K > 3:
        x[rng.integers(K)] *= 40.0  # an outlier channel
    return _bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("K", [1, 2, 7, 33, 64])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1.0])
def test_rmsnorm_matches_the_exact_rounding(K, eps):
    rng = np.random.default_rng(1000 + K)
    x = np.stack([_row(rng, K, sc) for sc in (1.0, 3e-4, 250.0, 0.02)])
    gamma = (rng.uniform(0.2, 2.5, K) * rng.choice([-1.0, 1.0], K)).astype(np.float32)
    h = _bf16_value(O.rmsnorm(x, gamma, np.float32(eps)))
    xv = _bf16_value(x)
    for r in range(x.shape[0]):
        exact = brute.rmsnorm_row([float(v) for v in xv[r]], [float(g) for g in gamma], float(np.float32(eps)))
        got = [Fraction(float(v)) for v in h[r]]
        assert got == exact, (K, eps, r)


def test_rmsnorm_closed_forms():
    # rows of one magnitude c: h = sign(x) gamma exactly (eps = 0), whatever c and K
    for c, K in ((1.0, 8), (3.0, 5), (0.0078125, 64), (1.5e-5, 16), (6.0e4, 3)):
        x = _bf16_bits(np.array([c if j % 3 else -c for j in range(K)], np.float32))
        gamma = _bf16_value(_bf16_bits(np.linspace(0.5, 2.0, K).astype(np.float32)))
        h = _bf16_value(O.rmsnorm(x[None], gamma, 0.0))[0]
        assert np.array_equal(h, np.where(_bf16_value(x) < 0, -gamma, gamma)), (c, K)
    # one non-zero entry a among K: mean square a^2 / K, so h = sign(a) sqrt(K) gamma (K = 4: exactly 2 gamma)
    x = _bf16_bits(np.array([[0.0, -5.0, 0.0, 0.0]], np.float32))
    h = _bf16_value(O.rmsnorm(x, np.full(4, 0.75, np.float32), 0.0))[0]
    assert h.tolist() == [0.0, -1.5, 0.0, 0.0]
    # eps inside the root: x = [1, 1], eps = 3 -> 1 / sqrt(1 + 3) = 0.5
    h = _bf16_value(O.rmsnorm(_bf16_bits(np.ones((1, 2), np.float32)), np.ones(2, np.float32), 3.0))[0]
    assert h.tolist() == [0.5, 0.5]
    # zero rows: zeros, with or without eps (no NaN from 0 * inf)
    for eps in (0.0, 1e-6):
        h = _bf16_value(O.rmsnorm(np.zeros((2, 16), np.uint16), np.ones(16, np.float32), eps))
        assert np.array_equal(h, np.zeros((2, 16), np.float32)) and not np.isnan(h).any()


def test_rmsnorm_scale_invariance():
    # with eps = 0 the normalization does not see a power-of-two factor of the row: identical bits
    rng = np.random.default_rng(5)
    x = np.stack([_row(rng, 96, 1.0) for _ in range(6)])
    gamma = rng.uniform(0.5, 1.5, 96).astype(np.float32)
    ref = O.rmsnorm(x, gamma, 0.0)
    for p in (-20, 7, 40):
        xp = _bf16_bits(_bf16_value(x) * np.float32(2.0 ** p))
        assert np.array_equal(_bf16_value(xp), _bf16_value(x) * np.float32(2.0 ** p))  # exact scaling
        assert np.array_equal(O.rmsnorm(xp, gamma, 0.0), ref), p


def test_rmsnorm_against_the_library_rmsnorm():
    # torch's RMSNorm in float64 (x / sqrt(mean(x^2) + eps) * weight), rounded once: within half a bf16 ulp of
    # the double value, and equal wherever the double value is not within 2^-30 of a rounding boundary
    rng = np.random.default_rng(9)
    R, K, eps = 48, 3584, 1e-6
    x = np.stack([_row(rng, K, sc) for sc in np.geomspace(1e-3, 1e2, R)])
    gamma = rng.uniform(0.02, 3.0, K).astype(np.float32)
    xt = torch.from_numpy(_bf16_value(x).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (K,), torch.from_numpy(gamma.astype(np.float64)), eps).numpy()
    h = _bf16_value(O.rmsnorm(x, gamma, np.float32(eps))).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7)
    assert (np.abs(h - ref) <= 0.5 * ulp * (1 + 2.0 ** -30)).all()
    # a sample compared exactly: the double value rounded once (by exact comparisons) where it is clear of a
    # rounding boundary by more than the double evaluation's error
    frac = np.abs(ref) / ulp - np.floor(np.abs(ref) / ulp)
    idx = rng.choice(h.size, 3000, replace=False)
    for i in idx:
        r, c = divmod(int(i), K)
        if abs(frac[r, c] - 0.5) > 2.0 ** -30:
            v = Fraction(float(ref[r, c]))
            want = brute.round_bf16_signed_sqrt(1 if v > 0 else -1, v * v)
            assert Fraction(float(h[r, c])) == want, (r, c)


@pytest.mark.parametrize("qtype", [O.INT8, O.FP8])
def test_rmsnorm_quantize_is_the_quantizer_of_h(qtype):
    # the producer's codes and scales: the exact token-wise quantizer of h, with h diag(1/s) when s is given
    rng = np.random.default_rng(11 + qtype)
    K = 24
    x = np.stack([_row(rng, K, sc) for sc in (1.0, 0.05, 30.0)])
    gamma = rng.uniform(0.3, 2.0, K).astype(np.float32)
    s = rng.uniform(0.5, 2.0, K).astype(np.float32)
    for sv in (None, s):
        codes, scales, h = O.rmsnorm_quantize(x, gamma, np.float32(1e-6), qtype, s=sv)
        assert np.array_equal(h, O.rmsnorm(x, gamma, np.float32(1e-6)))
        hv = _bf16_value(h)
        for r in range(x.shape[0]):
            bc, bS = brute.quantize_row([float(v) for v in hv[r]], qtype,
                                        s=None if sv is None else [float(v) for v in sv], recip=True)
            assert codes[r].tolist() == bc and Fraction(float(scales[r])) == bS, (qtype, sv is None, r)
