"""Pins of the oracle's codecs (FP8 E4M3, round-half-even, bfloat16) against the format definition,
closed forms, exact brute force and a library cross-check. CPU only."""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import core as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_format.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), val))
    return rows


def test_decode_matches_golden_table():
    rows = _golden()
    assert len(rows) >= 20
    for code, val in rows:
        got = O.e4m3_decode([code])[0]
        if val == "nan":
            assert math.isnan(got), hex(code)
        else:
            want = float(Fraction(val))
            assert got == want, (hex(code), got, want)
            if val.startswith("-0") and Fraction(val) == 0:
                assert math.copysign(1.0, got) < 0


def test_decode_closed_form_facts():
    vals = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = vals[~np.isnan(vals)]
    assert finite.size == 254  # 0x7F and 0xFF are NaN, nothing else
    assert np.nanmax(vals) == 448.0 and O.e4m3_decode([0x7E])[0] == 448.0
    assert O.e4m3_decode([0x01])[0] == 2.0 ** -9
    # every finite value is an exact integer multiple of 2^-9 with |units| <= 229376 = 448 * 2^9
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    units = O.e4m3_decode_units(codes)
    assert np.all(units * 2.0 ** -9 == O.e4m3_decode(codes))
    assert np.abs(units).max() == 229376
    # magnitudes increase strictly with the code over 0x00..0x7E (needed for the search encoder)
    mags = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(mags) > 0)
    # the decode agrees with the exact enumeration of Eq. (2)
    assert [Fraction(v) for v in mags] == brute.e4m3_values()


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)
    assert np.array_equal(O.e4m3_encode_search(vals), codes)


def test_encode_midpoints_go_to_even_and_neighbours_to_nearer():
    mags = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    for c in range(126):
        lo, hi = mags[c], mags[c + 1]
        mid = np.float32((lo + hi) / 2)  # exact: neighbours differ by a power of two times <= 3 bits
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        for sign, sbit in ((1, 0), (-1, 0x80)):
            v = np.float32(sign * mid)
            assert O.e4m3_encode([v])[0] == (even | sbit), (c, sign)
            below = np.nextafter(np.float32(mid), np.float32(0)) * sign
            above = np.nextafter(np.float32(mid), np.float32(1000)) * sign
            assert O.e4m3_encode([below])[0] == (c | sbit)
            assert O.e4m3_encode([above])[0] == ((c + 1) | sbit)


def test_encode_keeps_sign_of_zero():
    tiny = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, -(2.0 ** -10), 1e-40, -1e-40],
                    np.float32)
    got = O.e4m3_encode(tiny)
    # 2^-10 is the midpoint between 0 and 2^-9: ties to the even code 0
    assert list(got) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def _structured_patterns():
    """Every sign/exponent/top-7-mantissa pattern, with the low 16 bits set to values that exercise the
    round and sticky bits; kept to finite |v| <= 448."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    v = pats.view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= 448)
    return v[keep]


def test_encoders_agree_on_structured_patterns():
    v = _structured_patterns()
    assert v.size > 150_000
    assert np.array_equal(O.e4m3_encode(v), O.e4m3_encode_search(v))


def test_encoder_library_cross_check():
    # torch's cast (not an authority) rounds to nearest even and keeps -0; values are pre-clamped
    v = _structured_patterns()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_encoder_matches_exact_brute_force():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 200), rng.normal(0, 0.01, 200),
                        rng.normal(0, 3, 200)]).astype(np.float32)
    got = O.e4m3_encode(v)
    for x, g in zip(v, got):
        want = brute.e4m3_encode(Fraction(float(x)), bool(x < 0) or brute.neg_zero_sign(float(x)))
        assert g == want, (x, g, want)


def test_encoders_agree_exhaustively():
    """Every fp32 bit pattern, clamped to [-448, 448] as the quantizers do (NaN skipped): the arithmetic
    encoder and the search encoder give the same code. Patterns of magnitude above 448 all clamp to +-448, so
    the sweep covers the two sign halves up to 448 (0x43E00000) and one pattern above it on each side; a
    C loop inside the oracle library, run in chunks on all host cores (ctypes drops the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    top = 0x43E00000 + 1  # 448.0 is 0x43E00000
    chunk = 1 << 23
    ranges = []
    for sign in (0, 0x80000000):
        for lo in range(0, top, chunk):
            ranges.append((sign | lo, sign | min(lo + chunk, top)))
        ranges.append((sign | 0x7F000000, sign | 0x7F000001))  # a finite magnitude far above 448
    with ThreadPoolExecutor(max_workers=max(1, len(os.sched_getaffinity(0)))) as pool:
        results = list(pool.map(lambda r: O.e4m3_encoders_disagree(*r), ranges))
    covered = sum(hi - lo for lo, hi in ranges)
    assert covered == 2 * (top + 1)
    bad = [(r, res) for r, res in zip(ranges, results) if res[0] != 0]
    assert not bad, "encoders disagree: %d patterns, first 0x%08x" % (bad[0][1][0], bad[0][1][1])


def test_rne_matches_python_half_even():
    for k in range(-300, 300):
        x = k + 0.5
        assert O.rne(x) == round(x)
        assert O.rne(k + 0.49999997) == k
        assert O.rne(k) == k
    for x in np.random.default_rng(0).uniform(-200, 200, 1000):
        assert O.rne(float(np.float32(x))) == round(float(np.float32(x)))


def test_round_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(2)
    vals = list(rng.normal(0, 1, 300)) + list(rng.normal(0, 1e4, 100)) + [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                                                        -(1.0 + 2.0 ** -8)]
    for x in vals:
        q = Fraction(float(x))
        e = brute._floor_log2(abs(q))
        quantum = Fraction(2) ** (e - 7)
        want = round(q / quantum) * quantum
        bits = O.round_to_bf16(float(x))
        got = struct.unpack(">f", struct.pack(">I", bits << 16))[0]
        assert Fraction(got) == want, x


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    wide = O.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(wide[fin], ref[fin])
