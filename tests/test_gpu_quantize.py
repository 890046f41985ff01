"""GPU parity of the weight and activation quantizers (a1, a2): codes and scales bit-exact against the
oracle, on seeded inputs through the C ABI."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O
from quantized_rollout_amd import synth

from gpu_util import assert_codes_equal, assert_scales_equal, dev, host, log

pytestmark = pytest.mark.gpu

QT = [(O.INT8, qr.QR_INT8), (O.FP8, qr.QR_FP8_E4M3)]


def _inputs(rows, k, dtype, seed, std=0.02):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, k)) * std).astype(np.float32)
    cols = rng.choice(k, min(4, k), replace=False)
    x[:, cols] *= np.float32(20)
    if rows > 2:
        x[2] = 0.0  # all-zero row
    if rows > 3:
        x[3, ::3] = -0.0
    s = rng.uniform(0.5, 2.0, k).astype(np.float32)
    return (synth.f32_to_bf16_bits(x) if dtype == "bf16" else x), s


# sizes spanning every workgroup-size variant of the kernel (64..1024 threads), the register-overflow
# re-read path (rows longer than 1024 lanes x 8 chunks), ragged chunk counts, and a single row
SHAPES = [(1, 16), (5, 48), (37, 1552), (64, 3584), (9, 8960), (3, 18944), (2, 40960), (4, 65536 + 16)]


@pytest.mark.parametrize("oq,gq", QT)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("which", ["weights", "acts"])
@pytest.mark.parametrize("with_s", [False, True])
def test_quantizer_parity(oq, gq, dtype, which, with_s):
    for i, (rows, k) in enumerate(SHAPES):
        x, s = _inputs(rows, k, dtype, seed=100 + i)
        s_arg = s if with_s else None
        log("quantize %s %s %s s=%s rows=%d k=%d" % (which, dtype, oq, with_s, rows, k))
        mode = O.S_MUL if which == "weights" else O.S_MUL_RECIP
        c_ref, s_ref = O.quantize_rows(x, oq, s=s_arg, s_mode=mode)
        fn = qr.qr_quantize_weights if which == "weights" else qr.qr_quantize_acts
        c, sc = fn(dev(x), gq, s=None if s_arg is None else dev(s))
        torch.cuda.synchronize()
        assert_codes_equal(host(c), c_ref, "%s %dx%d" % (which, rows, k))
        assert_scales_equal(host(sc), s_ref, "%s %dx%d" % (which, rows, k))


@pytest.mark.parametrize("oq,gq", QT)
def test_quantizer_near_ties(oq, gq):
    """Values on and one ulp around the rounding boundaries of w / S, for many non-power-of-two scales: a
    division that is not correctly rounded, or a wrong tie rule, changes a code here."""
    qmax = O.QMAX[oq]
    rng = np.random.default_rng(7)
    rows = []
    if oq == O.INT8:
        targets = np.array([j + 0.5 for j in range(-127, 127)], np.float64)
    else:
        mags = O.e4m3_decode(np.arange(127, dtype=np.uint8))
        mids = (mags[:-1] + mags[1:]) / 2
        targets = np.concatenate([mids, -mids])
    for r in range(256):
        amax = np.float32(rng.uniform(1e-3, 10.0)) * np.float32(2.0 ** rng.integers(-20, 20))
        S = np.float32(amax / np.float32(qmax))
        base = (targets * np.float64(S)).astype(np.float32)
        row = np.concatenate([[amax], base, np.nextafter(base, np.float32(np.inf)),
                              np.nextafter(base, np.float32(-np.inf))]).astype(np.float32)
        row = np.clip(row, -amax, amax)
        pad = (-row.size) % 16
        rows.append(np.concatenate([row, np.zeros(pad, np.float32)]))
    width = max(r.size for r in rows)
    x = np.stack([np.pad(r, (0, width - r.size)) for r in rows]).astype(np.float32)
    log("near-ties %s rows=%d k=%d" % (oq, x.shape[0], x.shape[1]))
    c_ref, s_ref = O.quantize_rows(x, oq)
    c, sc = qr.qr_quantize_weights(dev(x), gq)
    torch.cuda.synchronize()
    assert_scales_equal(host(sc), s_ref, "near-tie scales")
    assert_codes_equal(host(c), c_ref, "near-tie codes")


def test_fp8_encoder_on_every_round_and_sticky_pattern():
    """Rows led by 448 have S = 1, so the codes are the E4M3 encodings of the raw values: this runs the
    device encoder on every sign/exponent/top-7-mantissa pattern with round and sticky variants."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    v = (hi[:, None] | lows[None, :]).ravel().view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    k = 4096
    per = k - 16
    nrows = (v.size + per - 1) // per
    x = np.zeros((nrows, k), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(nrows * per, np.float32)
    flat[:v.size] = v
    x[:, 16:] = flat.reshape(nrows, per)
    log("fp8 encoder patterns rows=%d" % nrows)
    c_ref, s_ref = O.quantize_rows(x, O.FP8)
    assert np.all(s_ref == 1.0)
    c, sc = qr.qr_quantize_weights(dev(x), qr.QR_FP8_E4M3)
    torch.cuda.synchronize()
    assert_scales_equal(host(sc), s_ref, "encoder scales")
    assert_codes_equal(host(c), c_ref, "encoder codes")


@pytest.mark.parametrize("oq,gq", QT)
def test_tiny_rows_take_exact_division(oq, gq):
    """Rows whose scale is below 2^-90 (and subnormal inputs) still match the oracle."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 64)) * 1e-30).astype(np.float32)
    x[1] *= np.float32(1e-8)
    x[2, :] = np.float32(1e-45) * rng.integers(-3, 4, 64).astype(np.float32)
    x[3, :] = np.float32(2.0 ** -126) * rng.uniform(-1, 1, 64).astype(np.float32)
    c_ref, s_ref = O.quantize_rows(x, oq)
    c, sc = qr.qr_quantize_weights(dev(x), gq)
    torch.cuda.synchronize()
    assert_scales_equal(host(sc), s_ref, "tiny scales")
    assert_codes_equal(host(c), c_ref, "tiny codes")


@pytest.mark.parametrize("oq,gq", QT)
def test_full_size_weight_quantization_sampled_rows(oq, gq):
    """7B-class linears at their full size, quantized in one launch each (as the benchmark does); the
    oracle checks a sample of rows (each row is independent)."""
    lin = {"int8": synth.QWEN_1P5B, "fp8": synth.DENSE_7B}["int8" if oq == O.INT8 else "fp8"]
    inp = synth.make_dense(lin, m_max=1)
    rng = np.random.default_rng(11)
    for name, w in inp.weights.items():
        log("full-size quantize %s %s %s" % (lin.name, name, w.shape))
        c, sc = qr.qr_quantize_weights(dev(w), gq)
        torch.cuda.synchronize()
        rows = np.sort(rng.choice(w.shape[0], 48, replace=False))
        rows[-1] = w.shape[0] - 1
        c_ref, s_ref = O.quantize_rows(w[rows], oq)
        assert_codes_equal(host(c)[rows], c_ref, name)
        assert_scales_equal(host(sc)[rows], s_ref, name)


def test_empty_and_errors():
    x = torch.zeros((0, 32), dtype=torch.float32, device="cuda")
    c, s = qr.qr_quantize_weights(x, qr.QR_INT8)
    assert c.shape == (0, 32)
    with pytest.raises(qr.QRError):
        qr.qr_quantize_weights(torch.zeros((4, 24), dtype=torch.float32, device="cuda"), qr.QR_INT8)
