"""GPU parity of the W4A16 row (group-wise INT4 weights, bfloat16 activations): the quantizer's packed codes and
scales bit-exact against the oracle, the linear within 1e-2 * max|ref| of the oracle's exact value (and
within fp32 summation error for fp32 output), every launch variant, the full-size 7B shape sampled."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O

from gpu_util import assert_codes_equal, assert_scales_equal, assert_y_close, dev, host, log

pytestmark = pytest.mark.gpu

G = O.W4_GROUP


def _bf16_bits(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _weights(n, k, seed, bf16):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :G] = 0.0                      # an all-zero group
    w[min(1, n - 1), G - 5] = 0.3       # one large value in a group
    if n > 2:
        w[2, :] *= np.float32(1e-30)    # tiny values: scales far below 2^-90 take the plain division
    return _bf16_bits(w) if bf16 else w


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("with_s", [False, True])
def test_w4_quantizer_parity(bf16, with_s):
    for i, (n, k) in enumerate([(3, 128), (37, 384), (200, 1536), (64, 18944)]):
        w = _weights(n, k, 500 + i, bf16)
        s = np.random.default_rng(600 + i).uniform(0.5, 2.0, k).astype(np.float32) if with_s else None
        log("w4 quantize bf16=%s s=%s n=%d k=%d" % (bf16, with_s, n, k))
        c_ref, s_ref = O.quantize_w4(w, s=s)
        c, sc = qr.qr_quantize_weights_w4(dev(w), s=None if s is None else dev(s))
        torch.cuda.synchronize()
        assert_codes_equal(host(c), c_ref, "w4 codes n=%d k=%d" % (n, k))
        assert_scales_equal(host(sc).ravel(), s_ref.ravel(), "w4 scales n=%d k=%d" % (n, k))


def _linear_case(m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, min(4, k), replace=False)] *= np.float32(20)
    xb = _bf16_bits(x)
    codes, scales = O.quantize_w4((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    return xb, codes, scales


SHAPES = [(1, 16, 128), (1, 37, 384), (5, 200, 1536), (16, 1000, 3584), (17, 64, 1024), (40, 96, 2048),
          (1, 1536, 8960), (3, 300, 18944)]


def _expected_plan(m, k, env):
    """(ring, x_lds) the library must choose for forced knobs: the LDS ring when the activation rows, the waves'
    rings and partials fit in 160 KiB; else activations in LDS when asked for (every register-stage plan here
    sets QR_W4_XLDS; a ring plan falls back only where the rows alone exceed 64 KiB) and rows and partials fit
    in 64 KiB."""
    tiles, waves, wk = env.get("QR_W4_TILES", 1), env["QR_W4_WAVES"], env["QR_W4_WK"]
    depth = env.get("QR_W4_DEPTH", 2)
    xb = min(m, 16) * (2 * k + 16)
    part = waves * 1024 if wk > 1 else 0
    if env.get("QR_W4_RING", 1) and xb + waves * max(depth, 2) * 1280 + part <= 163840:
        return 1, 1
    return 0, int(env.get("QR_W4_XLDS", 1) != 0 and xb + part * tiles <= 65536)


PLANS = [None,
         dict(QR_W4_RING=1, QR_W4_WAVES=1, QR_W4_WK=1, QR_W4_DEPTH=2),
         dict(QR_W4_RING=1, QR_W4_WAVES=8, QR_W4_WK=1, QR_W4_DEPTH=4),
         dict(QR_W4_RING=1, QR_W4_WAVES=16, QR_W4_WK=16, QR_W4_DEPTH=4),
         dict(QR_W4_RING=1, QR_W4_WAVES=6, QR_W4_WK=3, QR_W4_DEPTH=8),
         dict(QR_W4_RING=1, QR_W4_WAVES=4, QR_W4_WK=2, QR_W4_DEPTH=2),
         dict(QR_W4_RING=0, QR_W4_TILES=1, QR_W4_WAVES=3, QR_W4_WK=3, QR_W4_DEPTH=2, QR_W4_XLDS=1),
         dict(QR_W4_RING=0, QR_W4_TILES=2, QR_W4_WAVES=8, QR_W4_WK=4, QR_W4_DEPTH=2, QR_W4_XLDS=0),
         dict(QR_W4_RING=0, QR_W4_TILES=2, QR_W4_WAVES=5, QR_W4_WK=5, QR_W4_DEPTH=1, QR_W4_XLDS=1),
         dict(QR_W4_RING=0, QR_W4_TILES=4, QR_W4_WAVES=2, QR_W4_WK=1, QR_W4_DEPTH=1, QR_W4_XLDS=1),
         dict(QR_W4_RING=0, QR_W4_TILES=4, QR_W4_WAVES=16, QR_W4_WK=8, QR_W4_DEPTH=1, QR_W4_XLDS=0)]


@pytest.mark.parametrize("plan", PLANS, ids=lambda p: "default" if p is None else "-".join(
    "%s%d" % (k[6:].lower(), v) for k, v in p.items()))
def test_w4a16_linear_parity(plan, monkeypatch, capfd):
    for key, v in (plan or {}).items():
        monkeypatch.setenv(key, str(v))
    monkeypatch.setenv("QR_TRACE", "1")
    for i, (m, n, k) in enumerate(SHAPES):
        xb, codes, scales = _linear_case(m, n, k, 700 + i)
        log("w4a16 plan=%s m=%d n=%d k=%d" % (plan, m, n, k))
        y_ref, y64 = O.w4a16_linear(xb, codes, scales)
        y = qr.qr_w4a16_linear(dev(xb), dev(codes), dev(scales))
        yf = qr.qr_w4a16_linear(dev(xb), dev(codes), dev(scales), y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_y_close(host(y), y_ref, "w4a16 bf16 m=%d n=%d k=%d" % (m, n, k))
        # fp32 output: products are exact, so only the fp32 sums differ from the exact value
        bound = 1e-5 * np.abs(y64).max() + 1e-30
        assert np.abs(host(yf).astype(np.float64) - y64).max() <= bound, (m, n, k)
        err = capfd.readouterr().err
        if plan is not None:
            ring, xlds = _expected_plan(m, k, plan)
            want = "ring=%d tiles=%d waves=%d wk=%d" % (ring, plan.get("QR_W4_TILES", 1) if not ring else 1,
                                                        plan["QR_W4_WAVES"], plan["QR_W4_WK"])
            assert want in err and ("xlds=%d" % xlds) in err, (want, err)


def test_w4a16_deterministic_and_batch_rows_independent():
    xb, codes, scales = _linear_case(33, 300, 1536, 800)
    a = host(qr.qr_w4a16_linear(dev(xb), dev(codes), dev(scales)))
    b = host(qr.qr_w4a16_linear(dev(xb), dev(codes), dev(scales)))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)
    # every row depends only on its own activations: a batch prefix gives the same rows bit for bit
    for m in (1, 16, 17):
        p = host(qr.qr_w4a16_linear(dev(xb[:m]), dev(codes), dev(scales)))
        assert np.array_equal(p, a[:m]), m


def test_w4_full_size_7b_gate_up_sampled():
    """The 7B-shaped gate/up (37888 x 3584) quantized on the GPU from bf16 masters: sampled rows' codes and
    scales against the oracle, then the decode product at m = 1 and 16 on sampled channels."""
    rng = np.random.default_rng(900)
    n, k = 37888, 3584
    wb = _bf16_bits((rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    c, sc = qr.qr_quantize_weights_w4(dev(wb))
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(n, 24, replace=False))
    c_ref, s_ref = O.quantize_w4(wb[rows])
    assert_codes_equal(host(c)[rows], c_ref, "w4 7b codes")
    assert_scales_equal(host(sc)[rows].ravel(), s_ref.ravel(), "w4 7b scales")
    for m in (1, 16):
        xb = _bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        y = host(qr.qr_w4a16_linear(dev(xb), c, sc))
        torch.cuda.synchronize()
        y_ref, _ = O.w4a16_linear(xb, c_ref, s_ref)
        assert_y_close(y[:, rows], y_ref, "w4a16 7b m=%d" % m)


def test_w4_errors():
    t = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        qr.qr_quantize_weights_w4(t)  # k not a multiple of the group
    # the C ABI itself rejects it too, before any launch
    L = qr.lib()
    c = torch.empty((4, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty((4, 1), dtype=torch.float32, device="cuda")
    rc = L.qr_quantize_weights_w4(t.data_ptr(), qr.QR_F32, 4, 100, None, c.data_ptr(), s.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 2  # QR_ERR_UNSUPPORTED
    y = qr.qr_w4a16_linear(torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"),
                           torch.zeros((8, 64), dtype=torch.uint8, device="cuda"),
                           torch.zeros((8, 1), dtype=torch.float32, device="cuda"))
    assert y.shape == (0, 8)
