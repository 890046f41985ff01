"""GPU parity of the RMSNorm producer of a linear's quantized input (the next row that fuses the token-wise
activation quantizer into the kernel producing its input).

h, its codes and its scales are compared bit for bit with the oracle's RMSNorm followed by the oracle's
activation quantizer. Both sides take the normalization in fp64 and round once to bfloat16; the sums of squares
are exact per term and differ only in summation order (an error below 2^-40 relative for these row lengths),
so h could differ only where the fp64 value lies that close to a bfloat16 rounding boundary."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O
from quantized_rollout_amd import synth

from gpu_util import assert_codes_equal, assert_scales_equal, dev, host, log

pytestmark = pytest.mark.gpu

QT = [(O.INT8, qr.QR_INT8), (O.FP8, qr.QR_FP8_E4M3)]


def _check(oq, gq, x, gamma, eps, s, what, want_h=True):
    c_ref, s_ref, h_ref = O.rmsnorm_quantize(x, gamma, np.float32(eps), oq, s=s)
    log("rmsnorm_quantize %s" % what)
    out = qr.qr_rmsnorm_quantize(dev(x), dev(gamma), eps, gq, s=None if s is None else dev(s), want_h=want_h)
    torch.cuda.synchronize()
    if want_h:
        h = host(out[2])
        if not np.array_equal(h, h_ref):
            bad = np.argwhere(h != h_ref)
            raise AssertionError("%s: %d h values differ, first at %s" % (what, len(bad), tuple(bad[0])))
    assert_codes_equal(host(out[0]), c_ref, what + " codes")
    assert_scales_equal(host(out[1]), s_ref, what + " scales")
    return c_ref, s_ref


@pytest.mark.parametrize("oq,gq", QT)
@pytest.mark.parametrize("rows,k", [(1, 3584), (16, 3584), (64, 1536), (2048, 3584), (3, 16), (130, 2048),
                                    (7, 18944)])
@pytest.mark.parametrize("with_s", [False, True])
def test_rmsnorm_quantize_parity(oq, gq, rows, k, with_s):
    """Hidden states of the pages' models (1.5B: 1536, 7B: 3584, Qwen3-30B-A3B: 2048) at decode and rollout
    batches, a tiny ragged row, and a row of 18944 (the 7B intermediate size) whose teams hold it in registers;
    eps 1e-6, with and without the invariant scale."""
    inp = synth.make_norm_inputs(rows, k, seed=800 + rows + k)
    _check(oq, gq, inp.x, inp.gamma, 1e-6, inp.s if with_s else None,
           "%s rows=%d k=%d s=%s" % (oq, rows, k, with_s))


@pytest.mark.parametrize("lanes", [64, 128, 256, 512, 1024])
def test_every_team_width(lanes, monkeypatch):
    """Every team width forced on a row longer than the chunks a lane holds at 64 lanes (re-read and recomputed
    for the codes), on a short one, and on a ragged row count."""
    monkeypatch.setenv("QR_QUANT_THREADS", str(lanes))
    for rows, k in ((5, 9216), (9, 256), (1, 3584)):
        inp = synth.make_norm_inputs(rows, k, seed=900 + lanes + k)
        for oq, gq in QT:
            _check(oq, gq, inp.x, inp.gamma, 1e-5, inp.s, "lanes=%d %s rows=%d k=%d" % (lanes, oq, rows, k))


@pytest.mark.parametrize("oq,gq", QT)
def test_edge_rows(oq, gq):
    """An all-zero row (eps = 0: q = 0, no NaN; eps > 0: zeros), -0 entries, a row of one non-zero entry, a row
    at 1e30 whose squares overflow fp32 but not fp64, a row near the smallest normal bfloat16, a constant row,
    and eps large against the mean square."""
    k = 512
    x = np.zeros((8, k), np.float32)
    x[1, ::3] = -0.0
    x[2, 17] = -3.5
    x[3] = np.linspace(-1e30, 1e30, k, dtype=np.float32)
    x[4] = np.linspace(-1e-37, 2e-37, k, dtype=np.float32)
    x[5] = 0.75
    x[6] = np.linspace(-2, 2, k, dtype=np.float32)
    x[7] = np.linspace(-1e-3, 1e-3, k, dtype=np.float32)
    xb = synth.f32_to_bf16_bits(x)
    rng = np.random.default_rng(31)
    gamma = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.uniform(0.5, 1.5, k).astype(np.float32)))
    for eps in (0.0, 1e-6, 4.0):
        c, sc = _check(oq, gq, xb, gamma, eps, None, "edge rows %s eps=%g" % (oq, eps))
        assert not c[0].any() and sc[0] == 1.0


@pytest.mark.parametrize("oq,gq", QT)
def test_fused_equals_norm_then_quantizer(oq, gq):
    """The fused call's codes and scales are the library's own activation quantizer applied to the h it writes,
    and leaving h out changes nothing."""
    inp = synth.make_norm_inputs(64, 3584, seed=77)
    x, g, s = dev(inp.x), dev(inp.gamma), dev(inp.s)
    c1, s1, h = qr.qr_rmsnorm_quantize(x, g, 1e-6, gq, s=s, want_h=True)
    c2, s2 = qr.qr_rmsnorm_quantize(x, g, 1e-6, gq, s=s)
    c3, s3 = qr.qr_quantize_acts(h, gq, s=s)
    torch.cuda.synchronize()
    for c, sc in ((c2, s2), (c3, s3)):
        assert torch.equal(c1, c) and torch.equal(s1.view(torch.int32), sc.view(torch.int32))
