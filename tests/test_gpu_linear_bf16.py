"""GPU parity of the linear on bfloat16 activations (next row: the activation quantization fused with the
linear). Against the oracle's activation quantizer followed by its linear: INT8 accumulators bit-exact, FP8
within the fp32 summation of exact products, y within the tolerance; with the activation quantization inside
the GEMV (decode batches) and as two steps through the workspace, with and without the invariant scale."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O

from gpu_util import (assert_fp8_acc_within_bound, assert_y_close, assert_y_within_bound, dev, fp8_acc_bound,
                      host, log)

pytestmark = pytest.mark.gpu

GQ = {O.INT8: qr.QR_INT8, O.FP8: qr.QR_FP8_E4M3}
E4M3 = O.e4m3_decode(np.arange(256, dtype=np.uint8))  # value of every code


def _bf16_bits(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _case(m, n, k, q, seed, with_s):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, min(4, k), replace=False)] *= np.float32(20)
    if m > 1:
        x[m - 1, :] = 0.0  # an all-zero token row: scale 1, codes 0
    xb = _bf16_bits(x)
    s = rng.uniform(0.5, 2.0, k).astype(np.float32) if with_s else None
    wc, ws = O.quantize_rows((rng.standard_normal((n, k)) * 0.02).astype(np.float32), q)
    return xb, s, wc, ws


# decode shapes (the 1.5B down and gate/up, ragged n and a k with a partial last 256-byte slice) and batches
# on both sides of the fusion threshold (the 17920-channel gate/up, 1120 workgroups, above the workgroup limit of
# the fused form, at two batches to keep the oracle quick; batches past 64 run the quantizer and then a GEMM plan)
SHAPES = [(1536, 8960, (1, 3, 4, 5, 16, 64)), (17920, 1536, (1, 4)), (200, 1040, (1, 3, 4, 5, 16, 64, 65, 130)),
          (37, 272, (1, 3, 4, 5, 16, 64, 300))]


@pytest.mark.parametrize("q", [O.INT8, O.FP8])
@pytest.mark.parametrize("with_s", [False, True])
@pytest.mark.parametrize("fuse_max", [None, 4])
def test_linear_bf16_parity(q, with_s, fuse_max, monkeypatch, capfd):
    if fuse_max is not None:
        monkeypatch.setenv("QR_FUSE_MAX_M", str(fuse_max))
    monkeypatch.setenv("QR_TRACE", "1")
    limit = 1 if fuse_max is None else fuse_max
    for i, (n, k, batches) in enumerate(SHAPES):
        for m in batches:
            xb, s, wc, ws = _case(m, n, k, q, 2000 + 10 * i + m, with_s)
            what = "linear_bf16 q=%d s=%s fuse_max=%s m=%d n=%d k=%d" % (q, with_s, fuse_max, m, n, k)
            log(what)
            xc, xs = O.quantize_rows(xb, q, s=s, s_mode=O.S_MUL_RECIP if with_s else None)
            y_ref, acc_i, acc_f = O.linear(q, xc, xs, wc, ws, O.BF16)
            y, acc = qr.qr_w8a8_linear_bf16(GQ[q], dev(xb), dev(wc), dev(ws), s=None if s is None else dev(s),
                                            acc_out=True)
            torch.cuda.synchronize()
            acc = host(acc)
            bound = None
            if q == O.INT8:
                assert np.array_equal(acc, acc_i), what
            else:
                # FP8 accumulators on the matrix cores: within the measured truncation of the instructions plus
                # an fp32 sum in any order of the exact value
                bound = fp8_acc_bound(xc, wc)
                assert_fp8_acc_within_bound(acc, acc_f, bound, what)
            assert_y_within_bound(host(y), acc_f, xs, ws, bound, what)
            assert_y_close(host(y), y_ref, what)
            err = capfd.readouterr().err
            # the in-kernel quantization: one token tile, FP8 rows up to k = 8192, at most 256 workgroups
            fused = m <= limit and (q == O.INT8 or k <= 8192) and n < 16384
            assert ("fused=%d" % fused) in err or m > 16, (what, err)


def test_linear_bf16_equals_the_two_steps_bit_for_bit():
    """The fused path and the activation quantizer followed by the linear give the same bytes (y and
    accumulators), INT8 and FP8, at m = 1."""
    for q in (O.INT8, O.FP8):
        xb, s, wc, ws = _case(1, 1536, 8960, q, 2100 + q, True)
        x, sd, wcd, wsd = dev(xb), dev(s), dev(wc), dev(ws)
        y1, a1 = qr.qr_w8a8_linear_bf16(GQ[q], x, wcd, wsd, s=sd, acc_out=True)
        xc, xs = qr.qr_quantize_acts(x, GQ[q], s=sd)
        y2, a2 = qr.qr_w8a8_linear(GQ[q], xc, xs, wcd, wsd, acc_out=True)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(a1, a2)
