"""The W8A8 linear that allocates nothing (qr_w8a8_linear_noalloc, for callers that cannot allocate device
memory): called through the C ABI, it gives the same y and accumulators, bit for bit, as qr_w8a8_linear with a
caller-owned workspace, on two calls in a row whose plans split K into the library's device scratch (the second
smaller than the first, so it runs on what the first left there), on a call that needs no scratch, and INT8
accumulators equal the oracle's on sampled columns."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O

from quantized_rollout_amd._binding import NOALLOC_SCRATCH_BYTES

from gpu_util import assert_fp8_acc_within_bound, dev, fp8_acc_bound, host, log

pytestmark = pytest.mark.gpu

GQ = {O.INT8: qr.QR_INT8, O.FP8: qr.QR_FP8_E4M3}


def _codes(rng, rows, k, oq):
    if oq == O.INT8:
        return rng.integers(-127, 128, (rows, k)).astype(np.int8).view(np.uint8)
    c = rng.integers(0, 256, (rows, k)).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return c


def _noalloc(oq, xc, xs, wc, ws, y, acc):
    L = qr.lib()
    m, k = xc.shape
    n = wc.shape[0]
    return L.qr_w8a8_linear_noalloc(GQ[oq], m, n, k, ctypes.c_void_p(xc.data_ptr()), ctypes.c_void_p(xs.data_ptr()),
                                    ctypes.c_void_p(wc.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                    ctypes.c_void_p(y.data_ptr()), qr.QR_BF16, ctypes.c_void_p(acc.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (m, n, k): the 7B down projection at m = 512 (63 MiB of partial sums), then the 1.5B o projection at m = 128
# (a smaller split), then one token (no scratch)
CALLS = [(512, 3584, 18944), (128, 1536, 1536), (1, 1536, 8960)]


@pytest.mark.parametrize("oq", [O.INT8, O.FP8])
def test_noalloc_linear_matches_the_workspace_linear(oq):
    rng = np.random.default_rng(900 + oq)
    wsp = qr.Workspace()
    for i, (m, n, k) in enumerate(CALLS):
        need = qr.qr_workspace_bytes(GQ[oq], m, n, k)
        log("noalloc %s m=%d n=%d k=%d scratch %d bytes" % (oq, m, n, k, need))
        assert (need > 0) == (i < 2) and need <= NOALLOC_SCRATCH_BYTES
        xc_h, wc_h = _codes(rng, m, k, oq), _codes(rng, n, k, oq)
        xs_h = rng.uniform(0.001, 0.01, m).astype(np.float32)
        ws_h = rng.uniform(0.0001, 0.001, n).astype(np.float32)
        xc, wc, xs, ws = dev(xc_h), dev(wc_h), dev(xs_h), dev(ws_h)
        y_ref, acc_ref = qr.qr_w8a8_linear(GQ[oq], xc, xs, wc, ws, acc_out=True, workspace=wsp)
        y = torch.full((m, n), 7.0, dtype=torch.bfloat16, device="cuda")
        acc = torch.full((m, n), 3, dtype=torch.int32 if oq == O.INT8 else torch.float32, device="cuda")
        rc = _noalloc(oq, xc, xs, wc, ws, y, acc)
        assert rc == 0, qr.lib().qr_last_error()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (m, n, k)
        assert torch.equal(acc.view(torch.int32), acc_ref.view(torch.int32)), (m, n, k)
        # sampled columns against the oracle (INT8 bit-exact, FP8 within the fp32 summation bound)
        cols = np.sort(rng.choice(n, 6, replace=False))
        _, acc_i, acc_f = O.linear(oq, xc_h, xs_h, wc_h[cols], ws_h[cols], O.BF16)
        got = host(acc)[:, cols]
        if oq == O.INT8:
            assert np.array_equal(got, acc_i), (m, n, k)
        else:
            assert_fp8_acc_within_bound(got, acc_f, fp8_acc_bound(xc_h, wc_h[cols]), "noalloc")
