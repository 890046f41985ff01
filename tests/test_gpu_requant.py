"""GPU parity of the requantize + diff row (one publish of W + dW against the previous publish): codes, scales,
per-row change triples and their sums bit-exact against the oracle, in place and out of place, on every
quantizer launch shape (rows of one wavefront, of a workgroup, and longer than the register budget)."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O

from gpu_util import assert_codes_equal, assert_scales_equal, dev, host, log

pytestmark = pytest.mark.gpu

GQ = {O.INT8: qr.QR_INT8, O.FP8: qr.QR_FP8_E4M3}


def _bf16_bits(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _masters(n, k, seed, bf16):
    """W and W + dW (a small update: some codes change, most do not), fp32 or bfloat16 bits."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :] = 0.0  # an all-zero row stays all zero
    w2 = w + (rng.standard_normal((n, k)) * 2e-4).astype(np.float32)
    w2[0, :] = 0.0
    if n > 2:
        w2[2, 0] = np.float32(0.5)  # a row whose scale changes
    if bf16:
        return _bf16_bits(w), _bf16_bits(w2)
    return w, w2


# k per input dtype: one-wavefront rows (4 per workgroup), 256- and 1024-lane rows, and rows longer than the
# 1024-lane register budget (the remainder is re-read, and its previous codes loaded one chunk at a time)
SHAPES = [(9, 96), (5, 8960), (3, 18944), (2, 70016)]


@pytest.mark.parametrize("q", [O.INT8, O.FP8])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("in_place", [False, True])
def test_requantize_parity(q, bf16, in_place):
    for i, (n, k) in enumerate(SHAPES):
        w, w2 = _masters(n, k, 300 + i, bf16)
        s = np.random.default_rng(400 + i).uniform(0.5, 2.0, k).astype(np.float32) if i % 2 else None
        log("requantize q=%d bf16=%s in_place=%s n=%d k=%d s=%s" % (q, bf16, in_place, n, k, s is not None))
        pc, ps = O.quantize_rows(w, q, s=s)
        c_ref, s_ref, rc_ref, o3_ref = O.requantize_weights(w2, q, pc, ps, s=s)
        prev_c, prev_s = dev(pc), dev(ps)
        c, sc, rc, o3 = qr.qr_requantize_weights(dev(w2), GQ[q], prev_c, prev_s, s=None if s is None else dev(s),
                                                 in_place=in_place)
        torch.cuda.synchronize()
        assert_codes_equal(host(c), c_ref, "requant codes n=%d k=%d" % (n, k))
        assert_scales_equal(host(sc), s_ref, "requant scales n=%d k=%d" % (n, k))
        assert np.array_equal(host(rc), rc_ref), (host(rc), rc_ref)
        assert np.array_equal(host(o3), o3_ref), (host(o3), o3_ref)
        if in_place:
            assert c.data_ptr() == prev_c.data_ptr() and sc.data_ptr() == prev_s.data_ptr()
        else:
            assert np.array_equal(host(prev_c), pc) and np.array_equal(host(prev_s), ps)  # left untouched
        assert 0 < o3_ref[0] < n * k and o3_ref[2] >= (1 if n > 2 else 0)


def test_requantize_no_rows_zeroes_out3():
    w = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    pc = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    ps = torch.empty((0,), dtype=torch.float32, device="cuda")
    out3 = torch.full((3,), 77, dtype=torch.int64, device="cuda")
    qr.qr_requantize_weights(w, qr.QR_INT8, pc, ps, out3=out3)
    torch.cuda.synchronize()
    assert host(out3).tolist() == [0, 0, 0]


@pytest.mark.parametrize("q", [O.INT8, O.FP8])
def test_requantize_full_size_7b_gate_up(q):
    """The 7B gate/up (37888 x 3584) from bf16 masters, in place: the whole-tensor triple equals the separate
    quantize and count calls (each parity-tested against the oracle); sampled rows against the oracle."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    n, k = 37888, 3584
    w = (torch.randn((n, k), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (w.float() + torch.randn((n, k), generator=g, device="cuda") * 2e-4).to(torch.bfloat16)
    prev_c, prev_s = qr.qr_quantize_weights(w, GQ[q])
    ref_c, ref_s = qr.qr_quantize_weights(w2, GQ[q])
    ref3 = qr.qr_count_code_changes(prev_c, ref_c, GQ[q], prev_s, ref_s)
    keep_c, keep_s = prev_c.clone(), prev_s.clone()
    c, sc, rc, o3 = qr.qr_requantize_weights(w2, GQ[q], prev_c, prev_s, in_place=True)
    torch.cuda.synchronize()
    assert torch.equal(c, ref_c) and torch.equal(sc, ref_s)
    assert torch.equal(o3, ref3), (o3, ref3)
    assert torch.equal(rc.sum(dim=0, dtype=torch.int64), o3)
    rows = np.sort(np.random.default_rng(6).choice(n, 16, replace=False))
    w2_rows = host(w2[rows].view(torch.int16)).view(np.uint16)
    _, _, rc_ref, _ = O.requantize_weights(w2_rows, q, host(keep_c)[rows], host(keep_s)[rows])
    assert np.array_equal(host(rc)[rows], rc_ref)
