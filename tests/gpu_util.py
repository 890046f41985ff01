"""Helpers for the GPU parity tests: host<->device marshalling and the comparison gates.

Every input handed to the GPU comes from ``quantized_rollout_amd.synth`` or from the oracle; expected values
come only from the oracle.
"""
import sys

import numpy as np
import torch

from oracle import core as O
from quantized_rollout_amd import synth

QT_NAMES = {O.INT8: "int8", O.FP8: "fp8"}
REL_TOL = 1e-2  # max|y_gpu - y_ref| <= 1e-2 * max|y_ref| per tensor


def log(msg):
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def dev(a):
    """numpy -> CUDA tensor. uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t):
    """CUDA tensor -> numpy (bfloat16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def y_as_f64(y):
    if y.dtype == np.uint16:
        return synth.bf16_bits_to_f32(y).astype(np.float64)
    return y.astype(np.float64)


def assert_y_close(y_gpu, y_ref, what=""):
    g, r = y_as_f64(y_gpu), y_as_f64(y_ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), what
    ref_max = np.abs(r).max() if r.size else 0.0
    err = np.abs(g - r).max() if r.size else 0.0
    assert err <= REL_TOL * ref_max, "%s: max|err| %.3g > 1e-2 * max|ref| %.3g" % (what, err, ref_max)
    return err, ref_max


def assert_codes_equal(c_gpu, c_ref, what=""):
    if not np.array_equal(c_gpu, c_ref):
        bad = np.argwhere(c_gpu != c_ref)
        i = tuple(bad[0])
        raise AssertionError("%s: %d codes differ, first at %s: gpu 0x%02x oracle 0x%02x"
                             % (what, len(bad), i, c_gpu[i], c_ref[i]))


def assert_scales_equal(s_gpu, s_ref, what=""):
    a, b = s_gpu.view(np.uint32), s_ref.view(np.uint32)
    if not np.array_equal(a, b):
        i = int(np.argwhere(a != b)[0][0])
        raise AssertionError("%s: %d scales differ, first at %d: gpu %r oracle %r"
                             % (what, int((a != b).sum()), i, s_gpu[i], s_ref[i]))
