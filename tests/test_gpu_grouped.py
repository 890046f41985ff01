"""GPU parity of the grouped (MoE) linear (a4) and the changed-code count (a5)."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O
from quantized_rollout_amd import synth

from gpu_util import (QT_NAMES, assert_codes_equal, assert_grouped_within_bound, assert_scales_equal,
                      assert_y_close, assert_y_within_bound, dev, grouped_exact, host, log)

pytestmark = pytest.mark.gpu

QT = [(O.INT8, qr.QR_INT8), (O.FP8, qr.QR_FP8_E4M3)]


def _expert_weights(E, n, k, oq, rng):
    wc = np.empty((E, n, k), np.uint8)
    ws = np.empty((E, n), np.float32)
    for e in range(E):
        wc[e], ws[e] = O.quantize_rows((rng.standard_normal((n, k)) * 0.02).astype(np.float32), oq)
    return wc, ws


@pytest.mark.parametrize("oq,gq", QT)
def test_grouped_parity_small(oq, gq):
    rng = np.random.default_rng(300)
    T, E, n, k, top = 40, 8, 72, 528, 3
    x = rng.standard_normal((T, k)).astype(np.float32)
    xc, xs = O.quantize_rows(x, oq, s_mode=O.S_MUL_RECIP)
    wc, ws = _expert_weights(E, n, k, oq, rng)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 5] = -100.0  # expert 5 gets no tokens
    off, rows = synth.route_top_k(logits, top)
    assert off[6] == off[5]
    log("grouped small %s E=%d rows=%d" % (oq, E, rows.size))
    y_ref = O.grouped_linear(oq, off, rows, xc, xs, wc, ws)
    y = qr.qr_w8a8_grouped_linear(gq, dev(off), dev(rows), rows.size, dev(xc), dev(xs), dev(wc), dev(ws))
    torch.cuda.synchronize()
    assert_y_close(host(y), y_ref, "grouped small")
    assert_grouped_within_bound(host(y), oq, off, rows, xc, xs, wc, ws, "grouped small")
    # INT8: outputs come from exact accumulators, so per-expert rows equal the plain linear's bitwise
    if oq == O.INT8:
        for e in range(E):
            r = rows[off[e]:off[e + 1]]
            if r.size == 0:
                continue
            ye = qr.qr_w8a8_linear(gq, dev(xc[r]), dev(xs[r]), dev(wc[e]), dev(ws[e]))
            torch.cuda.synchronize()
            assert np.array_equal(host(ye), host(y)[off[e]:off[e + 1]]), e


@pytest.mark.parametrize("oq,gq", QT)
def test_grouped_identity_rows_and_many_rows_per_expert(oq, gq):
    rng = np.random.default_rng(301)
    E, n, k = 3, 40, 272
    counts = [70, 0, 33]  # more rows than two token tiles, an empty expert
    total = sum(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    xc, xs = O.quantize_rows(rng.standard_normal((total, k)).astype(np.float32), oq, s_mode=O.S_MUL_RECIP)
    wc, ws = _expert_weights(E, n, k, oq, rng)
    y_ref = O.grouped_linear(oq, off, None, xc, xs, wc, ws)
    y = qr.qr_w8a8_grouped_linear(gq, dev(off), None, total, dev(xc), dev(xs), dev(wc), dev(ws))
    torch.cuda.synchronize()
    assert_y_close(host(y), y_ref, "grouped identity")
    assert_grouped_within_bound(host(y), oq, off, None, xc, xs, wc, ws, "grouped identity")


def test_grouped_debug_check_of_token_lists():
    """Debug mode checks the token lists on the device before the grouped linear runs: valid lists give the
    same output bits as without the check; each broken condition (first offset, last offset, a decreasing
    pair, a row id outside [0, x_rows)) is refused with QR_ERR_ARG and its name, and nothing is launched after
    it (the output buffer keeps its sentinel)."""
    rng = np.random.default_rng(302)
    E, n, k, x_rows = 4, 48, 256, 12
    xc, xs = O.quantize_rows(rng.standard_normal((x_rows, k)).astype(np.float32), O.INT8, s_mode=O.S_MUL_RECIP)
    wc, ws = _expert_weights(E, n, k, O.INT8, rng)
    off = np.array([0, 3, 3, 7, 10], np.int32)
    rows = np.array([0, 5, 11, 2, 2, 9, 4, 1, 7, 3], np.int32)
    total = int(off[-1])
    y0 = qr.qr_w8a8_grouped_linear(qr.QR_INT8, dev(off), dev(rows), total, dev(xc), dev(xs), dev(wc), dev(ws))
    torch.cuda.synchronize()
    bad_cases = [
        ("first", np.array([1, 3, 3, 7, 10], np.int32), rows, "expert_offsets[0] != 0"),
        ("last", np.array([0, 3, 3, 7, 9], np.int32), rows, "expert_offsets[num_experts] != total_rows"),
        ("decreasing", np.array([0, 5, 3, 7, 10], np.int32), rows, "expert_offsets decreases"),
        ("row id", off, np.array([0, 5, 11, 2, 12, 9, 4, 1, 7, 3], np.int32), "row id outside"),
        ("negative row id", off, np.array([0, 5, 11, 2, 2, 9, -1, 1, 7, 3], np.int32), "row id outside"),
    ]
    qr.qr_set_debug(True)
    try:
        y1 = qr.qr_w8a8_grouped_linear(qr.QR_INT8, dev(off), dev(rows), total, dev(xc), dev(xs), dev(wc), dev(ws))
        torch.cuda.synchronize()
        assert np.array_equal(host(y1), host(y0))
        for what, o, r, text in bad_cases:
            log("grouped debug check: %s" % what)
            y = torch.full((total, n), 7.0, dtype=torch.bfloat16, device="cuda")
            with pytest.raises(qr.QRError) as ei:
                qr.qr_w8a8_grouped_linear(qr.QR_INT8, dev(o), dev(r), total, dev(xc), dev(xs), dev(wc), dev(ws), y=y)
            assert ei.value.status == 1 and text in str(ei.value), (what, str(ei.value))
            torch.cuda.synchronize()
            assert bool((y == 7.0).all()), what
    finally:
        qr.qr_set_debug(False)
    # debug off again: the lists are trusted (and clamped) as before, no error
    qr.qr_w8a8_grouped_linear(qr.QR_INT8, dev(bad_cases[2][1]), dev(rows), total, dev(xc), dev(xs), dev(wc), dev(ws))
    torch.cuda.synchronize()


def _assert_rows_within_bound(y, keep, oq, off, rows, xc, xs, wc, ws, what):
    """The element-wise bound on the rows marked in keep (the others are checked by the caller)."""
    acc, bnd, xw = grouped_exact(oq, off, rows, xc, xs, wc, ws)
    assert_y_within_bound(y[keep], acc[keep], None, None, None if bnd is None else bnd[keep], what, xw=xw[keep])


# every compiled grouped variant: (64-byte steps per K slice, 16-channel tiles per block)
GROUPED_VARIANTS = [(4, 1), (4, 2), (4, 4), (8, 1), (8, 2), (2, 2)]


@pytest.mark.parametrize("u,tb", GROUPED_VARIANTS)
@pytest.mark.parametrize("waves", [None, 1])
def test_every_grouped_variant(u, tb, waves, monkeypatch):
    """Each variant forced through the launch overrides, with the LDS reduction over several waves and with one
    wave: channels not a multiple of the block's 16 tb, K with a partial last slice, experts with 0, 1, 17 and
    more than 32 rows (several passes over their weights), gathered rows and one row id out of range (its
    output row is zero)."""
    monkeypatch.setenv("QR_GROUPED_UNROLL", str(u))
    monkeypatch.setenv("QR_GROUPED_TILES", str(tb))
    if waves is not None:
        monkeypatch.setenv("QR_GROUPED_WAVES", str(waves))
    for oq, gq in QT:
        rng = np.random.default_rng(320 + 10 * u + tb + oq)
        T, E = 48, 5
        n, k = 16 * tb * 3 + 5, 64 * u * 3 + 48
        counts = [1, 0, 40, 17, 33]
        total = sum(counts)
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        rows = rng.integers(0, T, total).astype(np.int32)
        x = rng.standard_normal((T, k)).astype(np.float32)
        xc, xs = O.quantize_rows(x, oq, s_mode=O.S_MUL_RECIP)
        wc, ws = _expert_weights(E, n, k, oq, rng)
        log("grouped variant u=%d tb=%d waves=%s %s n=%d k=%d" % (u, tb, waves, oq, n, k))
        y_ref = O.grouped_linear(oq, off, rows, xc, xs, wc, ws)
        bad = rows.copy()
        bad[20] = T + 3  # out of range: that output row must be zero
        y = qr.qr_w8a8_grouped_linear(gq, dev(off), dev(bad), total, dev(xc), dev(xs), dev(wc), dev(ws))
        torch.cuda.synchronize()
        y = host(y)
        assert not y[20].any()
        y_ref[20] = 0
        assert_y_close(y, y_ref, "grouped variant u=%d tb=%d" % (u, tb))
        keep = np.ones(total, bool)
        keep[20] = False  # the out-of-range row is checked above (zeros)
        _assert_rows_within_bound(y, keep, oq, off, rows, xc, xs, wc, ws, "grouped variant u=%d tb=%d" % (u, tb))


def test_grouped_full_size_qwen3_moe_fp8_sampled():
    """The Qwen3-30B-A3B-shaped MoE layer: 128 experts, top-8 of 256 tokens, gate/up 2048->2x768 and down
    768->2048, FP8; every expert's full weights in one launch, the oracle checks sampled channels."""
    inp = synth.make_moe()
    rng = np.random.default_rng(302)
    xc, xs = O.quantize_rows(inp.x, O.FP8, s_mode=O.S_MUL_RECIP)
    hc, hs = O.quantize_rows(inp.h, O.FP8, s_mode=O.S_MUL_RECIP)
    for name, w, acts, scales, rows in (("gate_up", inp.w_gate_up, xc, xs, inp.row_ids),
                                        ("down", inp.w_down, hc, hs, None)):
        E, n, k = w.shape
        wc = np.empty((E, n, k), np.uint8)
        ws = np.empty((E, n), np.float32)
        for e in range(E):
            wc[e], ws[e] = O.quantize_rows(w[e], O.FP8)
        total = int(inp.expert_offsets[-1])
        log("moe %s E=%d n=%d k=%d rows=%d" % (name, E, n, k, total))
        y = qr.qr_w8a8_grouped_linear(qr.QR_FP8_E4M3, dev(inp.expert_offsets), None if rows is None else dev(rows),
                                      total, dev(acts), dev(scales), dev(wc), dev(ws))
        torch.cuda.synchronize()
        cols = np.sort(rng.choice(n, 16, replace=False))
        y_ref = O.grouped_linear(O.FP8, inp.expert_offsets, rows, acts, scales, wc[:, cols], ws[:, cols])
        assert_y_close(host(y)[:, cols], y_ref, "moe " + name)
        assert_grouped_within_bound(host(y)[:, cols], O.FP8, inp.expert_offsets, rows, acts, scales, wc[:, cols],
                                    ws[:, cols], "moe " + name)


@pytest.mark.parametrize("oq,gq", QT)
def test_count_code_changes_parity(oq, gq):
    inp = synth.make_requant(linears=["qkv"], row_limit=1024)
    w, w2, s = inp.w["qkv"], inp.w2["qkv"], inp.s["qkv"]
    for with_s in (False, True):
        a, sa = O.quantize_rows(w, oq, s=s if with_s else None)
        b, sb = O.quantize_rows(w2, oq, s=s if with_s else None)
        ref = O.count_code_changes(a, b, oq, sa, sb)
        got = qr.qr_count_code_changes(dev(a), dev(b), gq, dev(sa), dev(sb))
        torch.cuda.synchronize()
        assert list(host(got)) == list(ref), (with_s, host(got), ref)
    # ragged byte count (not a multiple of 16), equal inputs, FP8 signed zeros
    z = np.array([0x00, 0x80, 0x38, 0x38] * 9 + [0x80], np.uint8)
    z2 = np.array([0x80, 0x00, 0x38, 0xB8] * 9 + [0x00], np.uint8)
    for aa, bb in ((z, z2), (z, z)):
        ref = O.count_code_changes(aa, bb, oq)
        ta = torch.zeros(48, dtype=torch.uint8, device="cuda")
        tb = torch.zeros(48, dtype=torch.uint8, device="cuda")
        ta[:aa.size] = dev(aa)
        tb[:bb.size] = dev(bb)
        got = qr.qr_count_code_changes(ta[:aa.size], tb[:bb.size], gq)
        torch.cuda.synchronize()
        assert list(host(got)) == list(ref)


@pytest.fixture(scope="module")
def requant_7b():
    """Config 4 inputs: the four 7B-shaped linears' fp32 masters W ~ N(0, 0.02), W2 = fl32(W + dW) with
    dW ~ N(0, 1e-5), and per-input-channel s ~ U(0.5, 2) (seed 0)."""
    log("generating the 7B requantization inputs (fp32 W, W + dW, s)")
    return synth.make_requant()


@pytest.mark.parametrize("oq,gq", QT)
def test_requant_full_size_7b_all_linears(oq, gq, requant_7b):
    """The weight publish between RL steps on all four 7B linears at full size (qkv 4608x3584, o 3584x3584,
    gate/up 37888x3584, down 3584x18944; fp32 masters), with and without s: every code byte and scale of W and
    W + dW quantized on the GPU equals the oracle's, the changed-code triple counted on the GPU equals the
    oracle's over the whole tensor, and the fused requantize + diff publishes the same codes and triple."""
    inp = requant_7b
    for name in ("qkv", "o", "gate_up", "down"):
        w, w2, s = inp.w[name], inp.w2[name], inp.s[name]
        wd, w2d = dev(w), dev(w2)
        for with_s in (False, True):
            what = "requant 7b %s %s s=%s n=%d k=%d" % (name, QT_NAMES[oq], with_s, w.shape[0], w.shape[1])
            log(what)
            sd = dev(s) if with_s else None
            a, sa = qr.qr_quantize_weights(wd, gq, s=sd)
            b, sb = qr.qr_quantize_weights(w2d, gq, s=sd)
            got = qr.qr_count_code_changes(a, b, gq, sa, sb)
            c, sc, rc, o3 = qr.qr_requantize_weights(w2d, gq, a, sa, s=sd)
            torch.cuda.synchronize()
            ra, rsa = O.quantize_rows_threaded(w, oq, s=s if with_s else None)
            rb, rsb = O.quantize_rows_threaded(w2, oq, s=s if with_s else None)
            assert_codes_equal(host(a), ra, what + " codes of W")
            assert_scales_equal(host(sa), rsa, what + " scales of W")
            assert_codes_equal(host(b), rb, what + " codes of W + dW")
            assert_scales_equal(host(sb), rsb, what + " scales of W + dW")
            ref = O.count_code_changes(ra, rb, oq, rsa, rsb)
            log("  changed: %d bytes, %d values, %d scales of %d codes (%.4f%%)"
                % (ref[0], ref[1], ref[2], w.size, 100.0 * ref[0] / w.size))
            assert list(host(got)) == list(ref), (what, host(got), ref)
            assert list(host(o3)) == list(ref), (what, host(o3), ref)
            assert torch.equal(c, b) and torch.equal(sc, sb), what
            assert 0 < ref[0] < w.size
            del a, b, c, sa, sb, sc, rc
        del wd, w2d
        torch.cuda.empty_cache()


