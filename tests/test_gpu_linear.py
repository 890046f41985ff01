"""GPU parity of the W8A8 linear (a3): INT8 accumulators bit-exact, outputs within 1e-2 * max|ref|, for
both kernels (small-m GEMV with split-K, tiled GEMM), ragged shapes, the toy and full-size workloads."""
import numpy as np
import pytest
import torch

import quantized_rollout_amd as qr
from oracle import core as O
from quantized_rollout_amd import synth

from gpu_util import (assert_fp8_acc_within_bound, assert_y_close, assert_y_within_bound, dev, fp8_acc_bound,
                      host, log)

pytestmark = pytest.mark.gpu

QT = [(O.INT8, qr.QR_INT8), (O.FP8, qr.QR_FP8_E4M3)]
GQ = {O.INT8: qr.QR_INT8, O.FP8: qr.QR_FP8_E4M3}


def _quantized_operands(m, n, k, oq, seed):
    """Activations (with outlier channels) and weights, quantized by the oracle."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, rng.choice(k, min(4, k), replace=False)] *= np.float32(20)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    xc, xs = O.quantize_rows(x, oq, s_mode=O.S_MUL_RECIP)
    wc, ws = O.quantize_rows(w, oq)
    return xc, xs, wc, ws


def _run(oq, xc, xs, wc, ws, y_dtype=torch.bfloat16):
    y, acc = qr.qr_w8a8_linear(GQ[oq], dev(xc), dev(xs), dev(wc), dev(ws), y_dtype=y_dtype, acc_out=True)
    torch.cuda.synchronize()
    return host(y), host(acc)


def _check(oq, xc, xs, wc, ws, what, y_type=O.BF16):
    y_ref, acc_i, acc_f = O.linear(oq, xc, xs, wc, ws, y_type)
    y, acc = _run(oq, xc, xs, wc, ws, torch.bfloat16 if y_type == O.BF16 else torch.float32)
    if oq == O.INT8:
        if not np.array_equal(acc, acc_i):
            bad = np.argwhere(acc != acc_i)
            i = tuple(bad[0])
            raise AssertionError("%s: %d INT32 accumulators differ, first %s gpu %d oracle %d"
                                 % (what, len(bad), i, acc[i], acc_i[i]))
    bound = fp8_acc_bound(xc, wc) if oq == O.FP8 else None
    if oq == O.FP8:
        # FP8 accumulators on the matrix cores: within the measured truncation of the instructions plus an fp32
        # sum in any order of the exact value
        assert_fp8_acc_within_bound(acc, acc_f, bound, what)
    assert_y_within_bound(y, acc_f, xs, ws, bound, what)
    assert_y_close(y, y_ref, what)


# (m, n, k): several 16-column tiles, ragged n (not a multiple of 16 / 128), ragged k (not a multiple of
# the 256-byte step), every GEMV token-tile count (1, 2, 4), split-K and no split, and the tiled GEMM
SHAPES = [(1, 16, 16), (4, 512, 256), (3, 37, 272), (16, 200, 1552), (17, 96, 512), (33, 130, 784),
          (64, 64, 4096), (1, 1536, 8960), (16, 2048, 1536), (65, 150, 528), (128, 256, 1024),
          (300, 333, 1040), (512, 384, 2048)]


@pytest.mark.parametrize("oq,gq", QT)
def test_linear_parity_shapes(oq, gq):
    for i, (m, n, k) in enumerate(SHAPES):
        log("linear %s m=%d n=%d k=%d" % (oq, m, n, k))
        xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=200 + i)
        _check(oq, xc, xs, wc, ws, "%s m=%d n=%d k=%d" % (oq, m, n, k))


@pytest.mark.parametrize("oq,gq", QT)
def test_linear_fp32_output(oq, gq):
    xc, xs, wc, ws = _quantized_operands(8, 96, 512, oq, seed=5)
    _check(oq, xc, xs, wc, ws, "fp32 out", y_type=O.F32)


def test_toy_workload_int8():
    """The toy INT8 linear: M=4, K=256, N=512, fp32 weights N(0, 0.02), activations N(0, 1) with 4 outlier
    channels x20, seed 0 -- quantized on the GPU and checked end to end (codes, accumulators, outputs)."""
    inp = synth.make_dense(synth.TOY)
    w, x = inp.weights["toy"], inp.acts["toy"]
    wc_ref, ws_ref = O.quantize_rows(w, O.INT8)
    xc_ref, xs_ref = O.quantize_rows(x, O.INT8, s_mode=O.S_MUL_RECIP)
    y_ref, acc_ref, _ = O.linear(O.INT8, xc_ref, xs_ref, wc_ref, ws_ref, O.BF16)
    wc, ws = qr.qr_quantize_weights(dev(w), qr.QR_INT8)
    xc, xs = qr.qr_quantize_acts(dev(x), qr.QR_INT8)
    y, acc = qr.qr_w8a8_linear(qr.QR_INT8, xc, xs, wc, ws, acc_out=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(wc), wc_ref) and np.array_equal(host(xc), xc_ref)
    assert np.array_equal(host(acc), acc_ref)
    assert_y_close(host(y), y_ref, "toy")
    # the quantized product stays close to the unquantized one despite the outlier channels
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    yf = synth.bf16_bits_to_f32(host(y)).astype(np.float64)
    assert np.abs(yf - ref).max() <= 0.05 * np.abs(ref).max()


def test_int8_batch_prefix_and_determinism():
    """INT8: row i of y is bitwise the same for every batch prefix (exact accumulators, elementwise
    epilogue) and for repeated calls; crosses the GEMV/GEMM switch."""
    xc, xs, wc, ws = _quantized_operands(200, 272, 1040, O.INT8, seed=77)
    y_full, _ = _run(O.INT8, xc, xs, wc, ws)
    y_again, _ = _run(O.INT8, xc, xs, wc, ws)
    assert np.array_equal(y_full, y_again)
    for m in (1, 5, 16, 17, 64, 65, 129):
        y, _ = _run(O.INT8, xc[:m], xs[:m], wc, ws)
        assert np.array_equal(y, y_full[:m]), m


def test_fp8_determinism():
    xc, xs, wc, ws = _quantized_operands(16, 1536, 8960, O.FP8, seed=78)
    a, _ = _run(O.FP8, xc, xs, wc, ws)
    b, _ = _run(O.FP8, xc, xs, wc, ws)
    assert np.array_equal(a, b)


def test_no_workspace_needed():
    """A plan that reduces inside its blocks works with no workspace at all (7B o shape at m = 16)."""
    xc, xs, wc, ws = _quantized_operands(16, 3584, 3584, O.INT8, seed=79)
    assert qr.qr_workspace_bytes(qr.QR_INT8, 16, 3584, 3584) == 0
    y_ref, acc_i, _ = O.linear(O.INT8, xc, xs, wc, ws, O.BF16)
    y = torch.empty((16, 3584), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((16, 3584), dtype=torch.int32, device="cuda")
    L = qr.lib()
    ops = [dev(a) for a in (xc, xs, wc, ws)]  # kept alive until the kernel has run
    rc = L.qr_w8a8_linear(qr.QR_INT8, 16, 3584, 3584, *[t.data_ptr() for t in ops], y.data_ptr(), qr.QR_BF16,
                          acc.data_ptr(), None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), acc_i)
    assert_y_close(host(y), y_ref, "no workspace")


@pytest.mark.parametrize("splits", [None, 2, 3, 16])
def test_gemv_split_k(splits, monkeypatch, capfd):
    """The GEMV with K split across blocks (partial sums in the workspace, added in split order): INT8
    accumulators bit-exact, FP8 within the fp32 bound and deterministic, on the 1.5B down shape at every
    decode batch and on a ragged shape with a partial last slice."""
    if splits is not None:
        monkeypatch.setenv("QR_GEMV_SPLITS", str(splits))
    monkeypatch.setenv("QR_TRACE", "1")
    for i, (m, n, k) in enumerate([(1, 1536, 8960), (16, 1536, 8960), (64, 1536, 8960), (37, 200, 4368)]):
        for oq in (O.INT8, O.FP8):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1500 + 10 * i + oq)
            what = "gemv split=%s %s m=%d n=%d k=%d" % (splits, oq, m, n, k)
            log(what)
            _check(oq, xc, xs, wc, ws, what)
            if oq == O.FP8:
                a, _ = _run(oq, xc, xs, wc, ws)
                b, _ = _run(oq, xc, xs, wc, ws)
                assert np.array_equal(a, b), what
            err = capfd.readouterr().err
            assert "kind=0" in err, err
            if splits is not None:
                u = 4 if "unroll=4" in err else int(err.split("unroll=")[1].split()[0])
                slices = -(-k // (64 * u))
                per = -(-slices // min(splits, slices))
                assert "splits=%d " % (-(-slices // per)) in err, err
            elif n == 1536:
                assert ("splits=2 " if m > 32 else "splits=1 ") in err, err


@pytest.mark.parametrize("ks", [2, 4, 8])
def test_gemv_k_parts(ks, monkeypatch, capfd):
    """K cut into ks parts inside each MFMA (tiles of 16 / ks channels): INT8 accumulators bit-exact, FP8 within
    the tolerance, at m = 1 up to 16 / ks tokens, with channels not a multiple of the tile, K parts with a partial
    last slice, and the bfloat16-activation entry point (the activation quantization inside the kernel)."""
    monkeypatch.setenv("QR_GEMV_KSUB", str(ks))
    monkeypatch.setenv("QR_FUSE_MAX_BLOCKS", "1024")  # the in-kernel quantization also on 8 x 96 workgroups
    monkeypatch.setenv("QR_TRACE", "1")
    shapes = [(1, 1536, 8960), (1, 70, 1664), (min(4, 16 // ks), 100, 2048), (16 // ks, 37, 3584), (1, 3, 128 * ks)]
    for i, (m, n, k) in enumerate(shapes):
        for oq in (O.INT8, O.FP8):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1700 + 10 * i + oq + ks)
            what = "gemv ksub=%d %s m=%d n=%d k=%d" % (ks, oq, m, n, k)
            log(what)
            _check(oq, xc, xs, wc, ws, what)
            err = capfd.readouterr().err
            assert "ksub=%d " % ks in err, err
    # the entry point on bfloat16 activations at m = 1 (quantization inside the kernel)
    rng = np.random.default_rng(1790 + ks)
    for oq in (O.INT8, O.FP8):
        for n, k in ((1536, 8960), (70, 1664)):
            x = synth.f32_to_bf16_bits(rng.standard_normal((1, k)).astype(np.float32))
            w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
            wc, ws = O.quantize_rows(w, oq)
            xc, xs = O.quantize_rows(x, oq, s_mode=O.S_MUL_RECIP)
            y_ref, acc_i, _ = O.linear(oq, xc, xs, wc, ws, O.BF16)
            y, acc = qr.qr_w8a8_linear_bf16(GQ[oq], dev(x), dev(wc), dev(ws), acc_out=True)
            torch.cuda.synchronize()
            err = capfd.readouterr().err
            fused = not (oq == O.FP8 and k > 8192)  # the FP8 in-kernel quantization stops at k = 8192
            assert ("fused=1" in err) == fused, err
            assert "ksub=%d " % ks in err, err
            if oq == O.INT8:
                assert np.array_equal(host(acc), acc_i), (ks, n, k)
            assert_y_close(host(y), y_ref, "bf16 ksub=%d n=%d k=%d" % (ks, n, k))


@pytest.mark.parametrize("ks", [2, 4, 8])
def test_gemv_k_parts_token_blocks(ks, monkeypatch, capfd):
    """K parts with more tokens than one tile holds (16 / ks): token blocks of 16 / ks tokens, each its own row of
    workgroups; INT8 accumulators bit-exact, FP8 within the tolerance, ragged batches and channels."""
    monkeypatch.setenv("QR_GEMV_KSUB", str(ks))
    monkeypatch.setenv("QR_GEMV_KSUB_BLOCKS", "1")
    monkeypatch.setenv("QR_TRACE", "1")
    for i, (m, n, k) in enumerate([(16, 1536, 8960), (13, 70, 1664), (5, 37, 3584)]):
        for oq in (O.INT8, O.FP8):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1800 + 10 * i + oq + ks)
            what = "gemv ksub=%d token blocks %s m=%d n=%d k=%d" % (ks, oq, m, n, k)
            log(what)
            _check(oq, xc, xs, wc, ws, what)
            err = capfd.readouterr().err
            assert "ksub=%d " % ks in err, err


# every compiled GEMV variant: (token tiles, 64-byte loads per slice, weight tiles per block)
GEMV_VARIANTS = [(1, 4, 1), (1, 4, 2), (1, 4, 4), (1, 8, 1), (1, 8, 2), (2, 4, 1), (2, 4, 2), (2, 8, 1),
                 (4, 2, 1), (4, 2, 2), (4, 4, 1)]


@pytest.mark.parametrize("mt,u,tb", GEMV_VARIANTS)
def test_every_gemv_variant(mt, u, tb, monkeypatch, capfd):
    """Each variant, forced through the planner's overrides, on ragged shapes: n not a multiple of the block's
    16 tb channels, k with a partial last slice, m not a multiple of 16 -- INT8 accumulators bit-exact, FP8
    and bf16 outputs within the tolerance."""
    monkeypatch.setenv("QR_GEMV_UNROLL", str(u))
    monkeypatch.setenv("QR_GEMV_TILES", str(tb))
    monkeypatch.setenv("QR_TRACE", "1")
    m = {1: 13, 2: 29, 4: 61}[mt]
    for oq in (O.INT8, O.FP8):
        for i, (n, k) in enumerate([(16 * tb * 3 + 5, 64 * u * 3 + 48), (200, 64 * u * 17 + 16)]):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=900 + 10 * i + oq)
            log("variant mt=%d u=%d tb=%d %s m=%d n=%d k=%d" % (mt, u, tb, oq, m, n, k))
            _check(oq, xc, xs, wc, ws, "variant mt=%d u=%d tb=%d m=%d n=%d k=%d" % (mt, u, tb, m, n, k))
            err = capfd.readouterr().err
            assert "mt=%d" % mt in err and "unroll=%d tiles=%d" % (u, tb) in err, err


# every large-batch GEMM kernel: 0 = the LDS-ring kernel (256 or 128 activation rows per tile, with or without
# split K), 4 = the wide-wave kernel (128 x 128 outputs per wavefront, 128-byte stages; with or without split K),
# 1..3 = register-staged 256x128, 128x256, 128x128; shapes with ragged m and n, k with a partial last stage, a
# single partial stage and fewer stages than the ring holds, n not a multiple of 8 (element-wise epilogue) and
# whole 256-column tiles (the vectorized bf16 epilogue). The wide kernel takes K in whole 128-byte stages: its
# shapes have one, two and many stages, and a K it does not take runs on the ring kernel.
GEMM_SHAPES = [(65, 264, 16), (300, 512, 1040), (257, 520, 176), (130, 333, 4160), (512, 768, 2048),
               (100, 1000, 1552)]
WIDE_SHAPES = [(65, 264, 128), (300, 512, 1024), (257, 520, 256), (130, 333, 4096), (512, 768, 2048),
               (100, 1000, 1536), (300, 520, 1040)]
# (kernel, K splits, activation rows per tile, channels per tile): the ring kernel also with its narrow
# channel tiles (64 and 128 channels, 2 to 8 wavefronts per workgroup)
GEMM_CASES = [(0, None, None, None), (0, 1, 128, 256), (0, 1, 256, 256), (0, 3, 128, 256), (0, 3, 256, 256),
              (0, 64, 256, 256), (0, 1, 128, 64), (0, 3, 128, 128), (0, None, 256, 64), (0, 2, 256, 128),
              (4, None, None, None), (4, 1, 256, None), (4, 3, 256, None), (4, 64, 256, None),
              (1, None, None, None), (2, None, None, None), (3, None, None, None)]
STAGE_BYTES = {0: 64, 4: 128}


@pytest.mark.parametrize("tile,splits,bm,bn", GEMM_CASES)
def test_every_gemm_tile(tile, splits, bm, bn, monkeypatch, capfd):
    monkeypatch.setenv("QR_GEMM_TILE", str(tile))
    if splits is not None:
        monkeypatch.setenv("QR_GEMM_SPLITS", str(splits))
    if bm is not None:
        monkeypatch.setenv("QR_GEMM_BM", str(bm))
    if bn is not None:
        monkeypatch.setenv("QR_GEMM_BN", str(bn))
    monkeypatch.setenv("QR_TRACE", "1")
    wsp = qr.Workspace()
    for i, (m, n, k) in enumerate(WIDE_SHAPES if tile == 4 else GEMM_SHAPES):
        ran = tile if tile != 4 or k % 128 == 0 else 0
        for oq in (O.INT8, O.FP8):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1300 + 10 * i + oq)
            what = "gemm tile=%s splits=%s bm=%s bn=%s %s m=%d n=%d k=%d" % (tile, splits, bm, bn, oq, m, n, k)
            log(what)
            _check(oq, xc, xs, wc, ws, what)
            err = capfd.readouterr().err
            assert "kind=1" in err and "gemm=%d" % ran in err, err
            if bm is not None:
                assert "bm=%d" % bm in err, err
            if bn is not None and ran == 0:
                assert "bn=%d" % bn in err, err
            if splits is not None:
                stages = -(-k // STAGE_BYTES[ran])
                sps = -(-stages // min(splits, stages))
                assert "splits=%d" % (-(-stages // sps)) in err, err
            # without accumulators: the bf16 output takes the kernel's other epilogue where it has one, and
            # is bitwise the one written next to the accumulators
            y_ref, _, _ = O.linear(oq, xc, xs, wc, ws, O.BF16)
            y_acc, _ = _run(oq, xc, xs, wc, ws)
            y = qr.qr_w8a8_linear(GQ[oq], dev(xc), dev(xs), dev(wc), dev(ws), workspace=wsp)
            torch.cuda.synchronize()
            y = host(y)
            assert_y_close(y, y_ref, what + " (no accumulators)")
            assert np.array_equal(y, y_acc), what


# Whole rounds of tiles over all of K first, then the remaining band of output columns split over K: the planner's
# choice for tile counts just past a whole number of CU rounds, forced here with a round of 8 tiles.
# (m, n, k, rows per tile, channels per tile, splits, whole-K tiles): 2 x 11 tiles with a ragged 3-tile band and
# a partial last stage (wide kernel: a shorter last split); 2 x 9 tiles with a one-tile band of 253 columns
# (element-wise reduction) and a one-stage last split; 1 x 9 tiles with 13 (wide kernel: 16) splits; 2 x 41 tiles
# of 64 channels with a one-column band of 40 channels
HYB_CASES = [(0, 300, 2600, 1040, 256, 256, 3, 16), (0, 512, 2301, 1040, 256, 256, 5, 16),
             (0, 100, 2304, 4160, 128, 256, 16, 8), (0, 300, 2600, 1040, 256, 64, 3, 80),
             (4, 300, 2600, 1024, 256, 256, 3, 16), (4, 512, 2301, 1024, 256, 256, 5, 16),
             (4, 200, 2304, 4096, 256, 256, 16, 8)]


@pytest.mark.parametrize("tile,m,n,k,bm,bn,splits,dp", HYB_CASES)
def test_gemm_whole_tiles_then_split_band(tile, m, n, k, bm, bn, splits, dp, monkeypatch, capfd):
    monkeypatch.setenv("QR_GEMM_TILE", str(tile))
    monkeypatch.setenv("QR_GEMM_ROUND", "8")
    monkeypatch.setenv("QR_GEMM_HYB", str(splits))
    monkeypatch.setenv("QR_GEMM_BM", str(bm))
    monkeypatch.setenv("QR_GEMM_BN", str(bn))
    monkeypatch.setenv("QR_TRACE", "1")
    stages = -(-k // STAGE_BYTES[tile])
    sps = -(-stages // splits)
    used = -(-stages // sps)
    wsp = qr.Workspace()
    for oq in (O.INT8, O.FP8):
        xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1700 + m + oq)
        what = "gemm band split tile=%d %s m=%d n=%d k=%d bm=%d bn=%d splits=%d" % (tile, oq, m, n, k, bm, bn, splits)
        log(what)
        _check(oq, xc, xs, wc, ws, what)
        err = capfd.readouterr().err
        assert "kind=1" in err and "gemm=%d bm=%d splits=%d dp=%d " % (tile, bm, used, dp) in err, err
        assert "bn=%d" % bn in err, err
        y_acc, _ = _run(oq, xc, xs, wc, ws)
        for rep in range(2):  # one workspace object, called again: the same bytes
            y = qr.qr_w8a8_linear(GQ[oq], dev(xc), dev(xs), dev(wc), dev(ws), workspace=wsp)
            torch.cuda.synchronize()
            assert np.array_equal(host(y), y_acc), (what, rep)


# The wide kernel over all of K with the columns past whole rounds of 256-wide tiles run as a band of 256 x 160
# tiles in a second launch, forced on with a round of 8 tiles: (m, n, k, first band column or -1 for none).
# 2 x 11 tiles: two rounds, then a band of 552 columns (a partial last band tile); 1 x 2 and 2 x 2 tiles: the band
# alone (ragged rows, 512 = 3 x 160 + 32 columns, a one-stage K); 1 x 2 tiles with a deep K and 333 columns
# (the element-wise epilogue); 2 x 3 tiles, whose band would need 10 tiles: none.
BAND_CASES = [(300, 2600, 1024, 2048), (65, 264, 128, 0), (300, 512, 1024, 0), (130, 333, 4096, 0),
              (512, 768, 2048, -1)]


@pytest.mark.parametrize("m,n,k,band", BAND_CASES)
def test_wide_kernel_band_of_narrow_tiles(m, n, k, band, monkeypatch, capfd):
    monkeypatch.setenv("QR_GEMM_TILE", "4")
    monkeypatch.setenv("QR_GEMM_SPLITS", "1")
    monkeypatch.setenv("QR_GEMM_BAND", "1")
    monkeypatch.setenv("QR_GEMM_ROUND", "8")
    monkeypatch.setenv("QR_TRACE", "1")
    wsp = qr.Workspace()
    for oq in (O.INT8, O.FP8):
        xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=1900 + m + n + oq)
        what = "wide band %s m=%d n=%d k=%d" % (oq, m, n, k)
        log(what)
        _check(oq, xc, xs, wc, ws, what)
        err = capfd.readouterr().err
        assert "gemm=4 " in err and "band=%d\n" % band in err, err
        y_ref, _, _ = O.linear(oq, xc, xs, wc, ws, O.BF16)
        y_acc, _ = _run(oq, xc, xs, wc, ws)
        y = qr.qr_w8a8_linear(GQ[oq], dev(xc), dev(xs), dev(wc), dev(ws), workspace=wsp)
        torch.cuda.synchronize()
        y = host(y)
        assert_y_close(y, y_ref, what + " (no accumulators)")
        assert np.array_equal(y, y_acc), what


# The planner's band at one token tile (64 < m <= 128): taken only where the 256 x 160 tiles fill at least three
# quarters of a round over a K of at least 2048 bytes (the 7B gate/up: 237 tiles), not for the 1.5B gate/up
# (112 tiles, K = 1536) or the 7B down (23 tiles); (m, n, k, first band column or -1).
@pytest.mark.parametrize("m,n,k,band", [(128, 37888, 3584, 0), (96, 37888, 3584, 0), (128, 17920, 1536, -1),
                                        (128, 3584, 18944, -1)])
def test_band_plan_at_one_token_tile(m, n, k, band, monkeypatch, capfd):
    monkeypatch.setenv("QR_TRACE", "1")
    q = qr.QR_FP8_E4M3
    log("band plan m=%d n=%d k=%d" % (m, n, k))
    x = torch.zeros((m, k), dtype=torch.uint8, device="cuda")  # zero codes: only the plan is checked here
    xs = torch.ones(m, device="cuda")
    w = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    wsc = torch.ones(n, device="cuda")
    y = qr.qr_w8a8_linear(q, x, xs, w, wsc)
    torch.cuda.synchronize()
    assert not bool(y.float().abs().max() > 0)
    err = capfd.readouterr().err
    assert "kind=1" in err and ("band=%d\n" % band) in err, err
    if band >= 0:
        assert "gemm=4 " in err, err


def test_workspace_reuse_across_plans():
    """One workspace object serves a sequence of differently planned shapes: every call stays bit-exact (INT8)
    or within tolerance (FP8)."""
    wsp = qr.Workspace()
    wsp.get(64 << 20)
    shapes = [(64, 64, 4096), (1, 1536, 8960), (16, 200, 1552), (33, 130, 784), (1, 2048, 8960), (64, 64, 4096),
              (16, 1536, 8960)]
    for oq in (O.INT8, O.FP8):
        for i, (m, n, k) in enumerate(shapes * 2):
            xc, xs, wc, ws = _quantized_operands(m, n, k, oq, seed=400 + i)
            log("workspace reuse %s m=%d n=%d k=%d" % (oq, m, n, k))
            y_ref, acc_i, _ = O.linear(oq, xc, xs, wc, ws, O.BF16)
            y, acc = qr.qr_w8a8_linear(GQ[oq], dev(xc), dev(xs), dev(wc), dev(ws), acc_out=True, workspace=wsp)
            torch.cuda.synchronize()
            if oq == O.INT8:
                assert np.array_equal(host(acc), acc_i), (m, n, k)
            assert_y_close(host(y), y_ref, "reuse m=%d n=%d k=%d" % (m, n, k))


def test_fp8_all_max_codes_accumulate_exactly():
    """All-448 codes: every partial sum 200704 * j is exactly representable in fp32, so the accumulators equal
    200704 * k exactly (closed form; k = 18944 gives 2^21 * 1813)."""
    for (m, n, k) in [(1, 16, 18944), (16, 64, 3584), (200, 130, 2048)]:
        xc = np.full((m, k), 0x7E, np.uint8)
        wc = np.full((n, k), 0xFE, np.uint8)
        ones_m, ones_n = np.ones(m, np.float32), np.ones(n, np.float32)
        y, acc = qr.qr_w8a8_linear(qr.QR_FP8_E4M3, dev(xc), dev(ones_m), dev(wc), dev(ones_n), acc_out=True,
                                   y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.all(host(acc) == np.float32(-200704.0 * k)), (m, n, k)
        assert np.all(host(y) == np.float32(-200704.0 * k))


def _full_size_case(wl, oq, m_list, n_sample=48):
    inp = synth.make_dense(wl)
    rng = np.random.default_rng(12)
    for name, w in inp.weights.items():
        x = inp.acts[name]
        wc_ref, ws_ref = O.quantize_rows(w, oq)
        xc_all, xs_all = O.quantize_rows(x, oq, s_mode=O.S_MUL_RECIP)
        cols = np.sort(rng.choice(w.shape[0], n_sample, replace=False))
        cols[-1] = w.shape[0] - 1
        wcd, wsd = dev(wc_ref), dev(ws_ref)
        for m in m_list:
            log("full-size linear %s %s m=%d n=%d k=%d" % (wl.name, name, m, w.shape[0], w.shape[1]))
            y, acc = qr.qr_w8a8_linear(GQ[oq], dev(xc_all[:m]), dev(xs_all[:m]), wcd, wsd, acc_out=True)
            torch.cuda.synchronize()
            y_ref, acc_i, acc_f = O.linear(oq, xc_all[:m], xs_all[:m], wc_ref[cols], ws_ref[cols], O.BF16)
            y_h = host(y)[:, cols]
            what = "%s %s m=%d" % (wl.name, name, m)
            bound = None
            if oq == O.INT8:
                assert np.array_equal(host(acc)[:, cols], acc_i), (name, m)
            else:
                bound = fp8_acc_bound(xc_all[:m], wc_ref[cols])
                assert_fp8_acc_within_bound(host(acc)[:, cols], acc_f, bound, what)
            assert_y_within_bound(y_h, acc_f, xs_all[:m], ws_ref[cols], bound, what)
            assert_y_close(y_h, y_ref, what)


def test_full_size_qwen_1p5b_int8_sampled():
    _full_size_case(synth.QWEN_1P5B, O.INT8, [1, 16, 64])


def test_full_size_7b_fp8_sampled():
    _full_size_case(synth.DENSE_7B, O.FP8, [1, 16, 128, 512, 2048], n_sample=24)


def test_empty_and_errors():
    z = torch.zeros((0, 32), dtype=torch.uint8, device="cuda")
    zs = torch.zeros((0,), dtype=torch.float32, device="cuda")
    w = torch.zeros((8, 32), dtype=torch.uint8, device="cuda")
    wsc = torch.ones((8,), dtype=torch.float32, device="cuda")
    y = qr.qr_w8a8_linear(qr.QR_INT8, z, zs, w, wsc)
    assert y.shape == (0, 8)
    with pytest.raises(qr.QRError):
        qr.qr_w8a8_linear(qr.QR_INT8, torch.zeros((2, 24), dtype=torch.uint8, device="cuda"),
                          torch.ones(2, device="cuda"), torch.zeros((8, 24), dtype=torch.uint8, device="cuda"), wsc)
