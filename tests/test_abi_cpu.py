"""The C ABI on the CPU: libqr.so loads, exports every symbol include/qr.h declares, and its host-side
validation rejects bad arguments before anything is launched (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

from quantized_rollout_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qr.h")

# fake, 256-byte aligned device addresses: validation never dereferences them on the host and every call
# below fails (or is a no-op) before a launch
P = ctypes.c_void_p(0x7F0000000000)
P2 = ctypes.c_void_p(0x7F0000100000)
MIS = ctypes.c_void_p(0x7F0000000008)
NULL = None
S0 = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_auxiliaries():
    names = declared_functions()
    for f in ("qr_quantize_weights", "qr_quantize_acts", "qr_w8a8_linear", "qr_w8a8_grouped_linear"):
        assert f in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert re.match(r"^\d+\.\d+\.\d+$", B.qr_version())


def _err():
    return B.lib().qr_last_error().decode()


def test_linear_validation():
    L = B.lib()
    base = dict(q=0, m=16, n=1536, k=8960, x=P, xs=P, w=P, wsc=P, y=P, yt=1, acc=NULL, wsp=NULL, wsb=0)

    def call(**kw):
        a = dict(base, **kw)
        return L.qr_w8a8_linear(a["q"], a["m"], a["n"], a["k"], a["x"], a["xs"], a["w"], a["wsc"], a["y"], a["yt"],
                                a["acc"], a["wsp"], a["wsb"], S0)

    assert call(k=8968) == B.QR_ERR_UNSUPPORTED and "multiple of 16" in _err()
    assert call(k=0) == B.QR_ERR_ARG
    assert call(k=131072 + 16) == B.QR_ERR_UNSUPPORTED
    assert call(m=-1) == B.QR_ERR_ARG
    assert call(q=7) == B.QR_ERR_ARG and "qtype" in _err()
    assert call(yt=9) == B.QR_ERR_ARG
    assert call(x=NULL) == B.QR_ERR_ARG
    assert call(w=MIS) == B.QR_ERR_ALIGN
    assert call(y=MIS) == B.QR_ERR_ALIGN
    assert call(acc=MIS) == B.QR_ERR_ALIGN
    # a split-K plan needs its workspace, 256-byte aligned
    big = dict(m=512, n=3584, k=18944)
    need = B.qr_workspace_bytes(0, 512, 3584, 18944)
    assert call(**big) == B.QR_ERR_WORKSPACE and "workspace" in _err()
    assert call(wsp=P, wsb=need - 1, **big) == B.QR_ERR_WORKSPACE
    assert call(wsp=MIS, wsb=need, **big) == B.QR_ERR_ALIGN
    # empty problems are no-ops that launch nothing
    assert call(m=0) == B.QR_OK and _err() == ""
    assert call(n=0, x=NULL) == B.QR_OK


def test_linear_noalloc_validation():
    """The no-allocation linear validates like qr_w8a8_linear and rejects plans whose split-K partial sums exceed
    its device scratch before launching anything (no GPU call is reached on any of these paths)."""
    L = B.lib()
    base = dict(q=0, m=16, n=1536, k=8960, x=P, xs=P, w=P, wsc=P, y=P, yt=1, acc=NULL)

    def call(**kw):
        a = dict(base, **kw)
        return L.qr_w8a8_linear_noalloc(a["q"], a["m"], a["n"], a["k"], a["x"], a["xs"], a["w"], a["wsc"], a["y"],
                                        a["yt"], a["acc"], S0)

    assert call(k=8968) == B.QR_ERR_UNSUPPORTED and "multiple of 16" in _err()
    assert call(m=-1) == B.QR_ERR_ARG
    assert call(q=7) == B.QR_ERR_ARG
    assert call(x=NULL) == B.QR_ERR_ARG
    assert call(w=MIS) == B.QR_ERR_ALIGN
    assert call(m=0) == B.QR_OK and _err() == ""
    # a plan whose partial sums exceed the scratch: rejected with a clear message
    big = None
    for m, n, k in ((1024, 3584, 131072), (2048, 3584, 131072)):
        if B.qr_workspace_bytes(0, m, n, k) > B.NOALLOC_SCRATCH_BYTES:
            big = (m, n, k)
            break
    assert big is not None
    assert call(m=big[0], n=big[1], k=big[2]) == B.QR_ERR_UNSUPPORTED and "scratch" in _err()


def test_quantize_validation():
    L = B.lib()
    for fn in (L.qr_quantize_weights, L.qr_quantize_acts):
        assert fn(P, 1, 8, 24, NULL, 0, P, P, S0) == B.QR_ERR_UNSUPPORTED
        assert fn(P, 1, 8, -16, NULL, 0, P, P, S0) == B.QR_ERR_ARG
        assert fn(P, 1, -8, 16, NULL, 0, P, P, S0) == B.QR_ERR_ARG
        assert fn(P, 5, 8, 16, NULL, 0, P, P, S0) == B.QR_ERR_ARG
        assert fn(P, 1, 8, 16, NULL, 3, P, P, S0) == B.QR_ERR_ARG
        assert fn(NULL, 1, 8, 16, NULL, 0, P, P, S0) == B.QR_ERR_ARG
        assert fn(MIS, 1, 8, 16, NULL, 0, P, P, S0) == B.QR_ERR_ALIGN
        assert fn(P, 1, 8, 16, ctypes.c_void_p(0x7F0000000002), 0, P, P, S0) == B.QR_ERR_ALIGN
        assert fn(P, 1, 0, 16, NULL, 0, NULL, NULL, S0) == B.QR_OK


def test_w4_validation():
    L = B.lib()
    fn = L.qr_quantize_weights_w4
    assert fn(P, 1, 8, 136, NULL, P, P, S0) == B.QR_ERR_UNSUPPORTED and "multiple of 128" in _err()
    assert fn(P, 1, 8, 0, NULL, P, P, S0) == B.QR_ERR_ARG
    assert fn(P, 1, -8, 128, NULL, P, P, S0) == B.QR_ERR_ARG
    assert fn(P, 5, 8, 128, NULL, P, P, S0) == B.QR_ERR_ARG
    assert fn(MIS, 1, 8, 128, NULL, P, P, S0) == B.QR_ERR_ALIGN
    assert fn(P, 1, 8, 128, MIS, P, P, S0) == B.QR_ERR_ALIGN
    assert fn(P, 1, 0, 128, NULL, NULL, NULL, S0) == B.QR_OK
    lin = L.qr_w4a16_linear
    assert lin(4, 16, 200, P, P, P, P, 1, S0) == B.QR_ERR_UNSUPPORTED
    assert lin(4, 16, 128, NULL, P, P, P, 1, S0) == B.QR_ERR_ARG
    assert lin(4, 16, 128, MIS, P, P, P, 1, S0) == B.QR_ERR_ALIGN
    assert lin(4, 16, 128, P, P, P, P, 7, S0) == B.QR_ERR_ARG
    assert lin(0, 16, 128, NULL, NULL, NULL, NULL, 1, S0) == B.QR_OK
    # the codes of one weight must stay under 4 GiB (32-bit offsets in the kernel)
    assert lin(1, 1 << 20, 1 << 13, P, P, P, P, 1, S0) == B.QR_ERR_UNSUPPORTED and "4 GiB" in _err()


def test_grouped_validation():
    L = B.lib()

    def call(E=4, n=64, k=256, off=P, rows=P, total=32, xrows=8, x=P, xs=P, w=P, wsc=P, y=P, yt=1):
        return L.qr_w8a8_grouped_linear(1, E, n, k, off, rows, total, xrows, x, xs, w, wsc, y, yt, NULL, 0, S0)

    assert call(k=250) == B.QR_ERR_UNSUPPORTED
    assert call(E=-1) == B.QR_ERR_ARG
    assert call(E=70000) == B.QR_ERR_UNSUPPORTED
    assert call(off=NULL) == B.QR_ERR_ARG
    assert call(rows=NULL, xrows=8, total=32) == B.QR_ERR_ARG  # identity rows need x_rows >= total_rows
    assert call(x=MIS) == B.QR_ERR_ALIGN
    assert call(total=0) == B.QR_OK
    assert call(E=0) == B.QR_OK


def test_count_validation():
    L = B.lib()
    assert L.qr_count_code_changes(P, P, 64, 1, NULL, NULL, 0, NULL, S0) == B.QR_ERR_ARG
    assert L.qr_count_code_changes(NULL, P, 64, 1, NULL, NULL, 0, P, S0) == B.QR_ERR_ARG
    assert L.qr_count_code_changes(P, P, -1, 1, NULL, NULL, 0, P, S0) == B.QR_ERR_ARG
    assert L.qr_count_code_changes(MIS, P, 64, 1, NULL, NULL, 0, P, S0) == B.QR_ERR_ALIGN
    assert L.qr_count_code_changes(P, P, 64, 3, NULL, NULL, 0, P, S0) == B.QR_ERR_ARG


def test_requantize_validation():
    L = B.lib()

    def call(w=P, wt=1, n=8, k=128, s=NULL, q=0, pc=P, ps=P, c=P, sc=P, rc=P, o3=P):
        return L.qr_requantize_weights(w, wt, n, k, s, q, pc, ps, c, sc, rc, o3, S0)

    assert call(k=136) == B.QR_ERR_UNSUPPORTED
    assert call(k=0) == B.QR_ERR_ARG
    assert call(n=-1) == B.QR_ERR_ARG
    assert call(q=5) == B.QR_ERR_ARG
    assert call(o3=NULL) == B.QR_ERR_ARG
    assert call(rc=NULL) == B.QR_ERR_ARG
    assert call(pc=NULL) == B.QR_ERR_ARG
    assert call(w=MIS) == B.QR_ERR_ALIGN
    assert call(pc=MIS) == B.QR_ERR_ALIGN
    # the previous publish is the output itself, or disjoint from it; a partial overlap is refused
    base = 1 << 20
    assert call(pc=base, c=base + 512, ps=P, sc=P) == B.QR_ERR_ARG and "overlap" in _err()
    assert call(pc=base, c=base + 8 * 128, n=8, k=128, ps=1 << 22, sc=(1 << 22) + 16) == B.QR_ERR_ARG


def test_linear_bf16_validation_and_workspace(monkeypatch):
    L = B.lib()

    def call(q=0, m=4, n=64, k=256, x=P, s=NULL, wc=P, ws=P, y=P, yt=1, acc=NULL, wsp=NULL, wsb=0):
        return L.qr_w8a8_linear_bf16(q, m, n, k, x, s, wc, ws, y, yt, acc, wsp, wsb, S0)

    assert call(k=250) == B.QR_ERR_UNSUPPORTED
    assert call(m=-1) == B.QR_ERR_ARG
    assert call(x=NULL) == B.QR_ERR_ARG
    assert call(x=MIS) == B.QR_ERR_ALIGN
    assert call(q=4) == B.QR_ERR_ARG
    assert call(m=0) == B.QR_OK
    ws = B.qr_w8a8_linear_bf16_workspace_bytes if hasattr(B, "qr_w8a8_linear_bf16_workspace_bytes") else None
    for q in (B.QR_INT8, B.QR_FP8_E4M3):
        # m = 1: the activation quantization runs inside the linear, no workspace (FP8: for k <= 8192), on plans
        # of fewer than 1024 workgroups; the 1120 workgroups of n = 17920 quantize into the workspace first
        assert ws(q, 1, 2048, 1536) == 0  # in-kernel quantization: at most 256 workgroups
        assert ws(q, 1, 3584, 3584) == 3584 + 256  # 448 workgroups: the quantizer, then the linear
        assert ws(q, 1, 17920, 1536) == 1536 + 256
        assert ws(q, 1, 1536, 8960) == (0 if q == B.QR_INT8 else 8960 + 256)
        # larger batches: the activation codes (m k bytes) and scales (4 m), each rounded up to 256 bytes,
        # then the linear's own workspace
        assert ws(q, 16, 2048, 1536) == 16 * 1536 + 256
        assert ws(q, 64, 1536, 8960) == 64 * 8960 + 256 + 2 * 64 * 1536 * 4
        monkeypatch.setenv("QR_FUSE_MAX_M", "4")
        assert ws(q, 4, 2048, 1536) == 0
        monkeypatch.delenv("QR_FUSE_MAX_M")
        assert ws(q, 4, 2048, 1536) == 4 * 1536 + 256
    # a call that needs workspace and gets none is refused before any launch
    assert call(m=16, n=2048, k=1536) == B.QR_ERR_WORKSPACE


def test_linear_bf16_workspace_every_batch():
    """The bf16 entry point's workspace query for decode (GEMV) and large (GEMM) plans alike: no fused form past one
    token tile, so the activation codes and scales come first, then the linear's own workspace."""
    up = lambda b: (b + 255) // 256 * 256
    for q in (B.QR_INT8, B.QR_FP8_E4M3):
        for n, k in ((4608, 3584), (3584, 3584), (37888, 3584), (3584, 18944), (2048, 1536), (1536, 8960)):
            for m in (1, 2, 16, 17, 64, 65, 128, 512, 2048, 4096):
                need = B.qr_w8a8_linear_bf16_workspace_bytes(q, m, n, k)
                if m > 16:
                    assert need == up(m * k) + up(4 * m) + B.qr_workspace_bytes(q, m, n, k), (q, m, n, k)


def test_workspace_sizes(monkeypatch):
    for q in (B.QR_INT8, B.QR_FP8_E4M3):
        # GEMV plans with enough blocks, and GEMM plans with a tile for at least half the CUs, reduce inside
        # their workgroups
        for m, n, k in ((1, 1536, 8960), (16, 2048, 1536), (64, 37888, 3584), (1, 3584, 18944),
                        (2048, 37888, 3584), (128, 37888, 3584)):
            assert B.qr_workspace_bytes(q, m, n, k) == 0
        # GEMV with four token tiles, few channel tiles and a deep K (1.5B down at m = 64: 96 tiles, 35 slices
        # of 256 bytes): K split over 2 blocks per tile, the partial sums in the workspace; none at m <= 32
        for m in (1, 16, 32):
            assert B.qr_workspace_bytes(q, m, 1536, 8960) == 0
        for m in (33, 64):
            assert B.qr_workspace_bytes(q, m, 1536, 8960) == 2 * m * 1536 * 4
        monkeypatch.setenv("QR_GEMV_SPLITS", "7")
        assert B.qr_workspace_bytes(q, 5, 1536, 8960) == 7 * 5 * 1536 * 4
        monkeypatch.setenv("QR_GEMV_SPLITS", "64")  # never a split without a slice: 35 slices -> 35 splits
        assert B.qr_workspace_bytes(q, 5, 1536, 8960) == 35 * 5 * 1536 * 4
        monkeypatch.delenv("QR_GEMV_SPLITS")
        # few tiles: the planner's cost model splits K (runs of at least 4 stages of 64 bytes); the partial sums
        # take splits x m x n x 4 bytes
        assert B.qr_workspace_bytes(q, 512, 3584, 18944) == 9 * 512 * 3584 * 4    # 28 tiles of 256 x 256
        assert B.qr_workspace_bytes(q, 128, 4608, 3584) == 3 * 128 * 4608 * 4     # 72 tiles of 128 x 64
        assert B.qr_workspace_bytes(q, 128, 3584, 18944) == 9 * 128 * 3584 * 4    # 28 tiles of 128 x 128
        assert B.qr_workspace_bytes(q, 512, 3584, 3584) == 0                       # 224 tiles of 128 x 64
        assert B.qr_workspace_bytes(q, 2048, 3584, 18944) == 2 * 2048 * 3584 * 4  # 112 tiles, 296 stages
        # forced split counts never leave a split without a stage: 17 stages in 16 requested splits -> 9
        monkeypatch.setenv("QR_GEMM_SPLITS", "3")
        assert B.qr_workspace_bytes(q, 300, 333, 1040) == 3 * 300 * 333 * 4
        monkeypatch.setenv("QR_GEMM_SPLITS", "16")
        assert B.qr_workspace_bytes(q, 300, 333, 1040) == 9 * 300 * 333 * 4
        monkeypatch.delenv("QR_GEMM_SPLITS")
        assert B.qr_workspace_bytes(q, 256, 1536, 2048, 128) == 0
    assert B.qr_workspace_bytes(B.QR_INT8, 0, 10, 16) == 0


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_moe_glue_validation():
    L = B.lib()
    i64 = ctypes.c_int64

    def route(T=256, E=128, k=8, off=P, lg=P, ptr=P):
        return L.qr_moe_route(lg, T, E, k, ptr, ptr, off, ptr, ptr, ptr, S0)

    assert route(E=513) == B.QR_ERR_UNSUPPORTED and "512" in _err()
    assert route(E=0) == B.QR_ERR_ARG
    assert route(k=0) == B.QR_ERR_ARG and route(k=9, E=8) == B.QR_ERR_ARG and route(k=33, E=64) == B.QR_ERR_ARG
    assert route(T=-1) == B.QR_ERR_ARG
    assert route(off=NULL) == B.QR_ERR_ARG
    assert route(lg=NULL) == B.QR_ERR_ARG
    assert route(T=2 ** 28, k=8) == B.QR_ERR_UNSUPPORTED
    assert route(lg=ctypes.c_void_p(0x7F0000000002)) == B.QR_ERR_ALIGN

    def silu(rows=2048, inter=768, q=1, yg=P, codes=P, sc=P, h=NULL):
        return L.qr_silu_mul_quantize(yg, rows, inter, NULL, q, codes, sc, h, S0)

    assert silu(inter=760) == B.QR_ERR_UNSUPPORTED and "multiple of 16" in _err()
    assert silu(q=3) == B.QR_ERR_ARG
    assert silu(rows=-2) == B.QR_ERR_ARG
    assert silu(rows=0, yg=NULL) == B.QR_OK  # nothing to do
    assert silu(yg=NULL) == B.QR_ERR_ARG
    assert silu(codes=MIS) == B.QR_ERR_ALIGN and silu(h=MIS) == B.QR_ERR_ALIGN

    def combine(rows=2048, H=2048, T=256, k=8, yd=P, out=P):
        return L.qr_moe_combine(yd, i64(rows), i64(H), P, P, i64(T), i64(k), out, S0)

    assert combine(H=2044) == B.QR_ERR_UNSUPPORTED and "multiple of 8" in _err()
    assert combine(H=0) == B.QR_ERR_ARG and combine(k=0) == B.QR_ERR_ARG and combine(k=33) == B.QR_ERR_ARG
    assert combine(T=0, out=NULL) == B.QR_OK
    assert combine(out=NULL) == B.QR_ERR_ARG
    assert combine(out=MIS) == B.QR_ERR_ALIGN and combine(yd=MIS) == B.QR_ERR_ALIGN


def test_rmsnorm_quantize_validation():
    L = B.lib()

    def rms(rows=16, k=3584, q=1, x=P, g=P2, eps=1e-6, s=NULL, codes=P, sc=P, h=NULL):
        return L.qr_rmsnorm_quantize(x, rows, k, g, eps, s, q, codes, sc, h, S0)

    assert rms(k=3576) == B.QR_ERR_UNSUPPORTED and "multiple of 16" in _err()
    assert rms(k=0) == B.QR_ERR_ARG
    assert rms(q=2) == B.QR_ERR_ARG
    assert rms(rows=-1) == B.QR_ERR_ARG
    assert rms(eps=-1e-6) == B.QR_ERR_ARG and "eps" in _err()
    assert rms(eps=float("nan")) == B.QR_ERR_ARG and rms(eps=float("inf")) == B.QR_ERR_ARG
    assert rms(rows=0, x=NULL, g=NULL) == B.QR_OK  # nothing to do
    assert rms(x=NULL) == B.QR_ERR_ARG and rms(g=NULL) == B.QR_ERR_ARG and rms(sc=NULL) == B.QR_ERR_ARG
    assert rms(x=MIS) == B.QR_ERR_ALIGN and rms(g=MIS) == B.QR_ERR_ALIGN and rms(h=MIS) == B.QR_ERR_ALIGN
    assert rms(codes=MIS) == B.QR_ERR_ALIGN
    assert rms(sc=ctypes.c_void_p(0x7F0000000002)) == B.QR_ERR_ALIGN
    assert rms(s=ctypes.c_void_p(0x7F0000000002)) == B.QR_ERR_ALIGN
