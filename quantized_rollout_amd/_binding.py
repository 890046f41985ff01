"""ctypes binding of libqr.so (the C ABI in include/qr.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels. PyTorch provides device
memory (tensors) and the stream (``torch.cuda.current_stream()``). There is no fallback: if libqr.so is
missing or fails to load, every call raises.

The functions carry the C names (``qr_quantize_weights`` ...) and take torch CUDA tensors; outputs are
allocated here with torch unless passed in.
"""
import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqr.so")

# enums of qr.h
QR_OK, QR_ERR_ARG, QR_ERR_UNSUPPORTED, QR_ERR_ALIGN, QR_ERR_WORKSPACE, QR_ERR_HIP = range(6)
QR_F32, QR_BF16 = 0, 1
QR_INT8, QR_FP8_E4M3 = 0, 1
STATUS_NAMES = {0: "QR_OK", 1: "QR_ERR_ARG", 2: "QR_ERR_UNSUPPORTED", 3: "QR_ERR_ALIGN", 4: "QR_ERR_WORKSPACE",
                5: "QR_ERR_HIP"}

# every symbol include/qr.h declares
EXPORTS = ("qr_quantize_weights", "qr_quantize_acts", "qr_w8a8_linear", "qr_w8a8_grouped_linear",
           "qr_count_code_changes", "qr_workspace_bytes", "qr_last_error", "qr_version", "qr_quantize_weights_w4",
           "qr_w4a16_linear", "qr_requantize_weights", "qr_w8a8_linear_bf16", "qr_w8a8_linear_bf16_workspace_bytes",
           "qr_moe_route", "qr_silu_mul_quantize", "qr_moe_combine", "qr_w8a8_linear_noalloc", "qr_set_debug",
           "qr_rmsnorm_quantize")
NOALLOC_SCRATCH_BYTES = 64 << 20  # QR_NOALLOC_SCRATCH_BYTES
W4_GROUP = 128  # QR_W4_GROUP: input channels per INT4 scale group


class QRError(RuntimeError):
    def __init__(self, status, text):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), text))
        self.status = status


_lib = None
_lock = threading.Lock()


def lib():
    """Load libqr.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError("libqr.so is not built (run __graft_entry__.build() or "
                                       "python -m quantized_rollout_amd.build); no fallback exists")
                L = ctypes.CDLL(LIB_PATH)
                vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
                L.qr_quantize_weights.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp]
                L.qr_quantize_acts.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp]
                L.qr_w8a8_linear.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
                L.qr_w8a8_grouped_linear.argtypes = [i32, i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, vp, vp, i32,
                                                     vp, sz, vp]
                L.qr_count_code_changes.argtypes = [vp, vp, i64, i32, vp, vp, i64, vp, vp]
                L.qr_quantize_weights_w4.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
                L.qr_w4a16_linear.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32, vp]
                L.qr_requantize_weights.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp]
                L.qr_w8a8_linear_bf16.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
                L.qr_w8a8_linear_noalloc.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp]
                L.qr_w8a8_linear_bf16_workspace_bytes.argtypes = [i32, i64, i64, i64]
                L.qr_w8a8_linear_bf16_workspace_bytes.restype = sz
                L.qr_moe_route.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
                L.qr_silu_mul_quantize.argtypes = [vp, i64, i64, vp, i32, vp, vp, vp, vp]
                L.qr_rmsnorm_quantize.argtypes = [vp, i64, i64, vp, ctypes.c_float, vp, i32, vp, vp, vp, vp]
                L.qr_moe_combine.argtypes = [vp, i64, i64, vp, vp, i64, i64, vp, vp]
                for f in ("qr_quantize_weights", "qr_quantize_acts", "qr_w8a8_linear", "qr_w8a8_grouped_linear",
                          "qr_count_code_changes", "qr_quantize_weights_w4", "qr_w4a16_linear",
                          "qr_requantize_weights", "qr_w8a8_linear_bf16", "qr_moe_route", "qr_silu_mul_quantize",
                          "qr_moe_combine", "qr_w8a8_linear_noalloc", "qr_rmsnorm_quantize"):
                    getattr(L, f).restype = ctypes.c_int
                L.qr_workspace_bytes.argtypes = [i32, i64, i64, i64, i64]
                L.qr_workspace_bytes.restype = sz
                L.qr_last_error.argtypes = []
                L.qr_last_error.restype = ctypes.c_char_p
                L.qr_version.argtypes = []
                L.qr_version.restype = ctypes.c_char_p
                L.qr_set_debug.argtypes = [i32]
                L.qr_set_debug.restype = None
                _lib = L
    return _lib


def _check(status):
    if status != QR_OK:
        raise QRError(status, lib().qr_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return QR_BF16
    if t.dtype == torch.float32:
        return QR_F32
    raise TypeError("expected a bfloat16 or float32 tensor, got %s" % t.dtype)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def qr_set_debug(on):
    """Debug mode (device checks of device-side inputs, each call waiting for their verdict) on or off."""
    lib().qr_set_debug(1 if on else 0)


def qr_version():
    return lib().qr_version().decode()


def qr_workspace_bytes(qtype, m, n, k, num_experts=1):
    return int(lib().qr_workspace_bytes(int(qtype), int(m), int(n), int(k), int(num_experts)))


class Workspace:
    """Device workspace, grown on demand (its contents need no initialisation and are not preserved); calls
    that may overlap (different streams) need separate workspaces."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def default_workspace(device):
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _default_ws:
        _default_ws[idx] = Workspace(idx)
    return _default_ws[idx]


def _quantize(fn, t, qtype, s, codes, scales, stream):
    _need(t.is_cuda and t.dim() == 2 and t.is_contiguous(), "input must be a contiguous 2-D CUDA tensor")
    rows, k = t.shape
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=t.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=t.device)
    if s is not None:
        _need(s.is_cuda and s.dtype == torch.float32 and s.shape == (k,) and s.is_contiguous(),
              "s must be a contiguous float32 CUDA vector of length k")
    _need(codes.dtype == torch.uint8 and codes.shape == (rows, k) and codes.is_contiguous(), "bad codes tensor")
    _need(scales.dtype == torch.float32 and scales.shape == (rows,) and scales.is_contiguous(), "bad scales tensor")
    _check(fn(_ptr(t), _dtype_code(t), rows, k, _ptr(s), int(qtype), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def qr_quantize_weights(w, qtype, s=None, codes=None, scales=None, stream=None):
    """Per-output-channel codes [n,k] (uint8) and scales [n] of w [n,k] (optionally of W diag(s))."""
    return _quantize(lib().qr_quantize_weights, w, qtype, s, codes, scales, stream)


def qr_quantize_acts(x, qtype, s=None, codes=None, scales=None, stream=None):
    """Per-token codes [m,k] and scales [m] of x [m,k] (optionally of X diag(1/s))."""
    return _quantize(lib().qr_quantize_acts, x, qtype, s, codes, scales, stream)


def qr_requantize_weights(w, qtype, prev_codes, prev_scales, s=None, codes=None, scales=None, row_counts=None,
                          out3=None, in_place=False, stream=None):
    """One publish of w [n,k]: the codes and scales of qr_quantize_weights, and against the previous publish
    (prev_codes [n,k], prev_scales [n]) the per-row triples row_counts [n,3] (int32: bytes, values, scale
    changed) and their sums out3 [3] (int64). With in_place the new codes and scales overwrite prev_codes and
    prev_scales. Returns (codes, scales, row_counts, out3)."""
    _need(w.is_cuda and w.dim() == 2 and w.is_contiguous(), "w must be a contiguous 2-D CUDA tensor")
    n, k = w.shape
    _need(prev_codes.dtype == torch.uint8 and tuple(prev_codes.shape) == (n, k) and prev_codes.is_contiguous(),
          "prev_codes must be contiguous uint8 [n,k]")
    _need(prev_scales.dtype == torch.float32 and prev_scales.numel() == n, "prev_scales must be float32 [n]")
    if in_place:
        codes, scales = prev_codes, prev_scales
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=w.device)
    if row_counts is None:
        row_counts = torch.empty((n, 3), dtype=torch.int32, device=w.device)
    if out3 is None:
        out3 = torch.empty(3, dtype=torch.int64, device=w.device)
    if s is not None:
        _need(s.dtype == torch.float32 and s.numel() == k, "s must be float32 [k]")
    _check(lib().qr_requantize_weights(_ptr(w), _dtype_code(w), n, k, _ptr(s), int(qtype), _ptr(prev_codes),
                                       _ptr(prev_scales), _ptr(codes), _ptr(scales), _ptr(row_counts), _ptr(out3),
                                       _stream(stream)))
    return codes, scales, row_counts, out3


def qr_quantize_weights_w4(w, s=None, codes=None, scales=None, stream=None):
    """Group-wise INT4 codes [n, k/2] (two per byte, even channel in the low nibble) and scales [n, k/128] of
    w [n,k] (optionally of W diag(s))."""
    _need(w.is_cuda and w.dim() == 2 and w.is_contiguous(), "w must be a contiguous 2-D CUDA tensor")
    n, k = w.shape
    _need(k % W4_GROUP == 0, "k must be a multiple of %d" % W4_GROUP)
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // W4_GROUP), dtype=torch.float32, device=w.device)
    if s is not None:
        _need(s.is_cuda and s.dtype == torch.float32 and s.shape == (k,) and s.is_contiguous(),
              "s must be a contiguous float32 CUDA vector of length k")
    _need(codes.dtype == torch.uint8 and codes.shape == (n, k // 2) and codes.is_contiguous(), "bad codes tensor")
    _need(scales.dtype == torch.float32 and scales.shape == (n, k // W4_GROUP) and scales.is_contiguous(),
          "bad scales tensor")
    _check(lib().qr_quantize_weights_w4(_ptr(w), _dtype_code(w), n, k, _ptr(s), _ptr(codes), _ptr(scales),
                                        _stream(stream)))
    return codes, scales


def qr_w4a16_linear(x, w_codes, w_scales, y=None, y_dtype=torch.bfloat16, stream=None):
    """y [m,n] = sum over groups of w_scales * (x . q) with bfloat16 activations x [m,k] and INT4 weights."""
    m, k = x.shape
    n = w_codes.shape[0]
    for t in (x, w_codes, w_scales):
        _need(t.is_cuda and t.is_contiguous(), "operands must be contiguous CUDA tensors")
    _need(x.dtype == torch.bfloat16, "x must be bfloat16")
    _need(w_codes.dtype == torch.uint8 and w_codes.shape == (n, k // 2), "bad w_codes")
    _need(w_scales.dtype == torch.float32 and w_scales.shape == (n, k // W4_GROUP), "bad w_scales")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=x.device)
    _need(y.shape == (m, n) and y.is_contiguous(), "bad y")
    _check(lib().qr_w4a16_linear(m, n, k, _ptr(x), _ptr(w_codes), _ptr(w_scales), _ptr(y), _dtype_code(y),
                                 _stream(stream)))
    return y


def qr_w8a8_linear(qtype, x_codes, x_scales, w_codes, w_scales, y=None, y_dtype=torch.bfloat16, acc_out=None,
                   workspace=None, stream=None):
    """y [m,n] = (x_codes . w_codes^T) * x_scales[:,None] * w_scales[None,:]. ``acc_out`` True allocates the
    accumulator copy (int32 for INT8, float32 for FP8); a tensor is filled in place. Returns y or (y, acc)."""
    m, k = x_codes.shape
    n, k2 = w_codes.shape
    _need(k == k2, "k mismatch")
    dev = x_codes.device
    for t in (x_codes, x_scales, w_codes, w_scales):
        _need(t.is_cuda and t.is_contiguous(), "operands must be contiguous CUDA tensors")
    _need(x_codes.dtype == torch.uint8 and w_codes.dtype == torch.uint8, "codes must be uint8")
    _need(x_scales.dtype == torch.float32 and w_scales.dtype == torch.float32, "scales must be float32")
    _need(x_scales.shape == (m,) and w_scales.shape == (n,), "scale shapes")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=dev)
    _need(y.shape == (m, n) and y.is_contiguous(), "bad y")
    want_acc = acc_out is not None and acc_out is not False
    if acc_out is True:
        acc_out = torch.empty((m, n), dtype=torch.int32 if qtype == QR_INT8 else torch.float32, device=dev)
    elif acc_out is False:
        acc_out = None
    nbytes = qr_workspace_bytes(qtype, m, n, k)
    ws = (workspace if workspace is not None else default_workspace(dev)).get(nbytes)
    _check(lib().qr_w8a8_linear(int(qtype), m, n, k, _ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales),
                                _ptr(y), _dtype_code(y), _ptr(acc_out), _ptr(ws), nbytes, _stream(stream)))
    return (y, acc_out) if want_acc else y


def qr_w8a8_linear_noalloc(qtype, x_codes, x_scales, w_codes, w_scales, y=None, y_dtype=torch.bfloat16,
                           acc_out=None, stream=None):
    """qr_w8a8_linear without a workspace: split-K partial sums go to the library's device scratch (the same
    result bit for bit; QRError QR_ERR_UNSUPPORTED where the plan needs more scratch than the library holds).
    Allocates nothing when y (and acc_out, if wanted) are passed in."""
    m, k = x_codes.shape
    n, k2 = w_codes.shape
    _need(k == k2, "k mismatch")
    dev = x_codes.device
    for t in (x_codes, x_scales, w_codes, w_scales):
        _need(t.is_cuda and t.is_contiguous(), "operands must be contiguous CUDA tensors")
    _need(x_codes.dtype == torch.uint8 and w_codes.dtype == torch.uint8, "codes must be uint8")
    _need(x_scales.dtype == torch.float32 and w_scales.dtype == torch.float32, "scales must be float32")
    _need(x_scales.shape == (m,) and w_scales.shape == (n,), "scale shapes")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=dev)
    _need(y.shape == (m, n) and y.is_contiguous(), "bad y")
    want_acc = acc_out is not None and acc_out is not False
    if acc_out is True:
        acc_out = torch.empty((m, n), dtype=torch.int32 if qtype == QR_INT8 else torch.float32, device=dev)
    elif acc_out is False:
        acc_out = None
    _check(lib().qr_w8a8_linear_noalloc(int(qtype), m, n, k, _ptr(x_codes), _ptr(x_scales), _ptr(w_codes),
                                        _ptr(w_scales), _ptr(y), _dtype_code(y), _ptr(acc_out), _stream(stream)))
    return (y, acc_out) if want_acc else y


def qr_w8a8_linear_bf16_workspace_bytes(qtype, m, n, k):
    return int(lib().qr_w8a8_linear_bf16_workspace_bytes(int(qtype), int(m), int(n), int(k)))


def qr_w8a8_linear_bf16(qtype, x, w_codes, w_scales, s=None, y=None, y_dtype=torch.bfloat16, acc_out=None,
                        workspace=None, stream=None):
    """The W8A8 linear on bfloat16 activations x [m,k] (quantized per token, optionally as X diag(1/s)): the
    same y (and accumulators) as qr_quantize_acts then qr_w8a8_linear, with the activation quantization inside
    the linear's kernel at decode batches. Returns y or (y, acc)."""
    m, k = x.shape
    n, k2 = w_codes.shape
    _need(k == k2, "k mismatch")
    dev = x.device
    for t in (x, w_codes, w_scales):
        _need(t.is_cuda and t.is_contiguous(), "operands must be contiguous CUDA tensors")
    _need(x.dtype == torch.bfloat16, "x must be bfloat16")
    _need(w_codes.dtype == torch.uint8 and w_scales.dtype == torch.float32 and w_scales.shape == (n,),
          "weights must be uint8 codes [n,k] with float32 scales [n]")
    if s is not None:
        _need(s.dtype == torch.float32 and s.numel() == k and s.is_cuda, "s must be float32 [k]")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype, device=dev)
    _need(y.shape == (m, n) and y.is_contiguous(), "bad y")
    want_acc = acc_out is not None and acc_out is not False
    if acc_out is True:
        acc_out = torch.empty((m, n), dtype=torch.int32 if qtype == QR_INT8 else torch.float32, device=dev)
    elif acc_out is False:
        acc_out = None
    nbytes = qr_w8a8_linear_bf16_workspace_bytes(qtype, m, n, k)
    ws = (workspace if workspace is not None else default_workspace(dev)).get(nbytes)
    _check(lib().qr_w8a8_linear_bf16(int(qtype), m, n, k, _ptr(x), _ptr(s), _ptr(w_codes), _ptr(w_scales), _ptr(y),
                                     _dtype_code(y), _ptr(acc_out), _ptr(ws), nbytes, _stream(stream)))
    return (y, acc_out) if want_acc else y


def qr_w8a8_grouped_linear(qtype, expert_offsets, row_ids, total_rows, x_codes, x_scales, w_codes, w_scales, y=None,
                           y_dtype=torch.bfloat16, workspace=None, stream=None):
    """Grouped (MoE) linear. expert_offsets [E+1] int32 (device), row_ids [total_rows] int32 or None,
    w_codes [E,n,k], w_scales [E,n]. Returns y [total_rows, n]."""
    E, n, k = w_codes.shape
    x_rows, k2 = x_codes.shape
    _need(k == k2, "k mismatch")
    dev = x_codes.device
    _need(expert_offsets.dtype == torch.int32 and expert_offsets.shape == (E + 1,) and expert_offsets.is_cuda,
          "expert_offsets must be int32 [E+1] on the GPU")
    if row_ids is not None:
        _need(row_ids.dtype == torch.int32 and row_ids.shape == (total_rows,) and row_ids.is_cuda, "bad row_ids")
    _need(w_scales.shape == (E, n) and x_scales.shape == (x_rows,), "scale shapes")
    if y is None:
        y = torch.empty((total_rows, n), dtype=y_dtype, device=dev)
    nbytes = qr_workspace_bytes(qtype, total_rows, n, k, E) if E > 1 else 0
    ws = (workspace if workspace is not None else default_workspace(dev)).get(nbytes)
    _check(lib().qr_w8a8_grouped_linear(int(qtype), E, n, k, _ptr(expert_offsets), _ptr(row_ids), int(total_rows),
                                        x_rows, _ptr(x_codes), _ptr(x_scales), _ptr(w_codes), _ptr(w_scales),
                                        _ptr(y), _dtype_code(y), _ptr(ws), nbytes, _stream(stream)))
    return y


def qr_count_code_changes(a, b, qtype, sa=None, sb=None, out3=None, stream=None):
    """Device int64 [3]: bytes, decoded values and scales that differ between two code sets."""
    _need(a.dtype == torch.uint8 and b.dtype == torch.uint8 and a.numel() == b.numel(), "codes must match")
    ns = 0
    if sa is not None:
        _need(sb is not None and sa.numel() == sb.numel(), "scale vectors must match")
        ns = sa.numel()
    if out3 is None:
        out3 = torch.empty(3, dtype=torch.int64, device=a.device)
    _check(lib().qr_count_code_changes(_ptr(a), _ptr(b), a.numel(), int(qtype), _ptr(sa), _ptr(sb), ns, _ptr(out3),
                                       _stream(stream)))
    return out3


def qr_moe_route(logits, top_k, out=None, stream=None):
    """Top-k softmax routing of logits [T, E] (float32): a dict of device tensors topk_expert [T,k] (int32, expert
    order), topk_weight [T,k] (float32), expert_offsets [E+1] and row_ids [T k] (the CSR lists of
    qr_w8a8_grouped_linear), row_weights [T k] and pair_rows [T,k] (int32)."""
    _need(logits.is_cuda and logits.dtype == torch.float32 and logits.dim() == 2 and logits.is_contiguous(),
          "logits must be a contiguous float32 [T, E] CUDA tensor")
    T, E = logits.shape
    k = int(top_k)
    dev = logits.device
    if out is None:
        out = dict(topk_expert=torch.empty((T, k), dtype=torch.int32, device=dev),
                   topk_weight=torch.empty((T, k), dtype=torch.float32, device=dev),
                   expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   row_ids=torch.empty(T * k, dtype=torch.int32, device=dev),
                   row_weights=torch.empty(T * k, dtype=torch.float32, device=dev),
                   pair_rows=torch.empty((T, k), dtype=torch.int32, device=dev))
    _check(lib().qr_moe_route(_ptr(logits), T, E, k, _ptr(out["topk_expert"]), _ptr(out["topk_weight"]),
                              _ptr(out["expert_offsets"]), _ptr(out["row_ids"]), _ptr(out["row_weights"]),
                              _ptr(out["pair_rows"]), _stream(stream)))
    return out


def qr_silu_mul_quantize(y_gu, qtype, s=None, codes=None, scales=None, h=None, want_h=False, stream=None):
    """h = bf16(silu(g) u) of y_gu [rows, 2I] (bfloat16, gate columns first) and its per-row codes [rows, I] and
    scales [rows] (as qr_quantize_acts of h). Returns (codes, scales) or, with want_h / h given, (codes, scales, h)."""
    _need(y_gu.is_cuda and y_gu.dtype == torch.bfloat16 and y_gu.dim() == 2 and y_gu.is_contiguous(),
          "y_gu must be a contiguous bfloat16 [rows, 2I] CUDA tensor")
    rows, i2 = y_gu.shape
    _need(i2 % 2 == 0, "y_gu must have an even number of columns")
    inter = i2 // 2
    dev = y_gu.device
    if codes is None:
        codes = torch.empty((rows, inter), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=dev)
    if h is None and want_h:
        h = torch.empty((rows, inter), dtype=torch.bfloat16, device=dev)
    if s is not None:
        _need(s.is_cuda and s.dtype == torch.float32 and s.numel() == inter, "s must be float32 [I]")
    _need(codes.dtype == torch.uint8 and tuple(codes.shape) == (rows, inter) and codes.is_contiguous(), "bad codes")
    _need(scales.dtype == torch.float32 and scales.numel() == rows, "bad scales")
    if h is not None:
        _need(h.dtype == torch.bfloat16 and tuple(h.shape) == (rows, inter) and h.is_contiguous(), "bad h")
    _check(lib().qr_silu_mul_quantize(_ptr(y_gu), rows, inter, _ptr(s), int(qtype), _ptr(codes), _ptr(scales), _ptr(h),
                                      _stream(stream)))
    return (codes, scales, h) if h is not None else (codes, scales)


def qr_rmsnorm_quantize(x, gamma, eps, qtype, s=None, codes=None, scales=None, h=None, want_h=False, stream=None):
    """h = bf16(x q gamma) per row of x [rows, k] (bfloat16), q = 1 / sqrt(mean(x^2) + eps) in fp64, and its
    per-row codes [rows, k] and scales [rows] (as qr_quantize_acts of h, with h diag(1/s) when s is given).
    gamma: float32 [k]. Returns (codes, scales) or, with want_h / h given, (codes, scales, h)."""
    _need(x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous(),
          "x must be a contiguous bfloat16 [rows, k] CUDA tensor")
    rows, k = x.shape
    dev = x.device
    _need(gamma.is_cuda and gamma.dtype == torch.float32 and gamma.numel() == k and gamma.is_contiguous(),
          "gamma must be a contiguous float32 [k] CUDA tensor")
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=dev)
    if h is None and want_h:
        h = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    if s is not None:
        _need(s.is_cuda and s.dtype == torch.float32 and s.numel() == k and s.is_contiguous(), "s must be float32 [k]")
    _need(codes.dtype == torch.uint8 and tuple(codes.shape) == (rows, k) and codes.is_contiguous(), "bad codes")
    _need(scales.dtype == torch.float32 and scales.numel() == rows, "bad scales")
    if h is not None:
        _need(h.dtype == torch.bfloat16 and tuple(h.shape) == (rows, k) and h.is_contiguous(), "bad h")
    _check(lib().qr_rmsnorm_quantize(_ptr(x), rows, k, _ptr(gamma), float(eps), _ptr(s), int(qtype), _ptr(codes),
                                     _ptr(scales), _ptr(h), _stream(stream)))
    return (codes, scales, h) if h is not None else (codes, scales)


def qr_moe_combine(y_down, topk_weight, pair_rows, out=None, stream=None):
    """out [T, H] = bf16(sum_j topk_weight[t,j] y_down[pair_rows[t,j]]) (y_down bfloat16 [rows, H])."""
    _need(y_down.is_cuda and y_down.dtype == torch.bfloat16 and y_down.dim() == 2 and y_down.is_contiguous(),
          "y_down must be a contiguous bfloat16 [rows, H] CUDA tensor")
    rows, H = y_down.shape
    T, k = pair_rows.shape
    _need(pair_rows.dtype == torch.int32 and pair_rows.is_contiguous(), "pair_rows must be contiguous int32 [T,k]")
    _need(topk_weight.dtype == torch.float32 and tuple(topk_weight.shape) == (T, k) and topk_weight.is_contiguous(),
          "topk_weight must be contiguous float32 [T,k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y_down.device)
    _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (T, H) and out.is_contiguous(), "bad out")
    _check(lib().qr_moe_combine(_ptr(y_down), rows, H, _ptr(topk_weight), _ptr(pair_rows), T, k, _ptr(out),
                                _stream(stream)))
    return out
