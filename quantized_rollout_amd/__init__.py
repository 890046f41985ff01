"""quantized_rollout_amd: the quantized-actor W8A8 linear of quantized rollout, MI355X (gfx950) native.

The compute lives in libqr.so (hand-written HIP kernels behind the C ABI of include/qr.h); this package is
its ctypes binding (``_binding``), the in-tree build step (``build``) and the seeded synthetic inputs
(``synth``). The binding loads the library on first use and raises if it is missing: there is no fallback.
"""
from ._binding import (QR_BF16, QR_F32, QR_FP8_E4M3, QR_INT8, W4_GROUP, QRError, Workspace, lib,
                       qr_count_code_changes, qr_moe_combine, qr_moe_route, qr_quantize_acts, qr_quantize_weights,
                       qr_quantize_weights_w4, qr_requantize_weights, qr_rmsnorm_quantize, qr_set_debug, qr_silu_mul_quantize,
                       qr_version,
                       qr_w4a16_linear, qr_w8a8_grouped_linear, qr_w8a8_linear, qr_w8a8_linear_bf16,
                       qr_w8a8_linear_bf16_workspace_bytes, qr_w8a8_linear_noalloc, qr_workspace_bytes)

__all__ = ["QR_BF16", "QR_F32", "QR_FP8_E4M3", "QR_INT8", "W4_GROUP", "QRError", "Workspace", "lib",
           "qr_count_code_changes", "qr_moe_combine", "qr_moe_route", "qr_quantize_acts", "qr_quantize_weights",
           "qr_quantize_weights_w4", "qr_requantize_weights", "qr_rmsnorm_quantize", "qr_set_debug", "qr_silu_mul_quantize",
           "qr_version",
           "qr_w8a8_linear_bf16", "qr_w8a8_linear_bf16_workspace_bytes",
           "qr_w4a16_linear", "qr_w8a8_grouped_linear", "qr_w8a8_linear", "qr_w8a8_linear_noalloc", "qr_workspace_bytes"]
