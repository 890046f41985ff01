"""Host sanitizers on the CPU: the oracle (oracle/qr_oracle.c) and the host side of the C ABI (argument
validation and planning in qr_abi.hip / qr_linear.hip, up to the launch, which the QR_FAULT_INJECT=launch hook
replaces by a refused launch) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven through
every function by the C programs under tests/native/. Any memory error, leak (oracle) or undefined behaviour
aborts the program. Also: the hook in the shipped library, through ctypes in a fresh process."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "quantized_rollout_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _run(cmd, env=None, timeout=600):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env, timeout=timeout)
    return p.returncode, p.stdout.decode(errors="replace")


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    rc, out = _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "oracle", "qr_oracle.c"), os.path.join(NATIVE, "oracle_sanitize.c"), "-lm",
                    "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and out.strip().endswith("ok"), out


def test_abi_host_side_under_asan_ubsan(tmp_path):
    """qr_abi.hip and qr_linear.hip (validation, plans, launch set-up) compiled with host sanitizers (the device
    code is compiled as usual), linked with the other objects of the in-tree build into a library that the C
    test program tests/native/abi_sanitize.c loads."""
    from quantized_rollout_amd import build as B
    objdir = os.path.join(ROOT, "quantized_rollout_amd", "_build")
    rest = [os.path.join(objdir, os.path.basename(s) + ".o") for s in B.sources()
            if os.path.basename(s) not in ("qr_abi.hip", "qr_linear.hip")]
    if not all(os.path.exists(o) for o in rest):
        B.build()
    flags = [f for f in B.hipcc_flags() if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    objs = []
    procs = []
    for name in ("qr_abi.hip", "qr_linear.hip"):
        obj = str(tmp_path / (name + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC] + flags + SAN + ["-c", os.path.join(CSRC, name), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out.decode(errors="replace")
    lib = str(tmp_path / "libqr_san.so")
    rc, out = _run([HIPCC, "--offload-arch=" + B.ARCH, "-shared", "-fPIC"] + SAN + ["-shared-libsan", "-o", lib] +
                   objs + rest)
    assert rc == 0, out
    exe = str(tmp_path / "abi_sanitize")
    rc, out = _run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-shared-libsan", "-I", os.path.join(ROOT, "include"), os.path.join(NATIVE, "abi_sanitize.c"),
                    "-L", str(tmp_path), "-lqr_san", "-Wl,-rpath," + str(tmp_path), "-o", exe])
    assert rc == 0, out
    rc, res = _run([CLANG, "-print-resource-dir"])
    assert rc == 0, res
    rt = glob.glob(os.path.join(res.strip(), "lib", "*", "libclang_rt.asan-x86_64.so"))
    assert rt, "no shared AddressSanitizer runtime under " + res
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1",
               LD_LIBRARY_PATH=os.path.dirname(rt[0]) + os.pathsep + os.environ.get("LD_LIBRARY_PATH", ""))
    env.pop("QR_TUNE", None)
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and out.strip().endswith("ok"), out


FAULT_SCRIPT = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
from quantized_rollout_amd import _binding as B
L = B.lib()
P = [ctypes.c_void_p(0x7F0000000000 + (i << 20)) for i in range(8)]
res = {}
res["linear"] = L.qr_w8a8_linear(1, 16, 1536, 1536, P[0], P[1], P[2], P[3], P[4], 1, None, P[5], 1 << 30, None)
res["linear_text"] = L.qr_last_error().decode()
res["quantize"] = L.qr_quantize_weights(P[0], 1, 64, 256, None, 0, P[1], P[2], None)
res["bad_k"] = L.qr_w8a8_linear(1, 16, 1536, 1530, P[0], P[1], P[2], P[3], P[4], 1, None, P[5], 1 << 30, None)
try:
    B._check(res["linear"])
except B.QRError as e:
    res["raised"] = [e.status, str(e)]
print(json.dumps(res))
"""


def test_fault_injection_hook_in_the_shipped_library():
    """QR_FAULT_INJECT=launch: a call that passes validation returns QR_ERR_HIP with the injected text (and the
    binding raises it) instead of launching; validation errors keep their own status."""
    env = dict(os.environ, QR_FAULT_INJECT="launch")
    rc, out = _run([sys.executable, "-c", FAULT_SCRIPT, ROOT], env=env, timeout=300)
    assert rc == 0, out
    res = json.loads(out.strip().splitlines()[-1])
    assert res["linear"] == 5 and "injected" in res["linear_text"], res
    assert res["quantize"] == 5 and res["bad_k"] == 2, res
    assert res["raised"][0] == 5 and "QR_ERR_HIP" in res["raised"][1], res
