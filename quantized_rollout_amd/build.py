"""Build libqr.so (the gfx950 HIP library) in-tree with hipcc.

Flags: gfx950 only; -O3; no fast-math and no floating-point contraction (the quantizers are bit-exact by
construction and use explicit fused multiply-adds where they want them); packed-fp32 instructions disabled.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqr.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def hipcc_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source to an object (in parallel) and link libqr.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc] + hipcc_flags() + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, text))
        if verbose and text.strip():
            print(text)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
