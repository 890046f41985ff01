"""Compile the C oracle (test infrastructure only; see the package docstring)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libqr_oracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Build ``libqr_oracle.so`` with plain IEEE semantics (no contraction, no fast-math)."""
    src = os.path.join(HERE, "qr_oracle.c")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
