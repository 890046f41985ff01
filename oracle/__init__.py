"""CPU oracle for the quantized-actor W8A8 linear.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library ``libqr.so`` and the
``quantized_rollout_amd`` binding) never imports, links or calls anything here, and the two share no code.

Parts:
  - ``qr_oracle.c`` (plain C, built into ``libqr_oracle.so``) and its ctypes wrapper ``core.py``;
  - ``brute.py``: the same steps in exact rational arithmetic (``fractions.Fraction``) with an explicit
    binary32 rounding model, for tiny inputs; used to pin the C oracle.
"""
