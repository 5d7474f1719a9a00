"""Builds the oracle's shared library with gcc (test infrastructure only).

-ffp-contract=off: no multiply-add is fused except the explicit fma calls.
-mfma: those explicit calls become the hardware fused multiply-add.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "_build", "libtdls_oracle.so")


def build(verbose: bool = False, source_dir: str = _HERE, out: str = "") -> str:
    """Compile ``source_dir/gesv_oracle.c`` into ``out`` (default: the
    oracle's own library path)."""
    out = out or library_path()
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-mfma", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", os.path.join(source_dir, "gesv_oracle.c"), "-o", tmp,
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
