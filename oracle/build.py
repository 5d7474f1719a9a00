"""Builds the oracle's shared library with gcc (test infrastructure only).

-ffp-contract=off: no multiply-add is fused except the explicit fma calls.
-mfma: those explicit calls become the hardware fused multiply-add.

``python -m oracle.build --sanitize`` builds a second copy with
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts) at
sanitized_library_path(); the tests load it when TDLS_ORACLE_LIB names it
(with gcc's libasan and libubsan preloaded into the Python process).
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "_build", "libtdls_oracle.so")


def sanitized_library_path() -> str:
    return os.path.join(_HERE, "_build", "libtdls_oracle_san.so")


def build(verbose: bool = False, source_dir: str = _HERE, out: str = "",
          sanitize: bool = False) -> str:
    """Compile ``source_dir/gesv_oracle.c`` into ``out`` (default: the
    oracle's own library path, or the sanitized one)."""
    out = out or (sanitized_library_path() if sanitize else library_path())
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-mfma", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", os.path.join(source_dir, "gesv_oracle.c"), "-o", tmp,
           "-lm"]
    if sanitize:
        cmd[1:1] = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-g"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
