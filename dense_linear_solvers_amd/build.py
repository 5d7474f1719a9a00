"""Builds the HIP library (libtdls.so) for gfx950 in-tree.

Every shape listed in TDLS_FOR_EACH_SHAPE (csrc/tdls_internal.h) is compiled
from csrc/gesv_inst.hip in its own process, in parallel, then linked with the
host-side interface (csrc/tdls_api.cpp) into _build/libtdls.so.

Flags: -ffp-contract=off (no multiply-add is fused except the kernels'
explicit fma), packed FP32 instructions disabled in device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def library_path() -> str:
    return os.path.join(BUILD, "libtdls.so")


def shapes() -> list:
    """(sfx, Real, N, NRHS) entries of TDLS_FOR_EACH_SHAPE."""
    with open(os.path.join(CSRC, "tdls_internal.h"), encoding="utf-8") as fh:
        text = fh.read()
    body = text[text.index("#define TDLS_FOR_EACH_SHAPE"):]
    body = body[:body.index("\n\n")]
    found = re.findall(r"X\((f32|f64), (float|double), (\d+), (\d+)\)", body)
    if not found:
        raise RuntimeError("no shapes found in tdls_internal.h")
    return [(s, r, int(n), int(m)) for s, r, n, m in found]


def _run(cmd):
    t = time.time()
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l
                    and "argument unused during compilation" not in l)
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return time.time() - t, out


def build(jobs: int = 0, verbose: bool = False, incremental: bool = False) -> str:
    """Compile and link libtdls.so; returns its path.  ``incremental`` skips
    objects newer than every source (a developer convenience; the default
    rebuilds everything)."""
    os.makedirs(os.path.join(BUILD, "obj"), exist_ok=True)
    sources = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, "tdls.h")]
    newest_src = max(os.path.getmtime(s) for s in sources)
    jobs = jobs or min(16, os.cpu_count() or 4)

    cmds = []
    objs = []
    for sfx, real, n, nrhs in shapes():
        obj = os.path.join(BUILD, "obj", f"gesv_{sfx}_n{n}_r{nrhs}.o")
        objs.append(obj)
        cmd = [HIPCC, *COMMON, f"-DTDLS_INST_SFX={sfx}", f"-DTDLS_INST_REAL={real}",
               f"-DTDLS_INST_N={n}", f"-DTDLS_INST_NRHS={nrhs}", "-c",
               os.path.join(CSRC, "gesv_inst.hip"), "-o", obj]
        cmds.append((obj, cmd))
    api_obj = os.path.join(BUILD, "obj", "tdls_api.o")
    objs.append(api_obj)
    cmds.append((api_obj, [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, "tdls_api.cpp"),
                           "-o", api_obj]))
    if incremental:
        cmds = [(o, c) for o, c in cmds
                if not (os.path.exists(o) and os.path.getmtime(o) > newest_src)]
    # biggest shapes first: they are the critical path
    cmds.sort(key=lambda oc: -int(re.search(r"_n(\d+)_", oc[0]).group(1))
              if re.search(r"_n(\d+)_", oc[0]) else 0)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_run, c): o for o, c in cmds}
        for f in cf.as_completed(futs):
            dt, out = f.result()
            if verbose:
                print(f"[{time.time() - t0:6.1f}s] {os.path.basename(futs[f])} ({dt:.1f}s)",
                      flush=True)
                if out.strip():
                    print(out, flush=True)
    lib = library_path()
    tmp = lib + ".tmp%d" % os.getpid()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    if verbose:
        print(f"linked {lib} in {time.time() - t0:.1f}s", flush=True)
    return lib


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    inc = "--incremental" in sys.argv
    print(build(verbose=True, incremental=inc))
