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
    """The library the binding loads: _build/libtdls.so, or the file named
    by TDLS_LIB (the host-sanitized build, for CPU tests)."""
    return os.environ.get("TDLS_LIB") or os.path.join(BUILD, "libtdls.so")


def sanitized_library_path() -> str:
    return os.path.join(BUILD, "libtdls_hostsan.so")


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
    _write_build_info()
    if verbose:
        print(f"linked {lib} in {time.time() - t0:.1f}s", flush=True)
    return lib


def build_host_sanitized(verbose: bool = False) -> str:
    """The host side (argument checks, planner, dispatch: tdls_api.cpp)
    rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer (host code
    only: -Xarch_host before each -fsanitize), linked with the kernel
    objects of the last build into sanitized_library_path().  Load it with
    TDLS_LIB and clang's ASan runtime preloaded."""
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = os.path.join(BUILD, "obj", "tdls_api_hostsan.o")
    _run([HIPCC, *COMMON, *san, "-x", "hip", "-c", os.path.join(CSRC, "tdls_api.cpp"),
          "-o", obj])
    objs = [os.path.join(BUILD, "obj", f"gesv_{sfx}_n{n}_r{nrhs}.o") for sfx, _, n, nrhs in shapes()]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError("build the library first; missing " + ", ".join(missing[:3]))
    out = sanitized_library_path()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan", *san, *objs, obj,
          "-o", out])
    if verbose:
        print(out)
    return out


def _write_build_info():
    """_build/build_info.json: the source revision the library was built
    from (git HEAD and whether the tree had changes), for measurement
    records made where no repository is at hand."""
    import json
    root = os.path.dirname(HERE)
    info = {"built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    try:
        head = subprocess.run(["git", "rev-parse", "HEAD"], cwd=root, stdout=subprocess.PIPE,
                              stderr=subprocess.DEVNULL, text=True, timeout=10)
        dirty = subprocess.run(["git", "status", "--porcelain", "--untracked-files=no"],
                               cwd=root, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                               text=True, timeout=10)
        if head.returncode == 0:
            info["git_head"] = head.stdout.strip()
            info["git_dirty"] = bool(dirty.stdout.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(BUILD, "build_info.json"), "w", encoding="utf-8") as fh:
        json.dump(info, fh)


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized(verbose=True))
    else:
        inc = "--incremental" in sys.argv
        print(build(verbose=True, incremental=inc))
