#!/usr/bin/env python3
"""Benchmark of the batched gesv path on one MI355X.

One step = one call of the solver over the whole batch: load, pivot search,
row exchange, elimination with the forward substitution folded in, back
substitution and store, all in one kernel launch.  The default workload is
n = 32, nrhs = 1, batch = 262144, float64, column-major, A and B iid N(0, 1)
(the recipe ``n32_f64_col``; with seed 0 no system needs a pivot-gap redraw,
which tests/test_workloads.py checks over the whole batch), inputs resident
in HBM before timing starts.

Prints one JSON line.  ``value`` is systems solved per second over the
timed steps (wall clock, launches back to back); the roofline object
prices the kernel's algorithmic HBM bytes per launch against 8 TB/s, over
the mean of per-launch HIP-event times on the launch stream (median, min
and max are reported beside it); ``issue_floor`` is the VALU issue floor
from the committed SQ counters (when they match the sources);
``cpu_baseline`` is the plain CPU oracle timed on this host's cores on the
same inputs.  Working sets below 512 MiB rotate over several buffer sets so
that no launch is served from the 256 MB Infinity Cache.  After timing,
``api_wall_ms`` samples synchronous calls (allocation, submission,
execution and the wait), the ruSOLVER page's own measure.

  python bench.py [--steps K] [--warmup W] [--workload NAME]
                  [--op gesv|getrf|getrs|potrf|potrs|posv] [--interleave W] [--no-cpu]
  python bench.py --calibrate-copy      # a plain 1 GiB device copy, for
                                        # scaling the HBM byte counters
  python bench.py [--workload NAME] [--op OP] --summarize-counters \
                  FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
  python bench.py [--workload NAME] [--op OP] --summarize-sq PMC_DIR [PMC_DIR ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
FP64_VECTOR_PEAK_TFLOPS = 78.6   # MI355X, published
FP32_VECTOR_PEAK_TFLOPS = 157.3
METRIC = "systems/sec + achieved HBM GB/s, batched LUPP gesv n=32 fp32/fp64"
ROTATE_BELOW = 512 << 20         # working sets below this rotate buffer sets (MALL is 256 MB)
SIMDS = 1024                     # MI355X: 256 CUs x 4 SIMDs
CLOCK_GHZ = 2.4                  # MI355X peak engine clock, published
DEFAULT_WORKLOAD = "n32_f64_col"


def algorithmic_bytes(n: int, nrhs: int, es: int, op: str = "gesv") -> int:
    """Bytes the method must move per system.  gesv: A and B read once, X,
    piv and info written once.  getrf: A read once, LU, piv and info
    written once.  getrs: LU, piv and B read once, X written once.
    potrs reads only the lower triangle of L (the rest of the matrix is
    never part of its input)."""
    if op == "getrf":
        return 2 * n * n * es + 4 * n + 4
    if op == "getrs":
        return n * n * es + 4 * n + 2 * n * nrhs * es
    if op == "potrf":                    # A read, L written, info
        return 2 * n * n * es + 4
    if op == "potrs":                    # L's lower triangle, B read, X written
        return n * (n + 1) // 2 * es + 2 * n * nrhs * es
    if op == "posv":                     # A, B read, X, info written
        return n * n * es + 2 * n * nrhs * es + 4
    return n * n * es + 2 * n * nrhs * es + 4 * n + 4


def triangle_line_bytes(n: int, nrhs: int, es: int, layout: str) -> int:
    """potrs per system, priced by the 128-byte lines its input forces: the
    lines of a contiguous n x n matrix (the batch starts line-aligned and
    n*n*es is a multiple of 128 for every kernel size) that hold part of
    the lower triangle, plus B read and X written.  Reading a triangle out
    of a dense matrix fetches whole lines, so this is the traffic a potrs of
    this layout cannot avoid."""
    lines = set()
    for i in range(n):
        for j in range(i + 1):
            off = (j * n + i if layout == "col" else i * n + j) * es
            lines.add(off // 128)
    return len(lines) * 128 + 2 * n * nrhs * es


def algorithmic_flops(n: int, nrhs: int, op: str = "gesv") -> int:
    """Per system: elimination 2*sum(m^2) multiply-add flops plus sum(m)
    divisions (m = n-1 .. 1), forward and back substitution on nrhs columns
    2*n*(n-1) + n each; getrf counts the elimination, getrs the
    substitutions.  Cholesky: the factorization below, and solves that
    divide in both substitutions (2*n*(n-1) + 2*n per column)."""
    s2 = sum(m * m for m in range(1, n))
    s1 = sum(range(1, n))
    elim = 2 * s2 + s1
    subst = nrhs * (2 * n * (n - 1) + n)
    # Cholesky: column j costs j multiply-adds for the diagonal, (n-1-j)*j
    # for the entries below it, one square root and n-1-j divisions
    chol = sum(2 * j + 1 + (n - 1 - j) * (2 * j + 1) for j in range(n))
    # Cholesky solves divide in both substitutions
    chol_subst = nrhs * (2 * n * (n - 1) + 2 * n)
    return {"getrf": elim, "getrs": subst, "potrf": chol, "potrs": chol_subst,
            "posv": chol + chol_subst}.get(op, elim + subst)


def _code_only(text: str) -> str:
    """C/C++ source without comments, blank lines and indentation (so that a
    comment or layout edit does not mark the counters as stale)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (" ".join(re.sub(r"//.*$", "", ln).split()) for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_linear_solvers_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# the kernel each op launches (rocprofv3 -T truncates names to these)
KERNEL_OF_OP = {"gesv": "gesv_panel_kernel", "getrf": "gesv_panel_kernel",
                "getrs": "getrs_kernel", "potrf": "chol_kernel", "potrs": "chol_kernel",
                "posv": "chol_kernel"}


def traffic_path(workload: str, op: str) -> str:
    return os.path.join(ROOT, "profiles", f"{op}_{workload}_traffic.txt")


TRAFFIC_MARKER = "# data (read by bench.py while kernel_source_hash matches the sources):"


def traffic_lines(d: dict) -> list:
    """The data lines of a traffic summary: ``key = value``, one a line."""
    return [f"{k} = {v}" for k, v in d.items()]


def read_traffic(path: str) -> dict:
    """The ``key = value`` lines of a traffic summary (comments skipped)."""
    d = {}
    with open(path, encoding="utf-8") as fh:
        for line in fh:
            if line.startswith("#") or " = " not in line:
                continue
            k, v = line.rstrip("\n").split(" = ", 1)
            d[k] = v
    return d


def _line_bytes_entry(w, es: int, kernel_ms: float) -> dict:
    """potrs against the whole lines its triangle occupies (see
    triangle_line_bytes), next to the triangle-only roofline."""
    per = triangle_line_bytes(w.n, w.nrhs, es, w.layout)
    gbs = per * w.batch / (kernel_ms * 1e-3) / 1e9
    return {"bytes_per_system": per, "vs_triangle": per / algorithmic_bytes(w.n, w.nrhs, es, "potrs"),
            "achieved": gbs, "frac": gbs / HBM_PEAK_GBS}


def measured_traffic(workload: str, op: str = "gesv"):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = traffic_path(workload, op)
    if not os.path.exists(path):
        return None
    d = read_traffic(path)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    v = d.get("hbm_bytes_per_launch")
    return float(v) if v is not None else None


def _counter_values(csv_dir: str, counter: str, kernel_prefix: str) -> list:
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        with open(f, encoding="utf-8") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and r["Kernel_Name"].startswith(kernel_prefix):
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} values for {kernel_prefix} under {csv_dir}")
    return vals


def summarize_counters(workload: str, op: str, fetch_dir: str, write_dir: str,
                       copy_fetch_dir: str, copy_write_dir: str,
                       copy_bytes: int = 1 << 30) -> dict:
    """HBM bytes per launch of the solver kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for a plain device copy of ``copy_bytes`` bytes."""
    kern = KERNEL_OF_OP[op]
    fk = float(np.median(_counter_values(fetch_dir, "FETCH_SIZE", kern)))
    wk = float(np.median(_counter_values(write_dir, "WRITE_SIZE", kern)))
    cf = float(np.median(_counter_values(copy_fetch_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer")))
    cw = float(np.median(_counter_values(copy_write_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer")))
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    fetch_b = fk * 1024.0 * fetch_scale
    write_b = wk * 1024.0 * write_scale
    d = {"workload": workload, "op": op, "kernel": kern,
         "kernel_source_hash": kernel_source_hash(),
         "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
         "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
         "fetch_scale": fetch_scale, "write_scale": write_scale,
         "hbm_read_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
         "hbm_bytes_per_launch": fetch_b + write_b}
    out = traffic_path(workload, op)
    from dense_linear_solvers_amd.workloads import RECIPES, SPD_RECIPES
    r = RECIPES.get(workload) or SPD_RECIPES.get(workload)
    es = 8 if (r is not None and r.dtype == "f64") else 4
    algo = algorithmic_bytes(r.n, r.nrhs, es, op) * r.batch if r is not None else None
    pre = f"gpurun_out/pf/{op}_{workload}"
    cmd = f"python3 bench.py --workload {workload} --op {op} --no-cpu --steps 3 --warmup 1"
    head = [f"# HBM traffic of {kern} ({op}) on {workload}: rocprofv3 FETCH_SIZE and WRITE_SIZE per "
            "dispatch, each scaled by the same counter on a plain copy",
            "# commands (repository root, one MI355X), each counter in a run of its own:",
            f"#   rocprofv3 --pmc FETCH_SIZE -T -d {pre}_FETCH_SIZE -o t -f csv -- {cmd}",
            f"#   rocprofv3 --pmc WRITE_SIZE -T -d {pre}_WRITE_SIZE -o t -f csv -- {cmd}",
            "#   rocprofv3 --pmc FETCH_SIZE -T -d gpurun_out/pf/copy_FETCH_SIZE -o t -f csv -- "
            "python3 bench.py --calibrate-copy",
            "#   rocprofv3 --pmc WRITE_SIZE -T -d gpurun_out/pf/copy_WRITE_SIZE -o t -f csv -- "
            "python3 bench.py --calibrate-copy",
            f"#   python3 bench.py --workload {workload} --op {op} --summarize-counters "
            f"{pre}_FETCH_SIZE {pre}_WRITE_SIZE gpurun_out/pf/copy_FETCH_SIZE "
            "gpurun_out/pf/copy_WRITE_SIZE",
            "#",
            f"# calibration: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE = {cf:.0f} KiB and "
            f"WRITE_SIZE = {cw:.0f} KiB: fetch scale {fetch_scale:.4f}, write scale {write_scale:.4f}",
            f"# {kern} (median over dispatches): FETCH_SIZE {fk:.0f} KiB, WRITE_SIZE {wk:.0f} KiB; "
            f"scaled: read {fetch_b:.4e} B, write {write_b:.4e} B, total {fetch_b + write_b:.4e} B "
            "per launch" + (f" against {algo:.4e} B algorithmic "
                            f"({100 * ((fetch_b + write_b) / algo - 1):+.1f}%)" if algo else ""),
            TRAFFIC_MARKER]
    with open(out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(head + traffic_lines(d)) + "\n")
        fh.write("\n")
    return d


# the two SQ counter passes (eight SQ counters at most per rocprofv3 run)
SQ_PASSES = {
    "sqa": "SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
           "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_SCA",
    "sqb": "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT "
           "SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES SQ_IFETCH",
}


def sq_path(workload: str, op: str) -> str:
    return os.path.join(ROOT, "profiles", f"{op}_{workload}_sq_counters.txt")


def summarize_sq(workload: str, op: str, dirs: list) -> dict:
    """Per-wave SQ counters of the solver kernel from rocprofv3 --pmc runs
    (one directory per pass): each counter's median over dispatches of its
    per-dispatch total, divided by the waves of a launch (grid threads / 64).
    Counters named *CYCLES* or SQ_ACTIVE_INST_* / SQ_WAIT_* count quad-cycles
    (4 clock cycles), except SQ_BUSY_CYCLES and SQ_LDS_* (clock cycles), as
    rocprofv3's counter list states."""
    import csv
    import glob
    kern = KERNEL_OF_OP[op]
    per = {}          # counter -> list of per-dispatch totals
    waves = None
    for d in dirs:
        for f in glob.glob(os.path.join(d, "*counter_collection.csv")):
            rows = {}
            with open(f, encoding="utf-8") as fh:
                for r in csv.DictReader(fh):
                    if not r["Kernel_Name"].startswith(kern):
                        continue
                    rows.setdefault((r["Dispatch_Id"], r["Counter_Name"]), 0.0)
                    rows[(r["Dispatch_Id"], r["Counter_Name"])] += float(r["Counter_Value"])
                    waves = int(r["Grid_Size"]) // 64
            for (_, c), v in rows.items():
                per.setdefault(c, []).append(v)
    if not per:
        raise SystemExit(f"no counters for {kern} under {dirs}")
    d = {"workload": workload, "op": op, "kernel": kern,
         "kernel_source_hash": kernel_source_hash(), "waves_per_launch": waves}
    for c in sorted(per):
        d[f"{c}_per_wave"] = float(np.median(per[c])) / waves
    q = d.get("SQ_ACTIVE_INST_VALU_per_wave")
    if q is not None:
        d["valu_floor_ms"] = waves * q * 4 / SIMDS / (CLOCK_GHZ * 1e6)
    out = sq_path(workload, op)
    cmd = f"python3 bench.py --workload {workload} --op {op} --no-cpu --steps 3 --warmup 1"
    head = [f"# SQ counters of {kern} ({op}) on {workload}: per wave, the median over dispatches of "
            "each counter's per-dispatch total divided by the waves of a launch (grid threads / 64).",
            "# SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count quad-cycles (4 clock cycles); "
            "SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE and SQ_BUSY_CYCLES count clock cycles "
            "(SQ_BUSY_CYCLES per shader engine).",
            "# valu_floor_ms = waves x SQ_ACTIVE_INST_VALU x 4 cycles / 1024 SIMDs / 2.4 GHz.",
            "# commands (repository root, one MI355X), one pass each:"]
    for d_ in dirs:
        tag = os.path.basename(os.path.normpath(d_))
        cs = (SQ_PASSES.get(tag[-3:]) if tag[-3:] in SQ_PASSES else None)
        if cs:
            head.append(f"#   rocprofv3 --pmc {cs} -T -d gpurun_out/pf/{tag} -o t -f csv -- {cmd}")
    head += [f"#   python3 bench.py --workload {workload} --op {op} --summarize-sq "
             + " ".join(f"gpurun_out/pf/{os.path.basename(os.path.normpath(d_))}" for d_ in dirs),
             TRAFFIC_MARKER]
    with open(out, "w", encoding="utf-8") as fh:
        fh.write("\n".join(head + traffic_lines(d)) + "\n")
    return d


def stats_path(workload: str, op: str) -> str:
    return os.path.join(ROOT, "profiles", f"{op}_{workload}_kernel_stats.txt")


def summarize_trace(workload: str, op: str, trace_dir: str, bench_out: str, command: str) -> dict:
    """profiles/<op>_<workload>_kernel_stats.txt from a rocprofv3
    --kernel-trace --stats run of bench.py: the stats table, the solver
    kernel's average launch time, and the bench line the same run printed
    (its per-launch HIP-event times), so the two can be compared."""
    import csv
    import glob
    kern = KERNEL_OF_OP[op]
    files = glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    with open(files[0], encoding="utf-8") as fh:
        text = fh.read()
    rows = list(csv.DictReader(text.splitlines()))
    mine = [r for r in rows if r["Name"].startswith(kern)]
    if not mine:
        raise SystemExit(f"no {kern} row in {files[0]}")
    r = mine[0]
    avg_ms = float(r["AverageNs"]) * 1e-6
    line = None
    with open(bench_out, encoding="utf-8") as fh:
        for ln in fh:
            if ln.startswith("{"):
                line = json.loads(ln)
    d = {"workload": workload, "op": op, "kernel": kern,
         "kernel_source_hash": kernel_source_hash(), "calls": int(r["Calls"]),
         "trace_avg_ms": avg_ms, "trace_min_ms": float(r["MinNs"]) * 1e-6,
         "trace_max_ms": float(r["MaxNs"]) * 1e-6}
    head = [f"# rocprofv3 kernel statistics: {op} on {workload}",
            "# command (repository root, one MI355X):", f"#   {command}", "#"]
    for ln in text.strip().splitlines():
        head.append("# " + ln)
    if line is not None:
        kl = line["kernel_ms_per_launch"]
        d.update({"bench_kernel_ms_mean": kl["mean"], "bench_kernel_ms_median": kl["median"],
                  "bench_kernel_ms_min": kl["min"], "bench_kernel_ms_max": kl["max"],
                  "bench_ms_per_step": line["ms_per_step"],
                  "trace_vs_bench_mean": avg_ms / kl["mean"] - 1.0})
        head += ["#", f"# {kern}: trace average {avg_ms:.4f} ms over {r['Calls']} dispatches "
                 f"(min {d['trace_min_ms']:.4f}, max {d['trace_max_ms']:.4f}); the same run's "
                 f"bench line: per-launch HIP events mean {kl['mean']:.4f} ms, median "
                 f"{kl['median']:.4f}, min {kl['min']:.4f}, max {kl['max']:.4f}; ms_per_step "
                 f"{line['ms_per_step']:.4f} (trace average {100 * d['trace_vs_bench_mean']:+.1f}% "
                 "from the event mean)"]
    head.append(TRAFFIC_MARKER)
    with open(stats_path(workload, op), "w", encoding="utf-8") as fh:
        fh.write("\n".join(head + traffic_lines(d)) + "\n")
    return d


def issue_floor(workload: str, op: str):
    """VALU issue floor of one launch from the committed SQ summary, when it
    was taken on the current kernel sources and at this batch: every wave's
    VALU-active quad-cycles, 4 cycles each, spread over the 1024 SIMDs at the
    2.4 GHz peak clock.  The recipe's own batch only."""
    path = sq_path(workload, op)
    if not os.path.exists(path):
        return None
    d = read_traffic(path)
    if d.get("kernel_source_hash") != kernel_source_hash() or "valu_floor_ms" not in d:
        return None
    return {"valu_floor_ms": float(d["valu_floor_ms"]),
            "valu_active_quad_cycles_per_wave": float(d["SQ_ACTIVE_INST_VALU_per_wave"]),
            "waves_per_launch": int(d["waves_per_launch"]),
            "source": os.path.relpath(path, ROOT)}


def run_info() -> dict:
    """Device, software and source identity of a measurement (the ruSOLVER
    page records configuration, device and source with every timing)."""
    import platform
    import torch
    info = {"device": torch.cuda.get_device_name(0),
            "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
            "hip": torch.version.hip, "torch": torch.__version__,
            "host_cpu": platform.processor() or None,
            "kernel_source_hash": kernel_source_hash()}
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["host_cpu"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    bi = os.path.join(ROOT, "dense_linear_solvers_amd", "_build", "build_info.json")
    if os.path.exists(bi):
        with open(bi, encoding="utf-8") as fh:
            info["library_build"] = json.load(fh)
    return info


def interleave(x: np.ndarray, W: int) -> np.ndarray:
    """[batch, ...] -> [blocks, ..., W]: element e of system s at
    (s // W) W E + s % W + e W (the last block padded with zeros)."""
    batch = x.shape[0]
    blocks = -(-batch // W)
    pad = np.zeros((blocks * W,) + x.shape[1:], dtype=x.dtype)
    pad[:batch] = x
    pad = pad.reshape((blocks, W) + x.shape[1:])
    return np.ascontiguousarray(np.moveaxis(pad, 1, -1))


def deinterleave(t, batch: int):
    """Inverse of ``interleave`` for a torch tensor."""
    return t.movedim(-1, 1).reshape((-1,) + tuple(t.shape[1:-1]))[:batch].contiguous()


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "reps": reps, "ms": dt * 1e3, "gbs": 2 * nbytes / dt / 1e9}), flush=True)


def cpu_baseline(w, op: str = "gesv", min_seconds: float = 10.0,
                 max_seconds: float = 30.0, threads: int = 0) -> dict:
    """The CPU oracle, as it stands, on all cores of this host (or on
    ``threads`` of them), over the same inputs; repeated until at least
    ``min_seconds`` of work."""
    sys.path.insert(0, ROOT)
    import oracle
    cores = len(os.sched_getaffinity(0))
    if threads > 0:
        cores = min(cores, threads)
    A = np.ascontiguousarray(w.A)
    B = np.ascontiguousarray(w.B)
    n, nrhs, layout = w.n, w.nrhs, w.layout
    if op == "potrs":
        Lf, _ = oracle.potrf(A, n, layout, nthreads=cores)
        Lf = oracle.to_storage(Lf, layout)
    if op == "getrs":
        LU, ipiv, finfo, _ = oracle.getrf(A, n, layout, nthreads=cores)
        LU = oracle.to_storage(LU, layout)
        ipiv = np.where(finfo[:, None] != 0, -1, ipiv).astype(np.int32)

    def run(cnt):
        if op == "getrf":
            oracle.getrf(A[:cnt], n, layout, nthreads=cores)
        elif op == "potrf":
            oracle.potrf(A[:cnt], n, layout, nthreads=cores)
        elif op == "posv":
            oracle.posv(A[:cnt], B[:cnt], n, nrhs, layout, nthreads=cores)
        elif op == "potrs":
            oracle.potrs(Lf[:cnt], B[:cnt], n, nrhs, layout, nthreads=cores)
        elif op == "getrs":
            oracle.getrs(LU[:cnt], ipiv[:cnt], B[:cnt], n, nrhs, layout, nthreads=cores)
        else:
            oracle.gesv(A[:cnt], B[:cnt], n, nrhs, layout, nthreads=cores)

    # size one pass: the whole batch, or a prefix when a pass is too long
    t = time.perf_counter()
    run(2048)
    per_sys = max((time.perf_counter() - t) / 2048, 1e-9)
    count = int(min(w.batch, max(2048, max_seconds / 3 / per_sys)))
    passes, solved = 0, 0
    t = time.perf_counter()
    while True:
        run(count)
        passes += 1
        solved += count
        el = time.perf_counter() - t
        if el >= min_seconds or el + el / passes > max_seconds:
            break
    return {"value": solved / el, "unit": "systems/s", "cores": cores, "kind": "oracle",
            "sample": f"first {count} of the {w.batch} systems, {passes} passes, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--op", default="gesv",
                    choices=["gesv", "getrf", "getrs", "potrf", "potrs", "posv"],
                    help="gesv (default: factor and solve in one call), getrf (factor only), "
                         "getrs (solve from factors made, untimed, by getrf), or the Cholesky "
                         "potrf / potrs (from factors made, untimed, by potrf) / posv (on an "
                         "spd_* workload)")
    ap.add_argument("--batch", type=int, default=0, help="override the recipe's batch")
    ap.add_argument("--interleave", type=int, default=1,
                    help="store the batch with W systems interleaved element by element "
                         "(W = batch: structure of arrays); the *_ex calls")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rotate", action="store_true",
                    help="one buffer set even when the working set is below 512 MiB")
    ap.add_argument("--api-samples", type=int, default=10,
                    help="synchronous API wall-clock samples after the timed region")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "BENCH_OUT", "COMMAND"),
                    help="write profiles/<op>_<workload>_kernel_stats.txt from a rocprofv3 "
                         "--kernel-trace --stats directory and the bench line of the same run")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PMC_DIR",
                    help="write profiles/<op>_<workload>_sq_counters.txt from rocprofv3 --pmc "
                         "output directories of SQ counters (no GPU needed)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle baseline (default: every core of the process)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                             "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the data lines of profiles/<op>_<workload>_traffic.txt from rocprofv3 --pmc "
                         "output directories (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.workload, args.op, *args.summarize_trace), indent=1))
        return
    if args.summarize_sq:
        print(json.dumps(summarize_sq(args.workload, args.op, args.summarize_sq), indent=1))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.workload, args.op, *args.summarize_counters),
                         indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the batched solver shards systems across GPUs "
              "with no communication, so one GPU's share is what it measures.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return

    sys.path.insert(0, ROOT)
    import dense_linear_solvers_amd as tdls
    from dense_linear_solvers_amd import workloads

    t_gen = time.perf_counter()
    w = workloads.make(args.workload, seed=0, batch=args.batch or None)
    print(f"[bench] inputs {w.name} n={w.n} nrhs={w.nrhs} batch={w.batch} {w.dtype} "
          f"{w.layout} generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    W = max(1, args.interleave)
    if W > w.batch:
        raise SystemExit("--interleave must not exceed the batch")
    ex = {"interleave": W, "batch": w.batch} if W > 1 else {}
    A_host = interleave(w.A, W) if W > 1 else w.A
    B_host = interleave(w.B, W) if W > 1 else w.B
    stream = torch.cuda.current_stream(dev)
    op = args.op
    plan = tdls.plan_op(op, w.dtype, w.layout, w.n, w.nrhs, w.batch)

    def make_set():
        """Device buffers of one step: inputs (factors made here, untimed,
        for getrs / potrs) and outputs."""
        d = {"A": torch.from_numpy(A_host).to(dev), "B": torch.from_numpy(B_host).to(dev)}
        d["X"] = torch.empty_like(d["B"])
        d["piv"] = torch.empty((d["A"].shape[0], w.n, W) if W > 1 else (w.batch, w.n),
                               dtype=torch.int32, device=dev)
        d["info"] = torch.empty((w.batch,), dtype=torch.int32, device=dev)
        if op in ("getrf", "getrs"):
            d["LU"] = torch.empty_like(d["A"])
        if op == "getrs":
            tdls.getrf_batched(d["A"], w.layout, out=(d["LU"], d["piv"], d["info"]), **ex)
        if op in ("potrf", "potrs"):
            d["L"] = torch.empty_like(d["A"])
        if op == "potrs":
            tdls.potrf_batched(d["A"], w.layout, out=(d["L"], d["info"]), **ex)
        return d

    def run(d):
        if op == "gesv":
            tdls.gesv_batched(d["A"], d["B"], w.layout, out=(d["X"], d["piv"], d["info"]), **ex)
        elif op == "getrf":
            tdls.getrf_batched(d["A"], w.layout, out=(d["LU"], d["piv"], d["info"]), **ex)
        elif op == "getrs":
            tdls.getrs_batched(d["LU"], d["piv"], d["B"], w.layout, out=d["X"], **ex)
        elif op == "potrf":
            tdls.potrf_batched(d["A"], w.layout, out=(d["L"], d["info"]), **ex)
        elif op == "potrs":
            tdls.potrs_batched(d["L"], d["B"], w.layout, out=d["X"], **ex)
        else:
            tdls.posv_batched(d["A"], d["B"], w.layout, out=(d["X"], d["info"]), **ex)

    def raw_call(d):
        """The C entry point itself with the pointers of buffer set d,
        marshalled once: the timed loop then measures the library call and
        its kernel, not the Python wrapper's argument checks (run(d) takes
        the checked path once per set, before timing)."""
        lib = tdls.load_library()
        dt = tdls.F64 if w.dtype == "f64" else tdls.F32
        lay = tdls.COL_MAJOR if w.layout == "col" else tdls.ROW_MAJOR
        st = stream.cuda_stream
        p = {k: v.data_ptr() for k, v in d.items()}
        n, nrhs, b = w.n, w.nrhs, w.batch
        if W > 1:
            from dense_linear_solvers_amd import _binding as bd
            import ctypes
            o = ctypes.byref(bd.Options(0, 0, W))
            f = {"gesv": lambda: lib.tdls_gesv_batched_ex(dt, lay, n, nrhs, b, o, p["A"], p["B"],
                                                           p["X"], p["piv"], p["info"], st),
                 "getrf": lambda: lib.tdls_getrf_batched_ex(dt, lay, n, b, o, p["A"], p["LU"],
                                                             p["piv"], p["info"], st),
                 "getrs": lambda: lib.tdls_getrs_batched_ex(dt, lay, n, nrhs, b, o, p["LU"],
                                                             p["piv"], p["B"], p["X"], st),
                 "potrf": lambda: lib.tdls_potrf_batched_ex(dt, lay, n, b, 0.0, o, p["A"], p["L"],
                                                             p["info"], st),
                 "potrs": lambda: lib.tdls_potrs_batched_ex(dt, lay, n, nrhs, b, o, p["L"],
                                                             p["B"], p["X"], st),
                 "posv": lambda: lib.tdls_posv_batched_ex(dt, lay, n, nrhs, b, 0.0, o, p["A"],
                                                           p["B"], p["X"], p["info"], st)}[op]
        else:
            f = {"gesv": lambda: lib.tdls_gesv_batched(dt, lay, n, nrhs, b, p["A"], p["B"], p["X"],
                                                        p["piv"], p["info"], st),
                 "getrf": lambda: lib.tdls_getrf_batched(dt, lay, n, b, p["A"], p["LU"], p["piv"],
                                                          p["info"], st),
                 "getrs": lambda: lib.tdls_getrs_batched(dt, lay, n, nrhs, b, p["LU"], p["piv"],
                                                          p["B"], p["X"], st),
                 "potrf": lambda: lib.tdls_potrf_batched(dt, lay, n, b, 0.0, p["A"], p["L"],
                                                          p["info"], st),
                 "potrs": lambda: lib.tdls_potrs_batched(dt, lay, n, nrhs, b, p["L"], p["B"],
                                                          p["X"], st),
                 "posv": lambda: lib.tdls_posv_batched(dt, lay, n, nrhs, b, 0.0, p["A"], p["B"],
                                                        p["X"], p["info"], st)}[op]
        return f

    # Buffer rotation: a working set below 512 MiB could be served from the
    # 256 MB Infinity Cache when one launch follows another on the same
    # buffers, so such workloads rotate over enough sets to exceed 512 MiB
    # (at least 3); larger ones use one set.
    sets = [make_set()]
    ws_bytes = sum(t.numel() * t.element_size() for t in sets[0].values())
    nsets = 1 if ws_bytes >= ROTATE_BELOW or args.no_rotate else \
        min(4096, max(3, -(-ROTATE_BELOW // ws_bytes)))
    sets += [make_set() for _ in range(nsets - 1)]
    torch.cuda.synchronize()

    for d in sets:               # the checked call once per set
        run(d)
    calls = [raw_call(d) for d in sets]
    for i in range(args.warmup):
        rc = calls[i % nsets]()
        if rc != 0:
            raise SystemExit(f"{op}: {tdls.strerror(rc)}")
    torch.cuda.synchronize()

    # the timed region: exactly `steps` launches, one event pair around each
    # (on the launch stream) for the per-launch kernel time
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        calls[i % nsets]()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = np.array([a.elapsed_time(b) for a, b in evs])
    kernel_ms = float(per_launch.mean())
    ms_per_step = wall * 1e3 / args.steps

    # Secondary: synchronous API wall-clock per call (the ruSOLVER page's
    # measure: output allocation, submission, execution and the wait; no
    # upload or check), one sample per call
    api = []
    for i in range(args.api_samples):
        d = sets[i % nsets]
        t = time.perf_counter()
        if op == "gesv":
            tdls.gesv_batched(d["A"], d["B"], w.layout, **ex)
        else:
            run(d)
        torch.cuda.synchronize()
        api.append((time.perf_counter() - t) * 1e3)
    d0 = sets[0]
    A, B, X, piv, info = d0["A"], d0["B"], d0["X"], d0["piv"], d0["info"]
    LU = d0.get("LU")

    # sanity of the timed output (no oracle here): status and a residual
    # sample (for getrf: the solve of the timed factors)
    if op == "getrf":
        tdls.getrs_batched(LU, piv, B, w.layout, out=X, **ex)
        torch.cuda.synchronize()
    if op == "potrf":
        tdls.posv_batched(A, B, w.layout, out=(X, info), **ex)
        torch.cuda.synchronize()
    if W > 1:   # back to one system after another for the check
        A, B, X = (deinterleave(t, w.batch) for t in (A, B, X))
    info_h = info.cpu().numpy()
    rng = np.random.default_rng(0)
    sample = torch.from_numpy(rng.choice(w.batch, size=min(w.batch, 512), replace=False)).to(dev)
    As = A[sample].double()
    Xs = X[sample].double()
    Bs = B[sample].double()
    if w.layout == "col":
        As, Xs, Bs = As.transpose(1, 2), Xs.transpose(1, 2), Bs.transpose(1, 2)
    res = (torch.bmm(As.contiguous(), Xs.contiguous()) - Bs).abs().amax(dim=(1, 2))
    eps = 2.0 ** -52 if w.dtype == "f64" else 2.0 ** -23
    den = w.n * eps * As.abs().sum(dim=2).amax(dim=1) * Xs.abs().amax(dim=(1, 2))
    ok = info[sample] == 0
    resid_max = float((res[ok] / den[ok]).max().item()) if bool(ok.any()) else 0.0

    es = 8 if w.dtype == "f64" else 4
    bytes_per_launch = algorithmic_bytes(w.n, w.nrhs, es, op) * w.batch
    flops_per_launch = algorithmic_flops(w.n, w.nrhs, op) * w.batch
    achieved_gbs = bytes_per_launch / (kernel_ms * 1e-3) / 1e9
    achieved_tflops = flops_per_launch / (kernel_ms * 1e-3) / 1e12
    vec_peak = FP64_VECTOR_PEAK_TFLOPS if w.dtype == "f64" else FP32_VECTOR_PEAK_TFLOPS
    systems_per_s = w.batch / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": systems_per_s,
        "unit": "systems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "op": op, "n": w.n, "nrhs": w.nrhs, "batch": w.batch,
                   **({"interleave": W} if W > 1 else {}),
                   "layout": "column-major" if w.layout == "col" else "row-major",
                   "distribution": w.meta.get("recipe") + (
                       " (redraw off here: no system was redrawn)"
                       if w.meta.get("gap_filtered") is False else ""), "seed": 0,
                   **({"gap_filtered": False} if "gap_filtered" in w.meta else {}),
                   "group_size": plan["group_size"], "systems_per_wave": plan["systems_per_wave"]},
        "kernel_ms": kernel_ms,
        "kernel_ms_per_launch": {"mean": kernel_ms, "median": float(np.median(per_launch)),
                                 "min": float(per_launch.min()), "max": float(per_launch.max()),
                                 "launches": int(len(per_launch))},
        "api_wall_ms": ({"median": float(np.median(api)), "min": float(min(api)),
                         "max": float(max(api)), "samples": len(api)} if api else None),
        "buffer_sets": {"sets": nsets, "working_set_bytes": int(ws_bytes),
                        "rotated": nsets > 1},
        "hbm_gbs_algorithmic": achieved_gbs,
        "vector_tflops_algorithmic": achieved_tflops,
        "vector_frac": achieved_tflops / vec_peak,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(w.name, op)},
        **({"potrs_line_bytes": _line_bytes_entry(w, es, kernel_ms)} if op == "potrs" and W == 1
           else {}),
        "issue_floor": issue_floor(w.name, op) if not args.batch and W == 1 else None,
        "hbm_floor_ms": bytes_per_launch / (HBM_PEAK_GBS * 1e9) * 1e3,
        "run": run_info(),
        "check": {"failed_systems": int((info_h != 0).sum()), "residual_max_sample": resid_max},
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, op, threads=args.cpu_threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
