#!/usr/bin/env python3
"""Throughput benchmark: PCG iterations/s and achieved HBM bandwidth on one MI355X.

One step = one complete solve of the 1024x1024x128 float64 workload (graded
alpha_z, horizontally varying alpha_h, seeded uniform right-hand side) to
||r||/||r0|| < 1e-10 from x0 = 0: coefficient set-up already done at handle
creation, then initial residual, the interleaved PCG iterations and the final
x update.  Inputs are resident in device memory before the timed region.

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).
  python bench.py [--gpus 1] [--steps K] [--warmup W]
Options for profiling helpers:
  --copy-calibration   run only a plain 1 GiB device copy (counter calibration)
  --stream-probe       run only the streaming-bandwidth probe (lib/libmfprobe.so): the GB/s a
                       plain kernel reaches for the solver's read/write stream mixes
                       (--stream-probe-dtype f32: with 4-byte elements, the binary32 passes)
  --no-cpu-baseline    skip timing the CPU oracle
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "PCG iterations/s + achieved HBM GB/s (% roofline), fp64 1024×1024×128"

# Algorithmic bytes per grid point of each launch of a pass (float64 = 8 B;
# each vector read or written once per pass; stencil halos and coefficients
# not counted), as a function of the step k the launch belongs to.
#   interleaved: Algorithms 2-3, x updated every fourth step.
#     fused_prec  k = 0: read r, write z (16); k >= 1: read r, q, write r, z (32)
#     fused_spmv  k = 0: read z, write p, q (24); k mod 4 != 0: read z, p, q,
#                 write p, q (40); k mod 4 == 0, k >= 4: also read x and the
#                 three older directions, write x (80)
#     -> 82 B per point per step in steady state
#   interleaved_no_q: q never stored.
#     fused_prec  k = 0: 16; k >= 1: read r, p, write r, z (32)
#     fused_spmv  k = 0: read z, write p (16); k >= 1: read x, p, z, write x, p (40)
#     -> 72 B per point per step
#   f32: the interleaved loop with every vector in binary32 (4 B): half of
#     the interleaved figures -> 41 B per point per step
#   mixed: binary64 vectors, z in binary32:
#     fused_prec  k = 0: read r, write z (12); k >= 1: read r, q, write r, z (28)
#     fused_spmv  k = 0: read z, write p, q (20); k mod 4 != 0: read z, p, q,
#                 write p, q (36); k mod 4 == 0: also read x and the three
#                 older directions, write x (76)
#     -> 74 B per point per step
def _bytes_interleaved(kernel, k):
    if kernel == "fused_prec":
        return 16 if k == 0 else 32
    return 24 if k == 0 else (80 if k % 4 == 0 else 40)


def _bytes_no_q(kernel, k):
    if kernel == "fused_prec":
        return 16 if k == 0 else 32
    return 16 if k == 0 else 40


def _bytes_f32(kernel, k):
    return _bytes_interleaved(kernel, k) // 2


def _bytes_mixed(kernel, k):
    if kernel == "fused_prec":
        return 12 if k == 0 else 28
    return 20 if k == 0 else (76 if k % 4 == 0 else 36)


BYTES_BY_VARIANT = {"interleaved": (_bytes_interleaved, 82), "interleaved_no_q": (_bytes_no_q, 72),
                    "f32": (_bytes_f32, 41), "mixed": (_bytes_mixed, 74), "mg": (_bytes_interleaved, None)}


# mg: the interleaved loop with one multigrid V-cycle as the preconditioner
# pass; the stencil pass is the interleaved one.  Algorithmic bytes of one
# V(1,1) cycle, per level of n_l points whose coarser level has n_c points
# (0 on the coarsest), each vector read or written once per pass:
#   first sweep   read f (and q: r -= alpha q on level 0, k >= 1), write z
#                 (and r): 16, level 0 at k >= 1: 32
#   restriction   read f, z, write t: 24 per point; write f_c: 8 per coarse point
#   correction    read t, z (and f for the dot products on level 0), write z:
#                 24, level 0: 32; read z_c: 8 per coarse point
# and on the coarsest level: one column, the exact column solve (16);
# several, cs sweeps from z = 0 (coarse_sweeps = cs): the first 16, each
# further one 24 (read f, z, write z: one pass forming the residual from z
# and its neighbours), or 48 where the segments are longer than 8 levels
# (nz > 128), which run it as a residual pass (read f, z, write w) and a
# corrected column solve (read w, z, write z).  Chebyshev-accelerated
# sweeps (chebyshev=True) also read z_{k-1} from the second one on: 32 (56).
def mg_cycle_bytes(level_points, k, nu=1, coarse_sweeps=0, two_pass_sweeps=False, chebyshev=False):
    if nu != 1:
        raise ValueError("the byte model covers V(1,1) cycles")
    tot = 0
    for l, nl in enumerate(level_points):
        nc = level_points[l + 1] if l + 1 < len(level_points) else 0
        if nc == 0:
            per = 48 if two_pass_sweeps else 24
            further = max(coarse_sweeps - 1, 0)
            extra = 8 * max(further - 1, 0) if chebyshev else 0
            tot += (16 + per * further + extra) * nl
            continue
        first = 32 if (l == 0 and k > 0) else 16
        corr = 32 if l == 0 else 24
        tot += (first + 24 + corr) * nl + 16 * nc
    return tot


def step_class(variant, kernel, k):
    """Launches of a pass with the same work per point: the first step, and
    (interleaved stencil pass) the steps that defer the x update ("nox") and
    every fourth one, which applies four ("x4"), else the rest."""
    if k == 0:
        return "first"
    if variant in ("interleaved", "f32", "mixed") and kernel == "fused_spmv":
        return "x4" if k % 4 == 0 else "nox"
    return "rest"


# standard: the non-interleaved loop (one pass per BLAS-1 step, each fused
# with its dot product).  Per step k >= 1: q = A p with <p,q> (read p, write
# q: 16 B), x += alpha p with r -= alpha q and <r,r> (read x, p, r, q, write
# x, r: 48), z = M^-1 r with <r,z> (16), p = z + beta p (read z, p, write p:
# 24): 104 B per point per step; before the loop z = M^-1 r0 (16) and p = z
# (16).  The passes after the last stop test are launched but return at once
# (no bytes).  Totals per timed launch class over solves of K steps:
def standard_bytes(kind, iters, n):
    tot = 0
    for K in iters:
        if kind == "apply_A":
            tot += 16 * K
        elif kind == "precond":
            tot += 16 * K
        elif kind == "vector":
            tot += 16 + 48 * K + 24 * max(K - 1, 0)
    return tot * n


def mg_pass_bytes(level_points, iters, coarse_sweeps=0, two_pass_sweeps=False, period=1, chebyshev=False):
    """Total algorithmic bytes and count of the timed V-cycles (k = 0..K;
    with a profiling period P > 1 only those with k mod P < PROFILE_WINDOW)."""
    tot = cnt = 0
    for K in iters:
        for k in range(K + 1):
            if period > 1 and k % period >= PROFILE_WINDOW:
                continue
            tot += mg_cycle_bytes(level_points, k, coarse_sweeps=coarse_sweeps, two_pass_sweeps=two_pass_sweeps,
                                  chebyshev=chebyshev)
            cnt += 1
    return tot, cnt


def timed_steps(kernel, iters, period=1):
    """Step index k of every timed launch of a pass, over solves of `iters`
    steps each: the preconditioner pass runs at k = 0..K, the stencil pass at
    k = 0..K-1 (its launch at k = K, made before the stop test was read,
    returns at once and is not timed); with a profiling period P > 1 the
    library times only the steps with k mod P < PROFILE_WINDOW."""
    for K in iters:
        ks = range(K + 1) if kernel == "fused_prec" else range(K)
        yield from (k for k in ks if period <= 1 or k % period < PROFILE_WINDOW)


def pass_bytes(variant, kernel, iters, n, period=1):
    """Total algorithmic bytes and launch count of the timed launches of one
    pass over solves that took `iters` steps each (period: as timed_steps)."""
    f = BYTES_BY_VARIANT[variant][0]
    tot = cnt = 0
    for k in timed_steps(kernel, iters, period):
        tot += f(kernel, k) * n
        cnt += 1
    return tot, cnt


# The solve loops' passes are timed with HIP events on PROFILE_WINDOW
# consecutive steps in every PROFILE_PERIOD (the stencil pass's two forms as
# often as in a whole solve): each recorded event delays the next kernel by
# about 5.6 us, which bracketing every pass would add to the timed solves
# (21 ms per solve at 1024 x 1024 x 128).  The window is the library's.
PROFILE_WINDOW = 4
PROFILE_PERIOD = 16

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_fused_passes_varying-1024x1024x128.json")
KERNEL_SOURCE = os.path.join(ROOT, "matrix_free_pcg_amd", "csrc", "kernels.hpp")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest(path=None) -> str:
    """sha256 of the kernel source with // and /* */ comments removed and
    whitespace collapsed: a counter record stays valid across comment edits
    and is dropped once the code changes."""
    import hashlib
    import re
    src = open(path or KERNEL_SOURCE, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()


def measured_traffic(kernel: str, workload: str, variant: str, iters, period=1):
    """HBM bytes per launch of a pass from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE per dispatch, calibrated on a plain copy,
    per step class), averaged over the same launches as the timing; None when
    that summary was taken on different kernel code, variant or workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        digest = kernel_source_digest()
    except OSError:
        return None
    if rec.get("code_digest") != digest or rec.get("variant") != variant or rec.get("workload") != workload:
        return None
    classes = rec.get("passes", {}).get(kernel)
    if not classes:
        return None
    tot = cnt = 0
    for k in timed_steps(kernel, iters, period):
        c = classes.get(step_class(variant, kernel, k))
        if c is None:
            return None
        tot += c["traffic_bytes"]
        cnt += 1
    return int(round(tot / cnt)) if cnt else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5, 6],
                    help="5 = explicit-vs-matrix-free comparison at 2048x2048x128 (50 fixed steps)")
    ap.add_argument("--variant", default="interleaved",
                    choices=["interleaved", "interleaved_no_q", "standard", "f32", "mixed", "mg"],
                    help="f32: every vector in binary32, to tol 1e-5 (the workload's 1e-10 is below "
                         "binary32 rounding); mixed: binary64 with the preconditioner in binary32; "
                         "mg: one multigrid V(1,1) cycle as the preconditioner (--mg-* options)")
    ap.add_argument("--mg-omega", type=float, default=0.9, help="mg: damping of the column smoother")
    ap.add_argument("--mg-levels", type=int, default=5,
                    help="mg: levels of the hierarchy (0: down to one column); 5 ends at 64x64 columns at 1024^2")
    ap.add_argument("--mg-coarse-sweeps", type=int, default=16, help="mg: sweeps on the coarsest level")
    ap.add_argument("--mg-coarse-lo", type=float, default=0.02,
                    help="mg: lower end of the Chebyshev interval [lo, 2] of the coarsest sweeps (0: damped sweeps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=3)
    ap.add_argument("--cpu-steps-cfg5", type=int, default=1,
                    help="--config 5: CG steps of the oracle's CPU baseline at 2048x2048x128")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--stream-probe", action="store_true")
    ap.add_argument("--stream-probe-dtype", choices=["f64", "f32"], default="f64",
                    help="element of the probe's vectors: f64 (8-byte accesses, the binary64 passes) or "
                         "f32 (4-byte, the binary32 passes); 1 GiB vectors either way")
    ap.add_argument("--counter-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the HBM counter record of the fused passes from four rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE of a --fixed-iterations solve; the same of --copy-calibration)")
    ap.add_argument("--counter-steps", type=int, default=10, help="--counter-summary: the solve's fixed steps")
    ap.add_argument("--counter-commands", default="", help="--counter-summary: the commands, ';'-separated")
    ap.add_argument("--counter-out", default=None, help="--counter-summary: directory to write to (default profiles/)")
    ap.add_argument("--fixed-iterations", type=int, default=0,
                    help="run exactly N CG steps per solve (tol 0) instead of solving to 1e-10")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB (read 1 GiB, write 1 GiB),
    for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 27
    a = torch.ones(n, dtype=torch.float64, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    t = time.perf_counter()
    reps = 20
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t) / reps
    print(json.dumps({"copy_bytes_read": n * 8, "copy_bytes_written": n * 8,
                      "copy_ms": dt * 1e3, "copy_GBps": 2 * n * 8 / dt / 1e9}), flush=True)


def _counter_rows(run_dir):
    """(dispatch id, kernel name, counter name, value) of every row of the
    rocprofv3 counter-collection CSV files under run_dir."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    return rows


def _per_dispatch(rows, counter):
    """{dispatch id: (kernel name, summed counter value)} in dispatch order."""
    out = {}
    for d, k, c, v in rows:
        if c == counter:
            name, tot = out.get(d, (k, 0.0))
            out[d] = (name, tot + v)
    return dict(sorted(out.items()))


def _short_kernel(name):
    """`k_stencil<4, 8, true, double, double, 4>` from a demangled kernel name."""
    base = name.split("(")[0].replace("void ", "").replace("mfpcg::", "")
    return base.strip()


def counter_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, steps, commands, out_dir=None):
    """Write the HBM counter record of the binary64 fused passes (the JSON the
    roofline's `traffic` reads, and its Markdown summary) from four rocprofv3
    runs: FETCH_SIZE and WRITE_SIZE of a solve of `steps` fixed steps of
    varying-1024x1024x128 (bench.py --steps 1 --warmup 0 --fixed-iterations
    steps), and of the 1 GiB copy (bench.py --copy-calibration)."""
    import hashlib
    n = 1024 * 1024 * 128
    copy_bytes = 1 << 30
    cf = [v for _, (k, v) in _per_dispatch(_counter_rows(copy_fetch_dir), "FETCH_SIZE").items() if "copyBuffer" in k]
    cw = [v for _, (k, v) in _per_dispatch(_counter_rows(copy_write_dir), "WRITE_SIZE").items() if "copyBuffer" in k]
    if not cf or not cw:
        raise SystemExit("no copy dispatch in the calibration runs")
    f_kib, w_kib = sorted(cf)[len(cf) // 2], sorted(cw)[len(cw) // 2]     # the median dispatch
    fetch_scale, write_scale = copy_bytes / (f_kib * 1024), copy_bytes / (w_kib * 1024)
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")

    def classify(fetch_or_write):
        """Dispatch values of the two passes by step class, in launch order."""
        prec, spmv = [], []
        for _, (k, v) in fetch_or_write.items():
            short = _short_kernel(k)
            if short.startswith("k_column_full<16, 1, true, double, double, 0>"):
                prec.append((short, v))
            elif short.startswith("k_stencil<") and short.split(",")[1].strip() in ("0", "7", "9"):
                spmv.append((short, v))
        if len(prec) != steps + 1 or len(spmv) != steps + 1:
            raise SystemExit(f"expected {steps + 1} launches of each pass, found {len(prec)} and {len(spmv)}")
        spmv = spmv[:-1]   # the last stencil launch returns at once (the stop test had passed)
        out = {"fused_prec": {"first": [prec[0]], "rest": prec[1:]}, "fused_spmv": {"first": [], "nox": [], "x4": []}}
        for kk, e in enumerate(spmv):
            out["fused_spmv"][step_class("interleaved", "fused_spmv", kk)].append(e)
        return out

    cf_, cw_ = classify(fetch), classify(write)
    alg = {("fused_prec", "first"): 16, ("fused_prec", "rest"): 32, ("fused_spmv", "first"): 24,
           ("fused_spmv", "nox"): 40, ("fused_spmv", "x4"): 80}
    passes = {}
    lines = []
    for kern in ("fused_prec", "fused_spmv"):
        passes[kern] = {}
        for cls, fl in cf_[kern].items():
            wl = cw_[kern][cls]
            rb = sum(v for _, v in fl) / len(fl) * 1024 * fetch_scale
            wb = sum(v for _, v in wl) / len(wl) * 1024 * write_scale
            passes[kern][cls] = {"kernel": fl[0][0], "dispatches": len(fl), "read_bytes": rb, "write_bytes": wb,
                                 "traffic_bytes": rb + wb, "algorithmic_bytes": alg[(kern, cls)] * n}
            lines.append(f"| {kern} | {cls} | `{fl[0][0]}` | {len(fl)} | {rb / n:.2f} | {wb / n:.2f} | "
                         f"{(rb + wb) / 1e9:.3f} | {alg[(kern, cls)] * n / 1e9:.3f} |")
    src = KERNEL_SOURCE
    rec = {"variant": "interleaved", "source": "matrix_free_pcg_amd/csrc/kernels.hpp",
           "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "code_digest": kernel_source_digest(),
           "code_digest_note": "sha256 of kernels.hpp with comments removed and whitespace collapsed "
                               "(bench.kernel_source_digest)",
           "workload": "varying-1024x1024x128", "steps_profiled": steps,
           "calibration": {"copy_bytes": copy_bytes, "FETCH_SIZE_KiB_per_dispatch": f_kib,
                           "WRITE_SIZE_KiB_per_dispatch": w_kib, "fetch_scale": fetch_scale,
                           "write_scale": write_scale},
           "passes": passes}
    out_json = TRAFFIC_FILE if out_dir is None else os.path.join(out_dir, os.path.basename(TRAFFIC_FILE))
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    md = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "hbm_counters_fused_passes_varying-1024x1024x128.md")
    with open(md, "w") as f:
        f.write("# HBM traffic of the fused passes, varying-1024x1024x128 (fp64), variant `interleaved`\n\n")
        f.write("Commands (from /tmp, TMPDIR=/tmp; one counter per run), then the summary written by the last one:\n\n```\n")
        f.write("\n".join(commands) + "\n```\n\n")
        f.write(f"Calibration: a plain 1 GiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = {f_kib:.1f} KiB "
                f"and WRITE_SIZE = {w_kib:.1f} KiB per dispatch for 1048576 KiB moved each way, so read counts are "
                f"scaled by {fetch_scale:.4f} and write counts by {write_scale:.4f}.\n\n")
        f.write(f"Kernel source: `matrix_free_pcg_amd/csrc/kernels.hpp`, sha256 `{rec['source_sha256']}`.\n\n")
        f.write(f"A {steps}-step solve; dispatches grouped by the step class they belong to (the stencil pass "
                "defers the x update on three steps, `nox`, and applies the four pending terms on every fourth, "
                "`x4`). The stencil launch after the last step, which returns at once, is left out.\n\n")
        f.write("| pass | step class | kernel | dispatches | read B/point | write B/point | traffic GB per launch | "
                "algorithmic GB per launch |\n|---|---|---|---:|---:|---:|---:|---:|\n")
        f.write("\n".join(lines) + "\n\nN = 134217728 points.  Reads above the algorithmic count: in the stencil "
                "pass the i-halo lines at the edges of each XCD's strip of tiles (and a few j / k halo lines that "
                "miss L2); in the preconditioner pass the per-column Thomas multipliers at the boundaries of its "
                "16-level segments and the per-column coefficient tables (area and the two edge fields).\n")
    print(json.dumps({"written": [out_json, md]}), flush=True)


# (reads, writes, pass it stands for)
PROBE_MIXES = [(1, 1, "copy"), (2, 1, "residual r = b - A x"), (2, 2, "column pass (r, q -> r, z)"),
               (3, 2, "stencil pass deferring x (z, p, q -> p, q)"),
               (7, 3, "stencil pass of every fourth step (z, p, q, x and three older p -> p, q, x)")]


def stream_probe(dtype="f64", vector_bytes=1 << 30, reps=20):
    """GB/s of a plain streaming kernel (every element read / written once,
    loads batched before stores) for each stream mix of the solver's passes,
    with non-temporal and with ordinary loads and stores, on vectors of
    float64 or float32 elements (`dtype`, 1 GiB each at the default): the best over 1, 2, 4 or 8 elements per
    thread and 256- or 1024-thread workgroups.  The solver's passes add what a
    stream kernel does not have (neighbour reads, the column recurrences), so
    these rates are the measured ceiling for each mix, beside the published
    peak."""
    import ctypes
    import torch
    from matrix_free_pcg_amd import build as hipbuild
    if not os.path.exists(hipbuild.PROBE_LIB):
        raise SystemExit(f"{hipbuild.PROBE_LIB} is not built (python -m matrix_free_pcg_amd.build)")
    lib = ctypes.CDLL(hipbuild.PROBE_LIB)
    fn = lib.mfprobe_stream_f32 if dtype == "f32" else lib.mfprobe_stream
    esize = 4 if dtype == "f32" else 8
    n = vector_bytes // esize
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int64,
                                   ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]
    tdt = torch.float32 if dtype == "f32" else torch.float64
    vec = [torch.full((n,), 1.0 + k, dtype=tdt, device="cuda") for k in range(10)]
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for r, w, what in PROBE_MIXES:
        ins = (ctypes.c_void_p * r)(*[vec[k].data_ptr() for k in range(r)])
        outs = (ctypes.c_void_p * w)(*[vec[7 + k].data_ptr() for k in range(w)])
        row = {"reads": r, "writes": w, "stands_for": what}
        for nt in (1, 0):
            best = None
            for elems in (1, 2, 4, 8):
                for block in (256, 1024):
                    ms = ctypes.c_double(0.0)
                    rc = fn(r, w, nt, elems, block, n, ins, outs, reps, stream, ctypes.byref(ms))
                    if rc != 0:
                        raise SystemExit(f"mfprobe_stream[{dtype}]({r}, {w}, nt={nt}, {elems}, {block}) returned {rc}")
                    gbps = (r + w) * n * esize / (ms.value * 1e-3) / 1e9
                    if best is None or gbps > best[0]:
                        best = (gbps, elems, block)
            key = "nontemporal" if nt else "ordinary"
            row[key + "_GBps"] = round(best[0], 1)
            row[key + "_shape"] = f"{best[1]} elements x {best[2]} threads"
        out.append(row)
        print(json.dumps(row), flush=True)
    torch.cuda.synchronize()
    print(json.dumps({"stream_probe": out, "dtype": dtype, "vector_bytes": n * esize, "reps": reps}), flush=True)


def cpu_baseline(w, steps, variant="interleaved", mg_params=None):
    """The CPU oracle (single thread) on a bounded sample of the same workload:
    `steps` CG steps of the full problem, timed around the oracle's step loop
    (its set-up pass r0 = b - A x0, z0 = M^-1 r0 is not counted)."""
    import oracle
    from matrix_free_pcg_amd.workloads import GeneralProblem
    cpu = _host_cpu()
    # one core, as the pages' single-core CPU figures (affinity of this
    # process only, restored afterwards)
    old_aff = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if old_aff:
        os.sched_setaffinity(0, {min(old_aff)})
    # the manufactured workload: the oracle forms its own b = A x_true
    rhs = w.rhs if w.rhs is not None else oracle.apply_A(w.problem, w.x_true)
    t0 = time.perf_counter()
    if variant == "mg":
        gp = w.problem if isinstance(w.problem, GeneralProblem) else _as_general(w.problem)
        res = oracle.pcg_mg(gp, rhs, tol=0.0, maxit=steps, **(mg_params or {}))
        total = time.perf_counter() - t0
        per = total / (res["iters"] + 1)
        how = "multigrid PCG, timed around the whole call, its set-up pass counted as one more step"
    elif isinstance(w.problem, GeneralProblem):
        res = oracle.pcg_gen(w.problem, rhs, tol=0.0, maxit=steps)
        total = time.perf_counter() - t0
        per = total / (res["iters"] + 1)
        how = "timed around the whole call, its set-up pass counted as one more step"
    else:
        # one step more than timed: the last step of a call skips its
        # preconditioner application, so only the complete steps before it count
        res = oracle.pcg(w.problem, rhs, tol=0.0, maxit=steps + 1)
        total = time.perf_counter() - t0
        per = res["full_steps_seconds"] / max(1, res["full_steps"])
        how = (f"timed over its first {res['full_steps']} complete step(s) (stencil, preconditioner, "
               f"dots, updates; the call ran one more)")
    if old_aff:
        os.sched_setaffinity(0, old_aff)
    return {"value": round(1.0 / per, 4), "unit": "iterations/s", "cores": 1, "kind": "oracle",
            "sample": f"{res['iters']} CG steps of the {w.name} workload (single-threaded C, "
                      f"-O2, pinned to one core), {how}; {total:.1f} s of CPU time in all",
            "s_per_iteration": round(per, 3), "host_cpu": cpu["model"], "host_nproc": cpu["nproc"]}


def _host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count()}


def _as_general(prob):
    """The special operator in general form (|T| = 1, a = delta, d = 1, beta =
    alpha_z, edges the mean of the two cells' alpha_h), for the oracle."""
    import numpy as np
    from matrix_free_pcg_amd.workloads import GeneralProblem
    ah = prob.alpha_h_field()
    ax = 0.5 * (ah + np.roll(ah, -1, axis=1))
    ay = 0.5 * (ah + np.roll(ah, -1, axis=0))
    return GeneralProblem(prob.nx, prob.ny, prob.nz, np.full(prob.nz, prob.delta), np.ones(prob.nz),
                          np.asarray(prob.alpha_z_face, dtype=np.float64), np.ones((prob.ny, prob.nx)), ax, ay)


CSR_BYTES_PER_ROW = 108   # 7 x (8 B value + 4 B column) + row pointer + x + y (8 B each)


def explicit_comparison(args):
    """2048x2048x128: 50 fixed CG steps matrix-free (interleaved) and explicit
    (CSR matrix + stored column matrices, standard loop), and the isolated
    operator application both ways.  One JSON line."""
    import torch
    import matrix_free_pcg_amd as mf
    from matrix_free_pcg_amd import workloads as W
    dev = torch.device("cuda:0")
    t = time.perf_counter()
    w = W.make_workload(5)
    prob = w.problem
    n = prob.n
    log(f"[bench] {w.name}: inputs generated in {time.perf_counter() - t:.1f}s")
    b = torch.from_numpy(w.rhs).to(dev)
    x = torch.zeros_like(b)
    h = mf.pcg_create(prob, torch.cuda.current_stream())
    t = time.perf_counter()
    C = mf.pcg_csr_assemble(h)
    tri = mf.pcg_tridiag_assemble(h)
    torch.cuda.synchronize()
    t_asm = time.perf_counter() - t
    ws = torch.empty(mf.pcg_solve_workspace_bytes(h, w.maxit), dtype=torch.uint8, device=dev)
    out = {"workload": w.name, "steps": w.maxit, "nnz": C.col.numel(), "csr_assembly_s": round(t_asm, 3)}
    for name, fn in (("matrix_free", lambda: mf.pcg_solve(h, b, x, 0.0, w.maxit, ws)),
                     ("explicit", lambda: mf.pcg_solve_csr(h, C, tri, b, x, 0.0, w.maxit, ws))):
        x.zero_()
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            x.zero_()
            res = fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        out[name] = {"s_per_solve": round(dt, 4), "iterations_per_s": round(w.maxit / dt, 2),
                     "final_rel_res": res["final_rel_res"]}
    y = torch.empty_like(b)
    mf.pcg_profile_reset(h)
    mf.pcg_profile_enable(h, True)
    for _ in range(10):
        mf.pcg_apply_A(h, b, y)
        mf.pcg_csr_spmv(h, C, b, y)
    ms_mf, n_mf = mf.pcg_profile_read(h, mf.PCG_KID_APPLY_A)
    ms_csr, n_csr = mf.pcg_profile_read(h, mf.PCG_KID_CSR_SPMV)
    mf.pcg_profile_enable(h, False)
    a_mf, a_csr = ms_mf / n_mf, ms_csr / n_csr
    out["spmv"] = {"matrix_free_ms": round(a_mf, 4), "matrix_free_GBps": round(16 * n / a_mf / 1e6, 1),
                   "csr_ms": round(a_csr, 4), "csr_GBps": round(CSR_BYTES_PER_ROW * n / a_csr / 1e6, 1),
                   "speedup_matrix_free": round(a_csr / a_mf, 2)}
    mf.pcg_destroy(h)
    del C, tri, ws, b, x, y
    if not args.no_cpu_baseline:
        # the oracle on one CG step of the same 2048x2048x128 problem (its
        # 50-step solve takes about 20 minutes on one core)
        t = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_steps_cfg5)
        out["cpu_baseline"]["matrix_free_speedup_vs_oracle"] = round(
            out["matrix_free"]["iterations_per_s"] / out["cpu_baseline"]["value"], 1)
        log(f"[bench] cpu baseline in {time.perf_counter() - t:.1f}s")
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU path is a design, not a build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.counter_summary:
        counter_summary(*args.counter_summary, steps=args.counter_steps,
                        commands=[c.strip() for c in args.counter_commands.split(";") if c.strip()],
                        out_dir=args.counter_out)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stream_probe:
        stream_probe(args.stream_probe_dtype)
        return

    if args.config == 5:
        explicit_comparison(args)
        return

    import matrix_free_pcg_amd as mf
    from matrix_free_pcg_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = time.perf_counter()
    w = W.make_workload(args.config)
    prob = w.problem
    if w.rhs is None and w.x_true is None:
        raise SystemExit("the workload has neither a right-hand side nor a solution")
    log(f"[bench] {w.name}: inputs generated in {time.perf_counter() - t:.1f}s")
    n = prob.n
    vdtype = np.float32 if args.variant == "f32" else np.float64
    # outside the timed region, listed separately: host-to-device copy of b
    # and the set-up (handle: coefficient tables and Thomas multipliers)
    torch.cuda.synchronize()
    t = time.perf_counter()
    # the manufactured workload copies its solution and forms b = A x_true on
    # the device with the library's operator, before the timed region
    host_in = torch.from_numpy(w.rhs.astype(vdtype) if w.rhs is not None else w.x_true).to(dev)
    torch.cuda.synchronize()
    t_h2d = time.perf_counter() - t
    stream = torch.cuda.current_stream()
    t = time.perf_counter()
    h = mf.pcg_create(prob, stream)
    if w.rhs is None:
        b = torch.empty_like(host_in)
        mf.pcg_apply_A(h, host_in, b)
        if vdtype is np.float32:
            b = b.to(torch.float32)
        del host_in
    else:
        b = host_in
    x = torch.zeros_like(b)
    tol, maxit = (1e-5 if args.variant == "f32" else w.tol), w.maxit
    if args.fixed_iterations > 0:
        tol, maxit = 0.0, args.fixed_iterations
    level_points = None
    mg_params = None
    if args.variant == "mg":
        mg_params = dict(nu=1, omega=args.mg_omega, max_levels=args.mg_levels, coarse_sweeps=args.mg_coarse_sweeps,
                         coarse_lo=args.mg_coarse_lo)
        mf.pcg_mg_setup(h, **mg_params)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t
    overrides = mf.pcg_tuning_overrides(h)   # MFPCG_* launch-shape variables set at creation (0: none)
    if args.variant == "mg":
        level_points = [mf.pcg_mg_level(h, l)[0] * mf.pcg_mg_level(h, l)[1] * prob.nz
                        for l in range(mf.pcg_mg_num_levels(h))]
        # sweeps on the coarsest level (0: one column, solved exactly)
        mg_cs = 0 if level_points[-1] == prob.nz else mg_params["coarse_sweeps"]
        mg_two = prob.nz > 128   # segments longer than 8 levels: two-pass sweeps
        mg_cheb = mg_params["coarse_lo"] > 0.0
        ws = torch.empty(mf.pcg_mg_workspace_bytes(h, maxit), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(mf.pcg_solve_workspace_bytes(h, maxit), dtype=torch.uint8, device=dev)
    solve = {"interleaved": mf.pcg_solve, "interleaved_no_q": mf.pcg_solve_no_q,
             "standard": mf.pcg_solve_standard, "f32": mf.pcg_solve_f32,
             "mixed": mf.pcg_solve_mixed, "mg": mf.pcg_solve_mg}[args.variant]
    has_bytes = args.variant in BYTES_BY_VARIANT
    torch.cuda.synchronize()

    for s in range(args.warmup):
        x.zero_()
        res = solve(h, b, x, tol, maxit, ws)
        log(f"[bench] warmup {s}: iters={res['iters']} status={res['status']}")

    mf.pcg_profile_reset(h)
    mf.pcg_profile_enable(h, PROFILE_PERIOD)
    iters = []
    solve_s = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ts = time.perf_counter()
        x.zero_()
        res = solve(h, b, x, tol, maxit, ws)   # returns after the solve has finished
        solve_s.append(time.perf_counter() - ts)
        iters.append(res["iters"])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mf.pcg_profile_enable(h, False)
    total_iters = int(sum(iters))
    log(f"[bench] timed: {args.steps} solves, {total_iters} iterations in {elapsed:.3f}s")

    kern = {}
    names = {"fused_prec": mf.PCG_KID_FUSED_PREC, "fused_spmv": mf.PCG_KID_FUSED_SPMV,
             "apply_A": mf.PCG_KID_APPLY_A, "precond": mf.PCG_KID_PRECOND, "vector": mf.PCG_KID_VECTOR,
             "mg_vcycle": mf.PCG_KID_MG_VCYCLE}
    for name, kid in names.items():
        ms, cnt = mf.pcg_profile_read(h, kid)
        if cnt:
            avg = ms / cnt
            ent = {"launches": cnt, "avg_ms": avg, "total_ms": ms}
            if name == "mg_vcycle":
                tot, nl = mg_pass_bytes(level_points, iters, mg_cs, mg_two, PROFILE_PERIOD, mg_cheb)
                if nl != cnt:
                    raise SystemExit(f"{name}: {cnt} timed cycles, expected {nl}")
                ent["bytes_per_launch"] = tot / nl
                ent["GBps"] = tot / (ms * 1e-3) / 1e9
                ent["note"] = f"one V(1,1) cycle over {len(level_points)} levels: every kernel of the cycle"
            elif args.variant == "standard" and name in ("apply_A", "precond", "vector"):
                tot = standard_bytes(name, iters, n)
                ent["bytes_total"] = tot
                ent["GBps"] = tot / (ms * 1e-3) / 1e9
                ent["note"] = "algorithmic bytes of all timed launches / their total time"
            elif has_bytes and name in ("fused_prec", "fused_spmv"):
                tot, nl = pass_bytes(args.variant, name, iters, n, PROFILE_PERIOD)
                if nl != cnt:
                    raise SystemExit(f"{name}: {cnt} timed launches, expected {nl}")
                ent["bytes_per_launch"] = tot / nl          # average over the timed launches
                ent["GBps"] = tot / (ms * 1e-3) / 1e9
            kern[name] = ent

    # true residual of the last solve, with the library's own stencil
    xb, bb = x.double(), b.double()
    r = torch.empty_like(bb)
    mf.pcg_apply_A(h, xb, r)
    torch.cuda.synchronize()
    true_rel = float(torch.linalg.vector_norm(bb - r) / torch.linalg.vector_norm(bb))
    mf.pcg_destroy(h)

    it_s = total_iters / elapsed
    # every timed pass's algorithmic bytes over the whole timed region
    if args.variant == "mg":
        all_bytes = (pass_bytes(args.variant, "fused_spmv", iters, n)[0]
                     + mg_pass_bytes(level_points, iters, mg_cs, mg_two, chebyshev=mg_cheb)[0])
    elif args.variant == "standard":
        all_bytes = sum(standard_bytes(kind, iters, n) for kind in ("apply_A", "precond", "vector"))
    else:
        all_bytes = (sum(pass_bytes(args.variant, kname, iters, n)[0] for kname in ("fused_prec", "fused_spmv"))
                     if has_bytes else None)
    dom = max((k for k in kern if "GBps" in kern[k]), key=lambda k: kern[k]["total_ms"], default=None)
    roofline = None
    if dom is not None and "bytes_per_launch" not in kern[dom]:
        # standard loop: totals per launch class
        ach = kern[dom]["GBps"]
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "traffic_unit": "bytes per launch",
                    "kernel": dom, "avg_launch_ms": round(kern[dom]["avg_ms"], 4)}
    elif dom is not None:
        ach = kern[dom]["GBps"]
        traffic = measured_traffic(dom, w.name, args.variant, iters, PROFILE_PERIOD)
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": traffic,
                    "traffic_unit": "bytes per launch", "kernel": dom,
                    "bytes_per_launch": round(kern[dom]["bytes_per_launch"]),
                    "avg_launch_ms": round(kern[dom]["avg_ms"], 4)}
        if traffic is not None:
            # counter-measured bytes (calibrated HBM read + write) over this run's launch time
            cg = traffic / (kern[dom]["avg_ms"] * 1e-3) / 1e9
            roofline["traffic_GBps"] = round(cg, 1)
            roofline["traffic_frac"] = round(cg / HBM_PEAK_GBS, 4)

    out = {
        "metric": METRIC,
        "value": round(it_s, 2),
        "unit": "iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "mixed": "f64 (preconditioner f32)"}.get(args.variant, "f64"),
        "s_per_solve": round(elapsed / args.steps, 4),
        "median_s_per_solve": round(float(np.median(solve_s)), 4),
        "setup_s": round(t_setup, 4),
        "h2d_s": round(t_h2d, 4),
        "data": "synthetic",
        "config": {"workload": w.name, "nx": prob.nx, "ny": prob.ny, "nz": prob.nz,
                   "tol": tol, "maxit": maxit, "variant": args.variant,
                   "iterations_per_solve": iters, "status": res["status"],
                   "final_rel_res": res["final_rel_res"], "true_rel_res": true_rel,
                   "tuning_overrides": overrides,
                   **({"mg": mg_params} if mg_params else {})},
        # algorithmic bytes of both passes over the whole timed region / its wall time
        "hbm_GBps_whole_solve": round(all_bytes / elapsed / 1e9, 1) if all_bytes else None,
        "hbm_frac_whole_solve": round(all_bytes / elapsed / 1e9 / HBM_PEAK_GBS, 4) if all_bytes else None,
        "bytes_per_point_per_iteration": (104 if args.variant == "standard" else
                                          (BYTES_BY_VARIANT[args.variant][1] if args.variant != "mg"
                                           else round(50 + mg_cycle_bytes(level_points, 1, coarse_sweeps=mg_cs,
                                                                          two_pass_sweeps=mg_two,
                                                                          chebyshev=mg_cheb) / n, 2))
                                          if has_bytes else None),
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        t = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w, 1 if args.variant == "mg" else args.cpu_steps, args.variant,
                                           mg_params)
        log(f"[bench] cpu baseline in {time.perf_counter() - t:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
