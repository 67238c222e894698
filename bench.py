"""Benchmark of the decode-time quantized mat-vec on one MI355X.

Default workload: Q4_K weights, M = 4096 rows x K = 14336, n = 1 activation
column (the FFN down-projection shape of a 7B/8B-class model), fp32 output.
One step is one pass of the hot path over one activation: quantize the fp32
activation to q8_1, then the quantized mat-vec against a weight matrix. The
step runs as one fused launch (mmvq_f32: the row kernel quantizes its slice
of the activation in its prologue, the many-column kernel each block it
stages) unless ``--step two`` asks for the two
launches (mmvq_quantize_q8_1, then mmvq); both forms are timed and reported.

Measurement:
  * inputs (weights, activation) are resident in HBM before timing starts;
  * weights rotate over enough copies (>= 3 x the 256 MB last-level cache)
    that every step streams its matrix from HBM, not from cache;
  * exactly --steps launches are captured in one HIP graph (launch i uses
    weight copy i mod copies) and replayed once after a graph of --warmup
    untimed launches, so host launch cost does not pace microsecond kernels;
  * HIP events on the launch stream time each form: the fused step, the
    two-launch step, the mat-vec alone, the quantizer alone, and a
    streaming-read probe (mmvq_read_probe) over the same weight bytes, the
    read ceiling the kernels are compared with;
  * the CPU oracle (plain C, fp64) runs the same workload for a bounded
    time, rows split over every host core and then on one thread, as a
    reported baseline.

Prints one JSON line (rank 0). ``--all`` also prints one line per workload
and column count to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "quantized_decode_gemv_quantize_amd", "csrc")
LLC_BYTES = 256 * 2 ** 20    # MI355X Infinity Cache
TOKENS_DENOM_GB = 3.9        # weight bytes of one decode step of a 7B Q4_K model


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="q4_k_4096x14336")
    p.add_argument("--n", type=int, default=1, help="activation columns")
    p.add_argument("--step", choices=("fused", "two"), default="fused",
                   help="one fused launch per step, or quantize + mat-vec launches")
    p.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="wall-clock budget of the oracle baseline (0 disables it)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain device copy of known size (counter calibration)")
    p.add_argument("--moe", action="store_true",
                   help="time only the expert-indexed gate/up workload (one JSON line) and exit")
    p.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="write the headline profiles/ summaries from rocprofv3 csv output and exit")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="write profiles/<workload>_n<n>_kernel_trace.md for --workload/--n (or --moe) "
                        "from a rocprofv3 --kernel-trace --stats run of the same arguments, and exit")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/<workload>_n<n>_hbm_traffic.md for --workload/--n from two "
                        "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) with --copy-probe, and exit")
    p.add_argument("--summarize-sq", metavar="SQ_DIR",
                   help="write profiles/<workload>_n<n>_sq_counters.md for --workload/--n from a "
                        "rocprofv3 --pmc run of the SQ counters below, and exit")
    return p.parse_args()


# What the measured Q4_K mat-vec kernels (q8_1 and fp32 activations) are
# built from: their translation units, the headers they include and the
# compile flags.
HEADLINE_SOURCES = ["common.hpp", "q8.hpp", "formats.hpp", "plan.hpp", "mmvq_kernel.hpp", "launch.hpp",
                    "kernels_q4_k.hip", "kernels_q4_k_f32.hip", os.path.join("..", "..", "include", "mmvq.h")]
# ... and of every measured kernel, for the per-configuration summaries
ALL_SOURCES = HEADLINE_SOURCES + ["mmq_plan.hpp", "mmq_kernel.hpp", "mmq_launch.hpp", "kernels_mmq.hip",
                                  "kernels_mmq_f32.hip", "kernels_q4_0.hip",
                                  "kernels_q4_0_f32.hip", "kernels_q8_0.hip", "kernels_q8_0_f32.hip",
                                  "kernels_q6_k.hip", "kernels_q6_k_f32.hip", "kernels_q4_k_id.hip",
                                  "kernels_q4_k_f32_id.hip", "kernels_q4_1.hip", "kernels_q4_1_f32.hip",
                                  "kernels_q5_0.hip", "kernels_q5_0_f32.hip", "kernels_q5_1.hip",
                                  "kernels_q5_1_f32.hip", "kernels_q5_k.hip", "kernels_q5_k_f32.hip",
                                  "quantize.hip", "probe.hip", "api.hip"]


def kernel_source_hash(names=None) -> str:
    """sha256 over the sources and compile flags of the measured kernels:
    counters taken on one build are reported only while these are unchanged."""
    import hashlib
    from quantized_decode_gemv_quantize_amd import build as qbuild
    h = hashlib.sha256()
    for name in names or HEADLINE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(os.path.basename(name).encode() + b"\0" + f.read())
    h.update(" ".join(qbuild.HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def _targs(name: str) -> list:
    return name.split("<", 1)[1].split(">", 1)[0].split(", ")


def kernel_form(name: str, grid_y: int = 1, n_experts: int = 0) -> str | None:
    """Which benchmark form a kernel launch belongs to: 'fused' (fp32-activation
    mat-vec), 'gemv' (q8_1 mat-vec: row or many-column kernel), 'quantize',
    'probe' (streaming read), 'id' / 'id_fused' (expert-indexed, q8_1 / fp32
    activations), 'id_shared' (expert-indexed with the shared-expert slice),
    else None."""
    if name.startswith("void qmv::mmvq_rows_kernel<"):
        return "fused" if _targs(name)[5] == "true" else "gemv"      # <F, NC, R, P, G, XF, ...>
    if name.startswith("void qmv::mmvq_rows1_kernel<"):
        return "fused" if _targs(name)[3] == "true" else "gemv"      # <F, R, DEPTH, XF, TW>
    if name.startswith("void qmv::mmq_kernel<"):
        return "fused" if _targs(name)[5] == "true" else "gemv"      # <F, RT, CT, NW, G, XF>
    if name.startswith("qmv::quantize_q8_1_kernel"):
        return "quantize"
    if name.startswith("qmv::read_probe_kernel"):
        return "probe"
    if name.startswith("void qmv::mmvq_id_kernel<"):
        if n_experts and grid_y == n_experts + 1:
            return "id_shared"
        return "id_fused" if _targs(name)[4] == "true" else "id"    # <F, RB, P, G, XF, ...>
    return None


COPY_BYTES = 256 * 2 ** 20     # the --copy-probe copy: reads and writes this many bytes

# SQ counters of one --pmc pass (at most 8 SQ counters per pass)
SQ_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS",
               "SQ_INSTS_MFMA", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"]
# Issue ceiling of plain (non-packed) vector instructions: a wave64
# instruction occupies a 16-lane SIMD for 4 cycles; 256 CUs x 4 SIMDs at
# 2.4 GHz issue 256 * 4 * 2.4e9 / 4 = 614.4 G wave-instructions per second.
VALU_ISSUE_PEAK = 256 * 4 * 2.4e9 / 4


def _csv_rows(d: str, pat: str) -> list:
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", pat), recursive=True)
    if not f:
        raise FileNotFoundError(f"no {pat} under {d}")
    return list(csv.DictReader(open(f[0])))


def profile_name(workload: str, n: int, moe: bool) -> str:
    return "moe_q4_k_8x14336x4096" if moe else f"{workload}_n{n}"


def summarize_trace(trace_dir: str, workload: str, n: int, moe: bool, steps: int, warmup: int) -> None:
    """profiles/<workload>_n<n>_kernel_trace.md: the rocprofv3 --stats table
    and the average duration of each benchmark form, from a kernel-trace run
    of bench.py with the same arguments."""
    import statistics
    stats = _csv_rows(trace_dir, "*kernel_stats.csv")
    trace = _csv_rows(trace_dir, "*kernel_trace.csv")
    E = 8 if moe else 0
    dur = {}
    for r in trace:
        k = kernel_form(r["Kernel_Name"], int(r.get("Grid_Size_Y", 1) or 1), E)
        if k:
            dur.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    name = profile_name(workload, n, moe)
    args = "--moe" if moe else f"--workload {workload} --n {n} --steps {steps} --warmup {warmup}"
    cmd = (f"cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace_{name} -o bench "
           f"-- python3 <repo>/bench.py --cpu-seconds 0 {args}")
    forms = {k: {"launches": len(v), "avg_us": round(statistics.mean(v) / 1e3, 3),
                 "median_us": round(statistics.median(v) / 1e3, 3)} for k, v in sorted(dur.items())}
    labels = {"fused": "fused quantize + mat-vec (fp32 activation)", "gemv": "mat-vec (q8_1 activation)",
              "quantize": "q8_1 quantizer", "probe": "streaming-read probe over the same weight bytes",
              "id": "expert-indexed gate/up (q8_1 activation)",
              "id_fused": "expert-indexed gate/up (fp32 activation)",
              "id_shared": "expert-indexed gate/up, scales, bias rows and a shared expert"}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{name}_kernel_trace.md"), "w") as f:
        f.write(f"# Kernel trace: {name.replace('_n', ', n=')}\n\n")
        f.write(f"Command (MI355X, one GPU):\n\n    {cmd}\n\n")
        f.write("rocprofv3 --stats summary (durations in ns):\n\n")
        f.write("| kernel | calls | avg ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| {r['Name'][:100]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                    f"{r['MinNs']} | {r['MaxNs']} |\n")
        f.write("\nPer form (from the trace):\n\n")
        for k, g in forms.items():
            f.write(f"- {labels.get(k, k)}: {g['launches']} launches, average {g['avg_us']} us, "
                    f"median {g['median_us']} us\n")
        f.write("\n```json\n" + json.dumps({"profile": name, "source_sha256_16": kernel_source_hash(ALL_SOURCES),
                                            "forms": forms}, indent=1) + "\n```\n")
    print(json.dumps({"profile": name, "forms": forms}))


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str, n: int) -> None:
    """profiles/<workload>_n<n>_hbm_traffic.md: HBM bytes per launch of each
    benchmark form (median FETCH_SIZE and WRITE_SIZE over dispatches, scaled
    by what the counters read for the 256 MiB calibration copy), against the
    form's algorithmic bytes."""
    import statistics
    from quantized_decode_gemv_quantize_amd import synth
    wl = synth.BY_NAME[workload]

    def big_copy(d):
        return max(float(r["Counter_Value"]) for r in _csv_rows(d, "*counter_collection.csv")
                   if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"))

    def med(d, kind):
        v = [float(r["Counter_Value"]) for r in _csv_rows(d, "*counter_collection.csv")
             if kernel_form(r["Kernel_Name"]) == kind]
        return (statistics.median(v), len(v)) if v else (None, 0)

    fs, ws = COPY_BYTES / 1024 / big_copy(fetch_dir), COPY_BYTES / 1024 / big_copy(write_dir)
    alg = {"fused": fused_bytes(wl, n), "gemv": algorithmic_bytes(wl, n), "probe": wl.weight_bytes,
           "quantize": n * wl.K * 4 + n * (wl.K // 32) * 36}
    forms = {}
    for kind, a in alg.items():
        fk, nf = med(fetch_dir, kind)
        wk, nw = med(write_dir, kind)
        if fk is None or wk is None:
            continue
        t = fk * 1024 * fs + wk * 1024 * ws
        forms[kind] = {"fetch_kib_per_launch": fk, "write_kib_per_launch": wk, "dispatches": [nf, nw],
                       "traffic_bytes_per_launch": int(t), "algorithmic_bytes_per_launch": a,
                       "traffic_over_algorithmic": round(t / a, 4)}
    name = f"{workload}_n{n}"
    cmd = (f"cd /tmp && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch_{name} "
           f"-o bench -- python3 <repo>/bench.py --cpu-seconds 0 --workload {workload} --n {n} --steps 50 "
           f"--warmup 10 --copy-probe")
    with open(os.path.join(PROFILES, f"{name}_hbm_traffic.md"), "w") as f:
        f.write(f"# HBM traffic: {workload}, n={n}\n\nCommands (MI355X, one GPU):\n\n    {cmd}\n    "
                f"{cmd.replace('FETCH_SIZE', 'WRITE_SIZE').replace('fetch_', 'write_')}\n\n")
        f.write(f"Calibration: a 256 MiB device copy in the same process; FETCH_SIZE scale {fs:.4f}, "
                f"WRITE_SIZE scale {ws:.4f}.\n\n| form | FETCH KiB | WRITE KiB | traffic MB | algorithmic MB | "
                f"ratio |\n|---|---|---|---|---|---|\n")
        for k, g in forms.items():
            f.write(f"| {k} | {g['fetch_kib_per_launch']:.1f} | {g['write_kib_per_launch']:.1f} | "
                    f"{g['traffic_bytes_per_launch'] / 1e6:.3f} | {g['algorithmic_bytes_per_launch'] / 1e6:.3f} | "
                    f"{g['traffic_over_algorithmic']} |\n")
        f.write("\n```json\n" + json.dumps({"workload": workload, "n": n, "source_sha256_16": kernel_source_hash(ALL_SOURCES),
                                            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                                            "forms": forms}, indent=1) + "\n```\n")
    print(json.dumps({"workload": workload, "n": n, "forms": forms}))


def summarize_sq(sq_dir: str, workload: str, n: int) -> None:
    """profiles/<workload>_n<n>_sq_counters.md: SQ counters per launch
    (median over dispatches) of each benchmark form, and the ALU ceiling they
    imply: VALU wave-instructions / the issue peak."""
    import statistics
    from quantized_decode_gemv_quantize_amd import synth
    wl = synth.BY_NAME[workload]
    vals = {}
    for r in _csv_rows(sq_dir, "*counter_collection.csv"):
        k = kernel_form(r["Kernel_Name"])
        if k:
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    forms = {}
    for k, cs in sorted(vals.items()):
        med = {c: statistics.median(v) for c, v in cs.items()}
        valu = med.get("SQ_INSTS_VALU", 0.0)
        forms[k] = {"dispatches": len(next(iter(cs.values()))), **{c: round(v) for c, v in med.items()},
                    "valu_issue_bound_us": round(valu / VALU_ISSUE_PEAK * 1e6, 3),
                    "valu_per_weight_byte_per_column": round(valu * 64 / (wl.weight_bytes * max(n, 1)), 4)}
    name = f"{workload}_n{n}"
    cmd = (f"cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv "
           f"-d <out>/sq_{name} -o bench -- python3 <repo>/bench.py --cpu-seconds 0 --workload {workload} "
           f"--n {n} --steps 50 --warmup 10")
    with open(os.path.join(PROFILES, f"{name}_sq_counters.md"), "w") as f:
        f.write(f"# SQ counters: {workload}, n={n}\n\n")
        f.write(f"Command (MI355X, one GPU):\n\n    {cmd}\n\n")
        f.write("Per launch, median over dispatches. `valu_issue_bound_us` = SQ_INSTS_VALU / 614.4e9 "
                "(256 CUs x 4 SIMDs x 2.4 GHz, one wave64 vector instruction per SIMD every 4 cycles): the "
                "time the vector instructions alone take with every SIMD issuing every cycle. "
                "`valu_per_weight_byte_per_column` counts lane-instructions (x64) per weight byte and "
                "activation column.\n\n")
        cols = ["dispatches"] + SQ_COUNTERS + ["valu_issue_bound_us", "valu_per_weight_byte_per_column"]
        f.write("| form | " + " | ".join(cols) + " |\n|" + "---|" * (len(cols) + 1) + "\n")
        for k, g in forms.items():
            f.write(f"| {k} | " + " | ".join(str(g.get(c, "")) for c in cols) + " |\n")
        f.write("\n```json\n" + json.dumps({"workload": workload, "n": n, "source_sha256_16": kernel_source_hash(ALL_SOURCES),
                                            "forms": forms}, indent=1) + "\n```\n")
    print(json.dumps({"workload": workload, "n": n, "forms": forms}))


def committed_figures(fname: str, names=None):
    """The JSON block of a profiles/ summary, or None when it is absent or
    the kernel sources changed since it was taken (names: the sources its
    hash covers; the per-configuration summaries cover every kernel)."""
    path = os.path.join(PROFILES, fname)
    if not os.path.exists(path):
        return None
    try:
        fig = json.loads(open(path).read().split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    return fig if fig.get("source_sha256_16") == kernel_source_hash(names) else None


def summarize(trace_dir: str, fetch_dir: str, write_dir: str) -> None:
    """Write the kernel-trace and HBM-traffic summaries of the default
    workload under profiles/ (text with one JSON block of the figures), for
    the fused kernel and the two-launch form's mat-vec kernel."""
    import statistics
    rows = _csv_rows

    stats = rows(trace_dir, "*kernel_stats.csv")
    trace = rows(trace_dir, "*kernel_trace.csv")
    dur = {"fused": [], "gemv": [], "quantize": [], "probe": []}
    for r in trace:
        k = kernel_form(r["Kernel_Name"])
        if k in dur:
            dur[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))

    # calibration: the 256 MiB device copy (reads and writes COPY_BYTES)
    def big_copy(d):
        return max(float(r["Counter_Value"]) for r in rows(d, "*counter_collection.csv")
                   if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"))
    fetch_copy, write_copy = big_copy(fetch_dir), big_copy(write_dir)   # weight clones are smaller
    fetch_scale = COPY_BYTES / 1024 / fetch_copy
    write_scale = COPY_BYTES / 1024 / write_copy

    from quantized_decode_gemv_quantize_amd import synth
    wl = synth.BY_NAME["q4_k_4096x14336"]
    figures = {"workload": wl.name, "n": 1, "source_sha256_16": kernel_source_hash(),
               "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
               "quantize_avg_us": round(statistics.mean(dur["quantize"]) / 1e3, 3) if dur["quantize"] else None}
    kinds = [("fused", fused_bytes(wl, 1)), ("gemv", algorithmic_bytes(wl, 1))]

    def probe_counter(d):
        return [float(r["Counter_Value"]) for r in rows(d, "*counter_collection.csv")
                if kernel_form(r["Kernel_Name"]) == "probe"]
    if probe_counter(fetch_dir) and probe_counter(write_dir):
        kinds.append(("probe", wl.weight_bytes))

    def counter(d, kind):
        vals = [float(r["Counter_Value"]) for r in rows(d, "*counter_collection.csv")
                if kernel_form(r["Kernel_Name"]) == kind]
        return statistics.median(vals), len(vals)

    for kind, alg in kinds:
        fk, nf = counter(fetch_dir, kind)
        wk, nw = counter(write_dir, kind)
        traffic = fk * 1024 * fetch_scale + wk * 1024 * write_scale
        d = dur.get(kind) or [0]
        figures[kind] = {
            "launches": len(dur.get(kind, [])), "avg_us": round(statistics.mean(d) / 1e3, 3),
            "median_us": round(statistics.median(d) / 1e3, 3),
            "fetch_kib_per_launch": fk, "write_kib_per_launch": wk, "counter_dispatches": [nf, nw],
            "traffic_bytes_per_launch": int(traffic), "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": round(traffic / alg, 4)}
    os.makedirs(PROFILES, exist_ok=True)
    cmd_trace = ("cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o bench "
                 "-- python3 <repo>/bench.py --cpu-seconds 0")
    cmd_fetch = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch -o bench "
                 "-- python3 <repo>/bench.py --cpu-seconds 0 --steps 50 --warmup 10 --copy-probe")
    cmd_write = cmd_fetch.replace("FETCH_SIZE", "WRITE_SIZE").replace("pmc_fetch", "pmc_write")
    names = {"fused": "fused quantize + mat-vec (mmvq_f32, fp32 activation)",
             "gemv": "mat-vec of the two-launch form (mmvq, q8_1 activation)",
             "probe": "streaming-read probe over the same weight bytes (mmvq_read_probe)"}
    with open(os.path.join(PROFILES, "mmvq_q4_k_4096x14336_n1_kernel_trace.md"), "w") as f:
        f.write("# Kernel trace: Q4_K mat-vec 4096x14336, n=1 (default bench workload)\n\n")
        f.write(f"Command (MI355X, one GPU):\n\n    {cmd_trace}\n\n")
        f.write("rocprofv3 --stats summary (durations in ns):\n\n")
        f.write("| kernel | calls | avg ns | min ns | max ns |\n|---|---|---|---|---|\n")
        for r in stats:
            f.write(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                    f"{r['MinNs']} | {r['MaxNs']} |\n")
        f.write("\n")
        for kind in ("fused", "gemv", "probe"):
            if kind not in figures:
                continue
            g = figures[kind]
            f.write(f"{names[kind]}: {g['launches']} launches, average {g['avg_us']} us, "
                    f"median {g['median_us']} us.\n")
        if figures["quantize_avg_us"] is not None:
            f.write(f"q8_1 quantizer (two-launch form): average {figures['quantize_avg_us']} us.\n")
    with open(os.path.join(PROFILES, "mmvq_q4_k_4096x14336_n1_hbm_traffic.md"), "w") as f:
        f.write("# HBM traffic: Q4_K mat-vec 4096x14336, n=1\n\n")
        f.write(f"Commands:\n\n    {cmd_fetch}\n    {cmd_write}\n\n")
        f.write("Calibration: the same process copies a 256 MiB device buffer (reads and writes 256 MiB);\n"
                f"FETCH_SIZE reads {fetch_copy:.0f} KiB for it (scale {fetch_scale:.4f}), WRITE_SIZE "
                f"{write_copy:.0f} KiB (scale {write_scale:.4f}).\n\n")
        for kind in ("fused", "gemv", "probe"):
            if kind not in figures:
                continue
            g = figures[kind]
            f.write(f"{names[kind]}, per launch (median over dispatches): FETCH_SIZE "
                    f"{g['fetch_kib_per_launch']:.1f} KiB, WRITE_SIZE {g['write_kib_per_launch']:.1f} KiB -> "
                    f"{g['traffic_bytes_per_launch'] / 1e6:.3f} MB of HBM traffic against "
                    f"{g['algorithmic_bytes_per_launch'] / 1e6:.3f} MB algorithmic "
                    f"({g['traffic_over_algorithmic']}x).\n\n")
        f.write("```json\n" + json.dumps(figures, indent=1) + "\n```\n")
    print(json.dumps(figures))


def measured_traffic(kind: str):
    """Traffic per launch of the 'fused' or 'gemv' kernel from the committed
    counter summary, or None when the kernel sources changed since the
    counters were taken."""
    fig = committed_figures("mmvq_q4_k_4096x14336_n1_hbm_traffic.md")
    if fig is None or kind not in fig:
        return None
    return fig[kind]["traffic_bytes_per_launch"]


def fused_bytes(wl, n: int) -> int:
    """Bytes one fused (fp32-activation) launch must move: weights once, the
    fp32 columns, the fp32 outputs."""
    return wl.weight_bytes + n * wl.K * 4 + n * wl.M * 4


def algorithmic_bytes(wl, n: int) -> int:
    """Bytes one mat-vec launch must move: weights once, the q8_1 columns,
    the fp32 outputs (plus the gate matrix and expert gather in fused/id
    modes, counted by the callers)."""
    return wl.weight_bytes + n * (wl.K // 32) * 36 + n * wl.M * 4


class Timer:
    """HIP events on the given stream."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream

    def __enter__(self):
        self.a = self.torch.cuda.Event(enable_timing=True)
        self.b = self.torch.cuda.Event(enable_timing=True)
        self.a.record(self.stream)
        return self

    def __exit__(self, *exc):
        self.b.record(self.stream)
        self.b.synchronize()
        self.ms = self.a.elapsed_time(self.b)


def gpu_setup(torch, wl, n: int, seed_offset: int = 0):
    from quantized_decode_gemv_quantize_amd import synth
    data = synth.make(wl, n)
    copies = max(2, math.ceil(3 * LLC_BYTES / wl.weight_bytes))
    W0 = torch.from_numpy(data["W"]).to("cuda:0")
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(data["x"]).to("cuda:0")
    y = torch.empty((n, wl.K // 32 * 36), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((n, wl.M), dtype=torch.float32, device="cuda:0")
    return data, Ws, x, y, out


def capture(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def launches_graph(torch, stream, launch, count: int, copies: int):
    """One HIP graph holding exactly `count` launches; launch i uses weight
    copy i mod copies."""
    def body():
        for i in range(count):
            launch(i % copies)
    return capture(torch, stream, body)


def timed_replay(torch, stream, g_warm, g_timed):
    """Untimed warmup graph, then the timed graph bracketed by synchronizes;
    HIP events on the launch stream. Returns (ms on the events, wall s)."""
    with torch.cuda.stream(stream):
        if g_warm is not None:
            g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with Timer(torch, stream) as t:
            g_timed.replay()
        torch.cuda.synchronize()
    return t.ms, time.perf_counter() - t0


def mmq_route(B, wl, n: int, fp32: bool = False) -> bool:
    """True where mmvq (q8_1 columns) or mmvq_f32 (fp32 columns) runs the
    many-column (matrix-core) kernel: K a multiple of 256 and n at least the
    library's crossover for that form."""
    if wl.K % 256:
        return False
    return n >= B.mmvq_many_columns_min(wl.wtype, False, fp32=fp32)


def time_workload(torch, B, wl, n: int, steps: int, warmup: int, probe: bool = True, glu: bool = False):
    """GPU timings of one workload: exactly `steps` timed launches of each
    form after `warmup` untimed ones, weights rotating over the copies.
    Forms: fused (mmvq_f32), two-launch step (quantize + mmvq), mat-vec alone
    (mmvq), quantizer alone, the gate/up form (mmvq_glu, SwiGLU, the next
    weight copy as the gate matrix: twice the weight bytes) and its fused
    form (mmvq_glu_f32), and the streaming-read probe over the same weight
    bytes."""
    data, Ws, x, y, out = gpu_setup(torch, wl, n)
    C = len(Ws)
    s = torch.cuda.Stream()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    forms = {
        "step": lambda c: (B.mmvq_quantize_q8_1(x, wl.K, n, wl.K, y, s), B.mmvq(Ws[c], wl.wtype, wl.M, wl.K, y, n, out, s)),
        "gemv": lambda c: B.mmvq(Ws[c], wl.wtype, wl.M, wl.K, y, n, out, s),
        "glu": (lambda c: B.mmvq_glu(Ws[(c + 1) % C], Ws[c], wl.wtype, wl.M, wl.K, y, n, B.GLU_SWIGLU, out, s))
        if glu else None,
        "glu_f32": (lambda c: B.mmvq_glu_f32(Ws[(c + 1) % C], Ws[c], wl.wtype, wl.M, wl.K, x, n, wl.K,
                                             B.GLU_SWIGLU, out, s)) if glu else None,
        "quant": lambda c: B.mmvq_quantize_q8_1(x, wl.K, n, wl.K, y, s),
        "fused": lambda c: B.mmvq_f32(Ws[c], wl.wtype, wl.M, wl.K, x, n, wl.K, out, s),
        "probe": (lambda c: B.mmvq_read_probe(Ws[c], wl.weight_bytes, sink, s)) if probe else None,
    }
    res = {"copies": C, "steps": steps, "warmup": warmup}
    # the two step forms must agree before either is timed: bit for bit,
    # except where only the q8_1 form runs the many-column kernel (another
    # summation order; a loose relative check)
    ref = torch.empty_like(out)
    B.mmvq_quantize_q8_1(x, wl.K, n, wl.K, y, s)
    B.mmvq(Ws[0], wl.wtype, wl.M, wl.K, y, n, ref, s)
    B.mmvq_f32(Ws[0], wl.wtype, wl.M, wl.K, x, n, wl.K, out, s)
    torch.cuda.synchronize()
    if mmq_route(B, wl, n) != mmq_route(B, wl, n, fp32=True):
        same = bool(((ref - out).abs() <= 1e-4 * ref.abs().max() + 1e-6).all())
    else:
        same = torch.equal(ref.view(torch.int32), out.view(torch.int32))
    if not same:
        raise RuntimeError(f"{wl.name} n={n}: fused and two-launch results differ")
    for key, launch in forms.items():
        if launch is None:
            res[f"{key}_us"] = None
            continue
        g_warm = launches_graph(torch, s, launch, warmup, C) if warmup > 0 else None
        g_timed = launches_graph(torch, s, launch, steps, C)
        ms, wall = timed_replay(torch, s, g_warm, g_timed)
        res[f"{key}_ms_total"] = ms
        res[f"{key}_us"] = ms * 1e3 / steps
        res[f"{key}_wall_s"] = wall
        del g_warm, g_timed
    return res, data, Ws, y, out


def time_moe(torch, B, wl, reps: int = 200):
    """The expert-indexed fused gate/up workload: quantize + mmvq_id_glu (two
    launches), mmvq_id_glu alone, and the fused mmvq_id_glu_f32, on two
    copies of the expert weights used alternately (each copy exceeds the
    last-level cache). Returns a dict of µs per call and the algorithmic
    bytes (distinct experts hit x gate and up matrices + activation + out)."""
    from quantized_decode_gemv_quantize_amd import synth
    n = wl.n[0]
    d = synth.make(wl, n)
    E, M, K, top_k = wl.n_experts, wl.M, wl.K, wl.top_k
    per = d["W_up"][0].size
    stride = (per + 15) // 16 * 16
    def stack(A):
        buf = np.zeros(E * stride, dtype=np.uint8)
        for e in range(E):
            buf[e * stride:e * stride + per] = A[e].reshape(-1)
        return torch.from_numpy(buf).to("cuda:0")
    copies = [(stack(d["W_gate"]), stack(d["W_up"]))]
    copies.append((copies[0][0].clone(), copies[0][1].clone()))
    x = torch.from_numpy(d["x"]).to("cuda:0")
    ids = torch.from_numpy(d["ids"]).to("cuda:0")
    y = torch.empty((n, K // 32 * 36), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((n * top_k, M), dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()

    def two():
        for g, u in copies:
            B.mmvq_quantize_q8_1(x, K, n, K, y, s)
            B.mmvq_id_glu(g, u, stride, E, wl.wtype, M, K, y, n, ids, top_k, B.GLU_SWIGLU, out, s)

    def gemv():
        for g, u in copies:
            B.mmvq_id_glu(g, u, stride, E, wl.wtype, M, K, y, n, ids, top_k, B.GLU_SWIGLU, out, s)

    def fused():
        for g, u in copies:
            B.mmvq_id_glu_f32(g, u, stride, E, wl.wtype, M, K, x, n, K, ids, top_k, B.GLU_SWIGLU, out, s)

    # full epilogue (per-expert scales and bias rows) plus a shared expert,
    # one launch: 2 more matrices per call, every token
    rng = np.random.default_rng(0)
    Sg = torch.from_numpy(synth.weights(wl.wtype, M, K, rng)).to("cuda:0")
    Su = torch.from_numpy(synth.weights(wl.wtype, M, K, rng)).to("cuda:0")
    biases = [torch.from_numpy(rng.standard_normal(E * M).astype(np.float32)).to("cuda:0") for _ in range(2)]
    scales = [torch.ones(E, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    epi = B.epilogue(up_bias=biases[0], gate_bias=biases[1], up_scale=scales[0], gate_scale=scales[1],
                     glu_op=B.GLU_SWIGLU)
    shared_out = torch.empty((n, M), dtype=torch.float32, device="cuda:0")

    def ex_shared():
        for g, u in copies:
            B.mmvq_id_ex(u, g, stride, E, wl.wtype, M, K, y, None, 0, n, ids, top_k, epi, Su, Sg, shared_out,
                         out, s)

    res = {}
    with torch.cuda.stream(s):
        for key, fn in (("two_launch_step_us", two), ("id_glu_us", gemv), ("fused_us", fused),
                        ("ex_shared_us", ex_shared)):
            g = capture(torch, s, fn)
            for _ in range(5):
                g.replay()
            torch.cuda.synchronize()
            with Timer(torch, s) as t:
                for _ in range(reps):
                    g.replay()
            res[key] = round(t.ms * 1e3 / (reps * len(copies)), 3)
    distinct = len(set(int(v) for v in d["ids"].reshape(-1)))
    alg = distinct * 2 * M * (K // 256) * 144 + n * (K // 32) * 36 + n * top_k * M * 4
    res.update(workload=wl.name, n=n, distinct_experts=distinct, bytes_per_call=alg,
               id_glu_gbs=round(alg / (res["id_glu_us"] * 1e-6) / 1e9, 1))
    res["frac"] = round(res["id_glu_gbs"] / HBM_PEAK_GBS, 4)
    ex_bytes = alg + 2 * M * (K // 256) * 144 + n * M * 4
    res["ex_shared_gbs"] = round(ex_bytes / (res["ex_shared_us"] * 1e-6) / 1e9, 1)
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, data, n: int, budget_s: float):
    """The oracle on the host: full mat-vecs (quantize + all rows), repeated
    until half the wall-clock budget is spent with the rows split over every
    host core, then for the other half on one thread."""
    import concurrent.futures as cf

    import oracle
    O = oracle.default()
    L = O.L
    W = np.ascontiguousarray(data["W"]).reshape(-1)
    x = np.ascontiguousarray(data["x"])
    out = np.zeros((n, wl.M))

    def rows(r0, r1, y):
        rc = L.orc_mmvq_rows(W.ctypes.data, wl.wtype, wl.M, wl.K, y.ctypes.data, n, int(r0), int(r1),
                             out.ctypes.data, None, None)
        assert rc == 0

    def run(threads: int, seconds: float):
        chunks = np.linspace(0, wl.M, threads + 1).astype(np.int64)
        reps = 0
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            while True:
                y = O.quantize_q8_1(x)
                list(ex.map(lambda i: rows(chunks[i], chunks[i + 1], y), range(threads)))
                reps += 1
                if time.perf_counter() - t0 >= seconds:
                    break
        return reps, time.perf_counter() - t0

    cores = os.cpu_count() or 1
    reps, dt = run(cores, budget_s / 2)
    reps1, dt1 = run(1, budget_s / 2)
    return {"value": round(wl.weight_bytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} full {wl.name} n={n} passes (q8_1 quantize + all {wl.M} rows) with rows split "
                      f"over {cores} threads in {dt:.1f} s wall, then {reps1} on one thread in {dt1:.1f} s",
            "us_per_gemv": round(dt / reps * 1e6, 1),
            "single_thread_gbs": round(wl.weight_bytes * reps1 / dt1 / 1e9, 4),
            "single_thread_us_per_gemv": round(dt1 / reps1 * 1e6, 1),
            "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.n, args.moe, args.steps, args.warmup)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.workload, args.n)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.workload, args.n)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(across GPUs the mat-vec would shard by rows, each GPU running this kernel on its share)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from quantized_decode_gemv_quantize_amd import binding as B
    from quantized_decode_gemv_quantize_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    B.lib()
    wl = synth.BY_NAME[args.workload]
    n = args.n

    if args.copy_probe:
        a = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.moe:
        print(json.dumps(time_moe(torch, B, synth.BY_NAME["moe_q4_k_8x14336x4096"])), flush=True)
        return

    res, data, Ws, y, out = time_workload(torch, B, wl, n, args.steps, args.warmup)
    # the fused forms take at most 8 columns; beyond that a step is the two launches
    fused = args.step == "fused" and res["fused_us"] is not None
    step_us = res["fused_us"] if fused else res["step_us"]
    step_ms = step_us / 1e3
    value = wl.weight_bytes / (step_us * 1e-6) / 1e9
    # roofline of the step's dominant kernel: the fused kernel reads the
    # weights and the fp32 activation; the two-launch form's mat-vec reads
    # the weights and the q8_1 activation
    kern_bytes = fused_bytes(wl, n) if fused else algorithmic_bytes(wl, n)
    kern_us = res["fused_us"] if fused else res["gemv_us"]
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, data, n, args.cpu_seconds)

    line = {
        "metric": f"{synth.TYPE_NAME[wl.wtype].upper()} GEMV effective weight GB/s (% of HBM peak) "
                  f"at {wl.M}\u00d7{wl.K}, n={n}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xu4 dot, f32 scale",
        "data": "synthetic (seeded; random codes and scales, x ~ N(0,1))",
        "config": {"workload": wl.name, "type": synth.TYPE_NAME[wl.wtype], "M": wl.M, "K": wl.K,
                   "n": n, "weight_bytes": wl.weight_bytes, "weight_copies": res["copies"],
                   "parallelism": "single GPU"},
        "detail": {
            "step_form": "one fused launch (mmvq_f32)" if fused else "quantize + mat-vec launches",
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "fused_us": None if res["fused_us"] is None else round(res["fused_us"], 3),
            "gemv_us": round(res["gemv_us"], 3),
            "quantize_us": round(res["quant_us"], 3),
            "two_launch_step_us": round(res["step_us"], 3),
            "gemv_weight_gbs": round(wl.weight_bytes / (res["gemv_us"] * 1e-6) / 1e9, 1),
            "gemv_per_s": round(1e6 / res["gemv_us"], 1),
            "decode_tokens_per_s_equiv": round(value / TOKENS_DENOM_GB, 1),
            "step_wall_s": round(res["step_wall_s"], 4),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic("fused" if fused else "gemv")
                                 if wl.name == "q4_k_4096x14336" and n == 1 else None),
                     "kernel": (f"mmq_kernel ({synth.TYPE_NAME[wl.wtype].upper()}, n={n}, int8 matrix cores, "
                                f"{'fp32' if fused else 'q8_1'} columns)"
                                if mmq_route(B, wl, n, fp32=fused) else
                                f"{'mmvq_rows1_kernel' if n == 1 and wl.wtype != B.Q6_K and wl.M >= 4096 else 'mmvq_rows_kernel'} "
                                f"({synth.TYPE_NAME[wl.wtype].upper()}, n={n}, "
                                f"{'fp32' if fused else 'q8_1'} activation)"),
                     "bytes_per_launch": kern_bytes,
                     "avg_launch_us": round(kern_us, 3),
                     # the same weight bytes through the streaming-read probe
                     # (mmvq_read_probe), same copies and step count: the
                     # read ceiling of one launch of this size on this part
                     "probe_us": round(res["probe_us"], 3),
                     "probe_gbs": round(wl.weight_bytes / (res["probe_us"] * 1e-6) / 1e9, 1),
                     "pct_of_probe": round(100 * res["probe_us"] / kern_us, 2)},
        "cpu_baseline": cpu,
    }
    # ALU ceiling of the dominant kernel from its committed SQ counters (same
    # sources): where its vector instructions alone need longer than its
    # bytes at the HBM peak, the kernel is bound by instruction issue and the
    # roofline is reported against the vector issue peak.
    sq = committed_figures(f"{wl.name}_n{n}_sq_counters.md", ALL_SOURCES)
    form = "fused" if fused else "gemv"
    if sq is not None and form in sq.get("forms", {}):
        valu = sq["forms"][form]["SQ_INSTS_VALU"]
        issue_us = valu / VALU_ISSUE_PEAK * 1e6
        hbm_us = kern_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
        alu = {"valu_wave_insts_per_launch": valu, "valu_issue_bound_us": round(issue_us, 3),
               "hbm_bound_us": round(hbm_us, 3), "issue_peak_tops": round(VALU_ISSUE_PEAK * 64 / 1e12, 2)}
        if issue_us > hbm_us:
            r = line["roofline"]
            r["hbm"] = {k: r[k] for k in ("achieved", "peak", "unit", "frac")}
            tops = valu * 64 / (kern_us * 1e-6) / 1e12
            r.update(bound="alu", achieved=round(tops, 2), peak=alu["issue_peak_tops"], unit="TOP/s",
                     frac=round(tops / alu["issue_peak_tops"], 4))
        line["roofline"]["alu"] = alu
    print(json.dumps(line), flush=True)

    if args.all:
        for name in ["q4_0_256x1024", "q4_k_4096x4096", "q4_k_4096x14336", "q4_k_14336x4096",
                     "q6_k_128256x4096", "q8_0_4096x14336", "q4_1_4096x14336", "q5_0_4096x14336",
                     "q5_1_4096x14336", "q5_k_4096x14336"]:
            w = synth.BY_NAME[name]
            many = ((16, 32, 64, 128) if name in ("q4_k_4096x14336", "q4_k_14336x4096")
                    else (16, 64) if name in ("q6_k_128256x4096", "q8_0_4096x14336") else (16,))
            for nn in tuple(w.n if name != "q4_k_4096x14336" else (1, 2, 4, 8)) + many:
                r, *_ = time_workload(torch, B, w, nn, 500, 50, glu=name == "q4_k_14336x4096")
                gb = algorithmic_bytes(w, nn) / (r["gemv_us"] * 1e-6) / 1e9
                print(json.dumps({"workload": name, "n": nn, "gemv_us": round(r["gemv_us"], 3),
                                  "glu_us": None if r["glu_us"] is None else round(r["glu_us"], 3),
                                  "glu_f32_us": None if r["glu_f32_us"] is None else round(r["glu_f32_us"], 3),
                                  "quantize_us": round(r["quant_us"], 3),
                                  "two_launch_step_us": round(r["step_us"], 3),
                                  "fused_us": None if r["fused_us"] is None else round(r["fused_us"], 3),
                                  "probe_us": round(r["probe_us"], 3),
                                  "gemv_gbs": round(gb, 1), "frac": round(gb / HBM_PEAK_GBS, 4)}),
                      file=sys.stderr, flush=True)
        print(json.dumps(time_moe(torch, B, synth.BY_NAME["moe_q4_k_8x14336x4096"])), file=sys.stderr,
              flush=True)


if __name__ == "__main__":
    main()
