"""Kernel-time and HBM-traffic measurement of the benchmark with rocprofv3.

    python -m tiered_kv_cache_hs_amd.profiling run --workloads 3 4 5 6 7 --out DIR

runs, for each workload, from the repository root:

  * one kernel-trace pass:
      rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace_wlN -o bench --
          python3 -u bench.py --workload N --steps 24 --warmup 8 --no-cpu
  * two counter passes (one counter each, as the profiler collects in one pass):
      rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/pmc_wlN_FETCH_SIZE -o run --
          python3 -u bench.py --workload N --steps 3 --warmup 1 --no-cpu
      (then WRITE_SIZE)
  * once, the same two counters over a 256 MiB device-to-device copy
    (bench.py --copy-calibration), which scale the counters to bytes;

each as a child process under a time limit (this process never touches the
GPU), and writes into DIR/report: one summary per workload
(hs_kernels_<workload>.md: the profiler's per-kernel statistics, warm
averages, the benchmark's own event-timed kernel durations from the same run
and the HBM bytes per dispatch) and pmc_traffic.json, the per-dispatch HBM
bytes that bench.py reports as `traffic`, keyed by the SHA-1 of each kernel's
sources so a reading is used only while the kernel is unchanged.

    python -m tiered_kv_cache_hs_amd.profiling report --workloads ... --out DIR

rebuilds the report from existing run directories.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time
from typing import Dict, List, Optional

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiered_kv_cache_hs_amd", "csrc")
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
COUNTERS = ("FETCH_SIZE", "WRITE_SIZE")
# one pass of shader-sequencer counters (at most 8 SQ counters per pass):
# where a kernel's cycles go
SQ_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
               "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_VALU_MFMA_BUSY_CYCLES",
               "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")
COPY_BYTES = 256 << 20

# the kernel's file, the shared header and the launch planner: a stored
# reading is used only while all three are unchanged
KERNEL_SOURCES = {
    "hs_k_resolve": ["resolve.hip", "hs_device.h", "runtime.hip"],
    "hs_k_gather": ["resolve.hip", "hs_device.h", "runtime.hip"],
    "hs_k_attn_latent": ["attn_latent.hip", "hs_device.h", "runtime.hip"],
    "hs_k_attn_mha": ["attn_mha.hip", "hs_device.h", "runtime.hip"],
    "hs_k_combine": ["attn_mha.hip", "hs_device.h", "runtime.hip"],
    "hs_k_combine_wave": ["attn_mha.hip", "hs_device.h", "runtime.hip"],
    "hs_k_stage": ["stage.hip", "hs_device.h", "runtime.hip"],
    "hs_k_append_next": ["resolve.hip", "hs_device.h", "runtime.hip"],
}


def kernel_sources_sha1(kernel: str) -> str:
    h = hashlib.sha1()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str, path: str = "auto") -> Optional[int]:
    """HBM bytes per dispatch of `kernel` on `workload` (benchmark --path
    `path`) from the committed counter readings, or None when there is none
    or the kernel's sources changed since it was taken."""
    try:
        with open(PMC_FILE) as fh:
            pmc = json.load(fh)
    except (OSError, ValueError):
        return None
    for e in pmc.get("entries", []):
        if (e.get("workload") == workload and e.get("kernel") == kernel
                and e.get("path", "auto") == path):
            if e.get("sources_sha1") != kernel_sources_sha1(kernel):
                return None
            return int(e["traffic_bytes"])
    return None


def short_name(name: str) -> str:
    m = re.search(r"(hs_k_\w+)", name)
    return m.group(1) if m else name.split("(")[0][:48]


def display_name(name: str) -> str:
    """hs_k_name<template arguments> out of a demangled kernel name."""
    m = re.search(r"(hs_k_\w+(<[^>]*>)?)", name)
    return m.group(1) if m else name.split("(")[0][:60]


def _one(pattern: str) -> Optional[str]:
    f = sorted(glob.glob(pattern, recursive=True))
    return f[0] if f else None


# ------------------------------------------------------------------ runs

def _child(cmd: List[str], log: str, limit: int) -> int:
    """Run cmd from the repository root under a time limit (killed with
    SIGKILL when it runs over); output to log."""
    print(f"[profiling] {' '.join(cmd)}", flush=True)
    t0 = time.time()
    with open(log, "w") as fh:
        try:
            p = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, cwd=ROOT, stdout=fh,
                               stderr=subprocess.STDOUT, timeout=limit + 30)
            rc = p.returncode
        except subprocess.TimeoutExpired:
            rc = 124
    print(f"[profiling]   rc={rc} in {time.time() - t0:.1f}s", flush=True)
    return rc


# bench.py --path for every run ("auto": the benchmark's own choice per record
# kind); another path gets its own run directories and summary names
PATH = "auto"


def _tag(wl: int) -> str:
    return f"wl{wl}" + ("" if PATH == "auto" else f"_{PATH}")


def path_args() -> List[str]:
    """bench.py options of the current path: --path fused / split, or (gather)
    --fetch kernel, the misses moved by a gather kernel of their own."""
    if PATH == "auto":
        return []
    return ["--fetch", "kernel"] if PATH == "gather" else ["--path", PATH]


def bench_cmd(wl: Optional[int], steps: int, warmup: int) -> List[str]:
    if wl is None:
        return ["python3", "-u", "bench.py", "--copy-calibration"]
    return ["python3", "-u", "bench.py", "--workload", str(wl), "--steps", str(steps),
            "--warmup", str(warmup), "--no-cpu"] + path_args()


def trace_cmd(out: str, wl: int) -> List[str]:
    return ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
            os.path.join(out, f"trace_{_tag(wl)}"), "-o", "bench", "--"] + bench_cmd(wl, 24, 8)


def pmc_cmd(out: str, tag: str, counter: str, wl: Optional[int]) -> List[str]:
    return ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d",
            os.path.join(out, f"pmc_{tag}_{counter}"), "-o", "run", "--"] + bench_cmd(wl, 3, 1)


def sq_cmd(out: str, wl: int) -> List[str]:
    return ["rocprofv3", "--pmc", *SQ_COUNTERS, "--output-format", "csv", "-d",
            os.path.join(out, f"sq_wl{wl}"), "-o", "run", "--"] + bench_cmd(wl, 3, 1)


def run_sq(workloads: List[int], out: str, limit: int) -> None:
    os.makedirs(out, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    for wl in workloads:
        if _child(sq_cmd(out, wl), os.path.join(out, f"sq_wl{wl}.log"), limit):
            raise SystemExit(f"counter pass of workload {wl} failed")


def read_counters_by_name(d: str) -> Dict[str, Dict[str, List[float]]]:
    """{kernel: {counter: [value per dispatch]}} from a counter-collection CSV."""
    f = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per: Dict[str, Dict[str, List[float]]] = {}
    if f:
        for r in csv.DictReader(open(f)):
            k = display_name(r["Kernel_Name"])
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return per


def sq_report(workloads: List[int], out: str) -> None:
    """hs_sq_<workload>.md: per kernel, the median of each SQ counter over
    its dispatches and the derived shares of busy cycles."""
    from . import inputs as I

    rep_dir = os.path.join(out, "report")
    os.makedirs(rep_dir, exist_ok=True)
    rel = os.path.relpath(out, ROOT)
    for wl in workloads:
        w = I.workload(wl)
        per = read_counters_by_name(os.path.join(out, f"sq_wl{wl}"))
        lines = [f"# Shader-sequencer counters: workload {w.name}", "",
                 "Made on one MI355X from the repository root by", "",
                 f"    python3 -u -m tiered_kv_cache_hs_amd.profiling sq --workloads "
                 f"{' '.join(str(x) for x in workloads)} --out {rel}", "",
                 "which runs", "", "    " + " ".join(sq_cmd(rel, wl)), "",
                 "Medians over each kernel's dispatches (counts summed over the device).", "",
                 "| kernel | dispatches | " + " | ".join(SQ_COUNTERS) + " |",
                 "|---|---|" + "---|" * len(SQ_COUNTERS)]
        derived = []
        for k, cs in sorted(per.items()):
            if not k.startswith("hs_k") or "buffer_init" in k:
                continue
            med = {c: statistics.median(cs[c]) if c in cs else float("nan") for c in SQ_COUNTERS}
            n = len(next(iter(cs.values())))
            lines.append(f"| {k} | {n} | " + " | ".join(f"{med[c]:.3g}" for c in SQ_COUNTERS) + " |")
            wave = med["SQ_WAVE_CYCLES"]
            # GRBM_GUI_ACTIVE is summed over the 8 XCDs (divided by 8 it
            # matches the traced kernel duration); 256 CUs x 4 SIMDs
            cycles = med["GRBM_GUI_ACTIVE"] / 8.0
            if wave > 0 and cycles > 0:
                derived.append(f"| {k} | {cycles:.0f} | {med['SQ_WAIT_INST_ANY'] / wave:.2f} | "
                               f"{med['SQ_ACTIVE_INST_VALU'] / wave:.2f} | "
                               f"{med['SQ_ACTIVE_INST_LDS'] / wave:.2f} | "
                               f"{med['SQ_ACTIVE_INST_VMEM'] / wave:.2f} | "
                               f"{100.0 * med['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * 1024):.1f} |")
        lines += ["", "Derived: kernel cycles = GRBM_GUI_ACTIVE / 8 (the counter is summed over "
                  "the 8 XCDs; so divided it matches the traced duration); the wait and "
                  "active-instruction counters as shares of wave cycles; MFMA busy = "
                  "SQ_VALU_MFMA_BUSY_CYCLES over kernel cycles x 1024 SIMDs.", "",
                  "| kernel | kernel cycles | waiting | VALU issue | LDS issue | VMEM issue | "
                  "MFMA busy % |", "|---|---|---|---|---|---|---|"] + derived
        with open(os.path.join(rep_dir, f"hs_sq_{w.name}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    print(f"[profiling] counter report in {rep_dir}", flush=True)


def run_all(workloads: List[int], out: str, limit: int) -> None:
    os.makedirs(out, exist_ok=True)
    env_ok = os.environ.get("TMPDIR")
    if not env_ok:
        os.environ["TMPDIR"] = "/tmp"
    for c in COUNTERS:
        if _child(pmc_cmd(out, "copy", c, None), os.path.join(out, f"pmc_copy_{c}.log"), limit):
            raise SystemExit("copy calibration pass failed")
    for wl in workloads:
        if _child(trace_cmd(out, wl), os.path.join(out, f"trace_{_tag(wl)}.log"), limit):
            raise SystemExit(f"trace pass of workload {wl} failed")
        for c in COUNTERS:
            if _child(pmc_cmd(out, _tag(wl), c, wl), os.path.join(out, f"pmc_{_tag(wl)}_{c}.log"),
                      limit):
                raise SystemExit(f"{c} pass of workload {wl} failed")


# ---------------------------------------------------------------- report

def read_counter(d: str) -> Dict[str, List[float]]:
    f = _one(os.path.join(d, "**", "*counter_collection.csv"))
    per: Dict[str, List[float]] = {}
    if f:
        for r in csv.DictReader(open(f)):
            per.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def read_stats(d: str):
    f = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    rows = []
    if f:
        for r in csv.DictReader(open(f)):
            rows.append(r)
    return rows


def read_trace(d: str):
    """({kernel: [durations us]}, {kernel: resource columns of its dispatches})."""
    f = _one(os.path.join(d, "**", "*kernel_trace.csv"))
    per: Dict[str, List[float]] = {}
    res: Dict[str, dict] = {}
    if f:
        for r in csv.DictReader(open(f)):
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            n = display_name(r["Kernel_Name"])
            per.setdefault(n, []).append(dur)
            res.setdefault(n, {k: r.get(k) for k in ("VGPR_Count", "Accum_VGPR_Count",
                                                      "SGPR_Count", "LDS_Block_Size",
                                                      "Scratch_Size", "Workgroup_Size_X",
                                                      "Grid_Size_X")})
    return per, res


def bench_line(log: str) -> Optional[dict]:
    try:
        for line in open(log):
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    except OSError:
        pass
    return None


def report(workloads: List[int], out: str) -> None:
    from . import inputs as I

    rep = os.path.join(out, "report")
    os.makedirs(rep, exist_ok=True)
    rel = os.path.relpath(out, ROOT)
    copy = {c: read_counter(os.path.join(out, f"pmc_copy_{c}")) for c in COUNTERS}
    copy_kib = {}
    for c in COUNTERS:
        vals = [v for k, vs in copy[c].items() if "copy" in k.lower() for v in vs]
        if not vals:
            raise SystemExit(f"no copy-kernel reading of {c}")
        copy_kib[c] = statistics.median(vals)
    scale = {c: COPY_BYTES / (copy_kib[c] * 1024.0) for c in COUNTERS}
    entries = []
    for wl in workloads:
        w = I.workload(wl)
        pmc = {c: read_counter(os.path.join(out, f"pmc_{_tag(wl)}_{c}")) for c in COUNTERS}
        stats = read_stats(os.path.join(out, f"trace_{_tag(wl)}"))
        trace, res = read_trace(os.path.join(out, f"trace_{_tag(wl)}"))
        bl = bench_line(os.path.join(out, f"trace_{_tag(wl)}.log"))
        lines = [f"# Kernel time and HBM traffic: workload {w.name}", "",
                 f"{w.n_requests} requests x {w.n_layers} layers, context "
                 f"{w.ctx[0] if len(set(w.ctx)) == 1 else 'per request'}, {w.kind} records of "
                 f"{w.rec_bytes} bytes, {w.n_q_heads} query heads, k = {w.k}, B = "
                 f"{w.B[0] if len(set(w.B)) == 1 else 'per request'}"
                 + (f", layer groups of {w.share}" if w.share > 1 else "") + ".",
                 "", "Made on one MI355X from the repository root by", "",
                 f"    python3 -u -m tiered_kv_cache_hs_amd.profiling run --workloads "
                 f"{' '.join(str(x) for x in workloads)} --out {rel}"
                 + ("" if PATH == "auto" else f" --path {PATH}"), "",
                 "which runs these passes for this workload, each under `timeout -s KILL`:", "",
                 "    " + " ".join(trace_cmd(rel, wl)),
                 "    " + " ".join(pmc_cmd(rel, _tag(wl), "FETCH_SIZE", wl)),
                 "    " + " ".join(pmc_cmd(rel, _tag(wl), "WRITE_SIZE", wl)),
                 "    " + " ".join(pmc_cmd(rel, "copy", "FETCH_SIZE", None)) + "   (and WRITE_SIZE)",
                 "", "The trace run replays the step graph for 32 decode steps (8 warm-up + 24 "
                 "timed), replays the whole trace three more times from a reset state, then "
                 "runs it once more eagerly with dispatch-timed HIP events on every kernel, so "
                 "each kernel has five dispatches per layer and step.", "",
                 "## rocprofv3 --stats (all dispatches)", "",
                 "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
        for r in stats:
            if "hs_k_" not in r["Name"]:
                continue
            lines.append(f"| {display_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1000:.2f} | "
                         f"{float(r['MinNs']) / 1000:.2f} | {float(r['MaxNs']) / 1000:.2f} | "
                         f"{float(r['Percentage']):.2f} |")
        lines += ["", "## Warm averages (kernel trace, End - Start; each pass's cold first step dropped)",
                  "", "| kernel | dispatches | avg us (warm) | median us (warm) |", "|---|---|---|---|"]
        steps_per_pass, passes = 32, BENCH_PASSES
        for name, durs in trace.items():
            if not name.startswith("hs_k") or "buffer_init" in name or "stage_set" in name:
                continue
            per_step = max(1, len(durs) // (passes * steps_per_pass))
            span = per_step * steps_per_pass
            warm = [d for p0 in range(0, len(durs), span) for d in durs[p0 + per_step:p0 + span]]
            if warm:
                lines.append(f"| {name[:60]} | {len(warm)} | {statistics.mean(warm):.2f} | "
                             f"{statistics.median(warm):.2f} |")
        lines += ["", "## Resources (first dispatch of each kernel)", "",
                  "LDS bytes as the profiler reports them: the static allocation (the "
                  "resolve kernel's dynamic LDS, (max(2H, 5k) + k) * 4 bytes for a hash "
                  "of H entries, is not included).", "",
                  "| kernel | VGPR | AGPR | SGPR | LDS bytes | scratch | workgroup | grid (threads) |",
                  "|---|---|---|---|---|---|---|---|"]
        for name, r in res.items():
            if name.startswith("hs_k") and "buffer_init" not in name:
                lines.append(f"| {name} | {r['VGPR_Count']} | {r['Accum_VGPR_Count']} | "
                             f"{r['SGPR_Count']} | {r['LDS_Block_Size']} | {r['Scratch_Size']} | "
                             f"{r['Workgroup_Size_X']} | {r['Grid_Size_X']} |")
        if bl:
            lines += ["", "## The benchmark's own timing in the same run", "",
                      f"Dispatch-timed kernel durations per launch (us): "
                      f"{json.dumps(bl.get('kernels_us'))}; value {bl.get('value')} us/layer under "
                      f"the profiler; path {bl.get('config', {}).get('path')}."]
        lines += ["", "## HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE; separate passes)", "",
                  f"Scale from the 256 MiB copy: FETCH_SIZE reads {copy_kib['FETCH_SIZE']:.1f} KiB "
                  f"(x{scale['FETCH_SIZE']:.4f}), WRITE_SIZE {copy_kib['WRITE_SIZE']:.1f} KiB "
                  f"(x{scale['WRITE_SIZE']:.4f}).", "",
                  "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | "
                  "HBM bytes per dispatch |", "|---|---|---|---|---|"]
        for k in sorted(set(pmc["FETCH_SIZE"]) & set(pmc["WRITE_SIZE"])):
            if k not in KERNEL_SOURCES:
                continue
            f = statistics.median(pmc["FETCH_SIZE"][k])
            wv = statistics.median(pmc["WRITE_SIZE"][k])
            b = int(round((f * scale["FETCH_SIZE"] + wv * scale["WRITE_SIZE"]) * 1024))
            lines.append(f"| {k} | {len(pmc['FETCH_SIZE'][k])} | {f:.1f} | {wv:.1f} | {b:,} |")
            entries.append({"workload": w.name, "path": PATH, "kernel": k,
                            "sources_sha1": kernel_sources_sha1(k),
                            "dispatches": len(pmc["FETCH_SIZE"][k]), "fetch_kib_median": round(f, 1),
                            "write_kib_median": round(wv, 1), "traffic_bytes": b})
        suffix = "" if PATH == "auto" else f"_{PATH}"
        with open(os.path.join(rep, f"hs_kernels_{w.name}{suffix}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    doc = {"about": "HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE "
                    "(separate passes), median over the dispatches of `python3 -u bench.py "
                    "--workload N --steps 3 --warmup 1 --no-cpu`; each counter scaled by its "
                    "reading for a 256 MiB device-to-device copy (`python3 -u bench.py "
                    "--copy-calibration`). Written by `python -m tiered_kv_cache_hs_amd.profiling`.",
           "scale": {"FETCH_SIZE": round(scale["FETCH_SIZE"], 4),
                     "WRITE_SIZE": round(scale["WRITE_SIZE"], 4),
                     "copy_fetch_kib": round(copy_kib["FETCH_SIZE"], 1),
                     "copy_write_kib": round(copy_kib["WRITE_SIZE"], 1), "copy_bytes": COPY_BYTES},
           "entries": entries}
    # readings of other workloads or paths already in the report (earlier
    # runs into the same directory) are kept
    path = os.path.join(rep, "pmc_traffic.json")
    try:
        with open(path) as fh:
            old = json.load(fh).get("entries", [])
    except (OSError, ValueError):
        old = []
    mine = {(e["workload"], e["path"], e["kernel"]) for e in entries}
    doc["entries"] = [e for e in old if (e["workload"], e.get("path", "auto"), e["kernel"])
                      not in mine] + entries
    with open(path, "w") as fh:
        json.dump(doc, fh, indent=1)
    print(f"[profiling] report in {rep}", flush=True)


# --------------------------------------------- the default benchmark command

# The benchmark's passes over the trace: the timed graph replays (W + K
# steps), three more replays of every step from a reset state, one eager
# pass with dispatch-timed events (the launches its kernel averages take).
BENCH_PASSES = 5
# the command the round's measurement runs
BENCH_DEFAULT = ["python3", "-u", "bench.py", "--gpus", "1", "--steps", "20", "--warmup", "5"]


def bench_trace_cmd(out: str) -> List[str]:
    return ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
            os.path.join(out, "trace_bench"), "-o", "bench", "--"] + BENCH_DEFAULT


def run_bench_trace(out: str, limit: int) -> None:
    """The measured benchmark command as it runs (no profiler), then again
    under the kernel tracer."""
    os.makedirs(out, exist_ok=True)
    os.environ.setdefault("TMPDIR", "/tmp")
    if _child(BENCH_DEFAULT, os.path.join(out, "plain_bench.log"), limit):
        raise SystemExit("the benchmark failed")
    if _child(bench_trace_cmd(out), os.path.join(out, "trace_bench.log"), limit):
        raise SystemExit("trace pass of the benchmark failed")


def bench_report(out: str) -> str:
    """Summary of the measured benchmark command's kernel trace: for every
    kernel, the rocprofv3 durations of the launches the benchmark itself
    times with dispatch events (its last, eager pass: the K steps after the
    W warm-up steps), beside the benchmark's own averages from the same run,
    and the launches of the timed graph replays; then the roofline fraction
    recomputed from the profiler's durations."""
    from . import inputs as I

    bl = bench_line(os.path.join(out, "trace_bench.log"))
    if bl is None:
        raise SystemExit("no benchmark line in the trace log")
    trace, res = read_trace(os.path.join(out, "trace_bench"))
    W, K = int(bl["warmup"]), int(bl["steps"])
    w = next(I.workload(i) for i in range(1, 8) if I.workload(i).name == bl["config"]["workload"])
    rel = os.path.relpath(out, ROOT)
    cls_of = {"hs_k_resolve": "resolve", "hs_k_gather": "gather", "hs_k_attn_latent": "attn",
              "hs_k_attn_mha": "attn", "hs_k_combine": "combine",
              "hs_k_combine_wave": "combine", "hs_k_stage": "stage", "hs_k_append": "append",
              "hs_k_append_next": "append"}
    lines = [f"# Kernel time of the default benchmark: workload {w.name}", "",
             f"{w.n_requests} requests x {w.n_layers} layers, {w.kind} records of "
             f"{w.rec_bytes} bytes, {w.n_q_heads} query heads, k = {w.k}; path "
             f"{bl['config'].get('path')}.", "",
             "Made on one MI355X from the repository root by", "",
             f"    python3 -u -m tiered_kv_cache_hs_amd.profiling bench --out {rel}", "",
             "which runs the measured benchmark command under the kernel tracer:", "",
             "    " + " ".join(bench_trace_cmd(rel)), "",
             f"The benchmark replays its step graph W + K = {W} + {K} times (the timed "
             "region: the last K), replays every step three more times from a reset state, "
             "then runs the steps once more eagerly in the graph's form with events that take "
             "each dispatch's own start and end (the launches whose average is its "
             "`kernels_us` and its roofline `avg_us`). Each kernel below has its dispatches "
             "in that order; the columns take the same launches the benchmark averages.", "",
             "| kernel | dispatches | rocprofv3 avg us (the benchmark's K eager launches) | "
             "median us | benchmark dispatch-timed avg us | rocprofv3 avg us (timed graph "
             "replays) |", "|---|---|---|---|---|---|"]
    ev = bl.get("kernels_us", {})
    prof_avg = {}
    for name, durs in trace.items():
        base = short_name(name)
        if base not in cls_of:
            continue
        per_step = max(1, len(durs) // (BENCH_PASSES * (W + K)))
        eager = durs[-K * per_step:]
        timed = durs[W * per_step:(W + K) * per_step]
        prof_avg[base] = statistics.mean(eager)
        lines.append(f"| {name[:60]} | {len(durs)} | {statistics.mean(eager):.2f} | "
                     f"{statistics.median(eager):.2f} | {ev.get(cls_of[base], 0.0):.2f} | "
                     f"{statistics.mean(timed):.2f} |")
    roof = bl.get("roofline") or {}
    lines += ["", f"Benchmark line of the traced run: value {bl['value']} us/layer; roofline "
              f"{json.dumps(roof)}. (Under the tracer every dispatch carries the profiler's "
              "own bookkeeping, which the benchmark's dispatch events see and the profiler's "
              "durations do not.)"]
    plain = bench_line(os.path.join(out, "plain_bench.log"))
    if plain:
        pr = plain.get("roofline") or {}
        lines += ["", f"The same command without the profiler, just before on the same machine: "
                  f"value {plain['value']} us/layer; kernels_us "
                  f"{json.dumps(plain.get('kernels_us'))}; roofline {json.dumps(pr)}."]
    k = roof.get("kernel")
    if k in prof_avg and roof.get("bytes_per_launch") and roof.get("peak"):
        unit = 1e9 if roof.get("unit") == "GB/s" else 1e12
        ach = roof["bytes_per_launch"] / (prof_avg[k] * 1e-6) / unit
        lines += ["", f"Roofline from the profiler's durations of the same launches: "
                  f"{roof['bytes_per_launch']:,} bytes / {prof_avg[k]:.2f} us = {ach:.2f} "
                  f"{roof.get('unit')}, frac {ach / roof['peak']:.4f} (the traced run's line: "
                  f"{roof.get('frac')}, from {roof.get('avg_us')} us"
                  + (f"; the run without the profiler: {pr.get('frac')}, from "
                     f"{pr.get('avg_us')} us" if plain else "") + ")."]
    os.makedirs(os.path.join(out, "report"), exist_ok=True)
    path = os.path.join(out, "report", f"hs_kernels_bench_default_{w.name}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"[profiling] {path}", flush=True)
    return path


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("action", choices=("run", "report", "sq", "sq-report", "bench",
                                       "bench-report"))
    ap.add_argument("--workloads", type=int, nargs="+", default=[3, 4, 5, 6, 7])
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out"))
    ap.add_argument("--limit", type=int, default=240, help="seconds per profiler pass")
    ap.add_argument("--path", choices=("auto", "fused", "split", "gather"), default="auto",
                    help="bench.py --path of every run (run/report); gather: bench.py --fetch "
                         "kernel")
    a = ap.parse_args()
    global PATH
    PATH = a.path
    if a.action in ("bench", "bench-report"):
        if a.action == "bench":
            run_bench_trace(a.out, a.limit)
        bench_report(a.out)
        return
    if a.action in ("sq", "sq-report"):
        if a.action == "sq":
            run_sq(a.workloads, a.out, a.limit)
        sq_report(a.workloads, a.out)
        return
    if a.action == "run":
        run_all(a.workloads, a.out, a.limit)
    report(a.workloads, a.out)


if __name__ == "__main__":
    main()
