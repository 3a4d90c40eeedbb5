"""rocprofv3 harness: kernel time, HBM bytes and matrix-core activity of the
attention kernels, measured on the GPU and written up as profiles/*.md.

    python -m global_attention_mimo_amd.prof run    --suite step --out gpurun_out/prof
    python -m global_attention_mimo_amd.prof report --suite step --out gpurun_out/prof

``run`` drives rocprofv3 over ``bench.py`` in separate passes, the program
directly after ``--`` and each pass under its own time limit:

  trace   --kernel-trace --stats     every dispatch's duration;
  fetch   --pmc FETCH_SIZE           HBM-side read KiB per dispatch;
  write   --pmc WRITE_SIZE           HBM-side write KiB per dispatch;
  mfma    --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE.

The counter passes add ``--copy-calibration`` to the bench command, so that
one plain 1 GiB device-to-device copy (1 GiB read, 1 GiB written) runs in the
same process; the ratio of its known size to what FETCH_SIZE / WRITE_SIZE
report for it scales every other dispatch's counts to bytes.  ``report``
parses the CSV files of those passes and writes the summary markdown (and, for
the bench step, the GA prefill traffic record that ``bench.py`` reports as its
roofline traffic, keyed by a digest of the kernel's sources).

Derived figures:
  * read / write bytes = counter KiB x 1024 x calibration scale;
  * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs),
    GRBM_GUI_ACTIVE being summed over the XCDs;
  * effective clock = (GRBM_GUI_ACTIVE / XCDs) / the kernel's median duration
    from the trace pass (a different run of the same command).

This module only runs and reads profiler output; it imports nothing that
touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import shlex
import statistics
import subprocess
import sys
import time
from typing import Dict, Iterable, List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# MI355X (gfx950): 256 compute units of 4 SIMDs in 8 XCDs.
SIMDS = 1024
XCDS = 8
CALIBRATION_BYTES = 1 << 30

# Which bench.py arguments each suite profiles: (trace pass, counter passes).
SUITES = {
    "step": ("--steps 20 --warmup 3 --no-cpu-baseline --no-next-rows",
             "--steps 1 --warmup 0 --no-cpu-baseline --no-next-rows"),
    "hybrid": ("--hybrid-only", "--hybrid-only"),
    "next-rows": ("--steps 1 --warmup 1 --no-cpu-baseline --no-hybrid",
                  "--steps 1 --warmup 0 --no-cpu-baseline --no-hybrid"),
}
# Where the waves' time goes: per-wave cycles split into waiting on
# dependencies (s_waitcnt: loads, LDS, barriers), ready but not issued (the
# unit it needs is busy, e.g. the matrix core or the memory pipeline) and
# issuing, the last by instruction kind.
STALL_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_VMEM"]
PASSES = {
    "trace": ["--kernel-trace", "--stats"],
    "fetch": ["--pmc", "FETCH_SIZE"],
    "write": ["--pmc", "WRITE_SIZE"],
    "mfma": ["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"],
    "stalls": ["--pmc", *STALL_COUNTERS],
}
PASS_LIMIT_S = {"trace": 900, "fetch": 600, "write": 600, "mfma": 600, "stalls": 600}

TITLES = {
    "step": "one bench step of the hybrid-attention hot path",
    "hybrid": "the 48-layer hybrid stack (prefill, then 64 decode steps)",
    "next-rows": "chunked prefill, paged and FP8 GA pools, prefill backward and RoPE",
}
WORKLOADS = {
    "step": "`bench.py` step = SWA prefill 4x8192 + GA prefill 1x32768 + decode step B=128, ctx U[4096,262144] "
            "(SWA ring + GA pool, attend then append).",
    "hybrid": "`bench.py --hybrid-only`: 48 layers (5 SWA : 1 GA), 32 prompts with lengths log-uniform in "
              "[512, 32768] (seed 0, 214486 tokens), a varlen prefill of every layer (attention + KV append), then "
              "64 decode steps of all 48 layers (fused attend + append per layer; steps 33-64 replayed from one HIP "
              "graph).  The torch kernels in the trace draw the synthetic inputs outside the timed calls.",
    "next-rows": "the rows `bench.py` times apart from its step (`next_rows`): chunked GA prefill (28672 cached + "
                 "4096 new) over the contiguous and the paged pool, chunked SWA prefill (4 x (8192 cached + 8192 "
                 "new)), the decode step's GA attention over a pool in pages of 16 and over an FP8 E4M3 pool, the "
                 "bulk quantising append, the prefill backward on the step's two prefill inputs, and RoPE.",
}

# Sources whose digest keys the GA prefill traffic record (any code change voids it).
TRAFFIC_SOURCES = ["global_attention_mimo_amd/csrc/prefill.hip", "global_attention_mimo_amd/csrc/device_common.hpp",
                   "global_attention_mimo_amd/csrc/launch.hpp", "global_attention_mimo_amd/build.py"]
def is_ga_prefill(short: str) -> bool:
    """The GA (non-chunked, bf16) instantiation of prefill_kernel: template
    arguments <waves, blocks, keys, SWA=false, waves per SIMD, then every
    remaining flag (chunked, paged, FP8, ...) false>."""
    if not short.startswith("prefill_kernel<") or not short.endswith(">"):
        return False
    args = [a.strip() for a in short[len("prefill_kernel<"):-1].split(",")]
    return len(args) >= 6 and args[3] == "false" and all(a == "false" for a in args[5:])


# -- names and numbers -------------------------------------------------------

def short_name(name: str) -> str:
    """Kernel name without return type, namespaces and argument list:
    'void mimo::(anonymous namespace)::ga_split_kernel<false>(unsigned ...)' -> 'ga_split_kernel<false>'."""
    n = name.strip()
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):  # the argument list is the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
            break
    n = n[:cut]
    n = re.sub(r"^void\s+", "", n)
    n = n.replace("(anonymous namespace)::", "")
    n = re.sub(r"^(mimo|at::native|at::native::\w+)::", "", n)
    return n.strip()


def is_library_kernel(name: str) -> bool:
    return "mimo::" in name


def code_digest(paths: Iterable[str], root: str = ROOT) -> str:
    """sha256 of the given sources with comments and whitespace removed (a record
    stays valid across comment edits, not across any change to the code)."""
    h = hashlib.sha256()
    for src in paths:
        text = open(os.path.join(root, src), encoding="utf-8").read()
        if src.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
        else:
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()


# -- running rocprofv3 ---------------------------------------------------------

def pass_command(suite: str, which: str, out: str, python: str = sys.executable) -> List[str]:
    trace_args, pmc_args = SUITES[suite]
    bench_args = shlex.split(trace_args if which == "trace" else pmc_args)
    if which != "trace" and "--copy-calibration" not in bench_args:
        bench_args.append("--copy-calibration")
    return (["rocprofv3", *PASSES[which], "--output-format", "csv", "-d", os.path.join(out, which), "-o", "run",
             "--", python, os.path.join(ROOT, "bench.py"), *bench_args])


def run(suite: str, out: str, passes: Iterable[str] = ("trace", "fetch", "write", "mfma", "stalls")) -> None:
    """Runs the profiler passes one after another (each under its own time limit,
    output to <out>/<pass>.log); stops at the first pass that fails."""
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
    for which in passes:
        cmd = pass_command(suite, which, out)
        print(f"[prof] {suite}/{which}: {' '.join(shlex.quote(c) for c in cmd)}", flush=True)
        t0 = time.time()
        with open(os.path.join(out, f"{which}.log"), "w") as log:
            try:
                rc = subprocess.run(cmd, stdout=log, stderr=subprocess.STDOUT, env=env,
                                    timeout=PASS_LIMIT_S[which]).returncode
            except subprocess.TimeoutExpired:
                rc = 124
        print(f"[prof] {suite}/{which}: exit {rc} after {time.time() - t0:.0f} s", flush=True)
        if rc != 0:
            raise SystemExit(f"rocprofv3 pass {which} failed with status {rc} (see {out}/{which}.log)")


# -- reading its output ------------------------------------------------------

def _csv_rows(directory: str, suffix: str) -> List[dict]:
    rows: List[dict] = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def trace_stats(rows: List[dict]) -> Dict[str, dict]:
    """Per kernel (full name): dispatch count and duration statistics in us,
    from kernel-trace rows (Start_Timestamp / End_Timestamp in ns)."""
    per: Dict[str, List[float]] = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(r["Kernel_Name"], []).append(d)
    return {k: {"dispatches": len(v), "median_us": statistics.median(v), "avg_us": sum(v) / len(v),
                "min_us": min(v), "max_us": max(v), "total_ms": sum(v) / 1e3} for k, v in per.items()}


def counter_values(rows: List[dict], counter: str) -> Dict[str, List[float]]:
    """Per kernel (full name), the counter's value of each dispatch, in dispatch
    order (rows of one dispatch and counter are summed)."""
    per: Dict[str, Dict[int, float]] = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], {})
        did = int(r["Dispatch_Id"])
        per[r["Kernel_Name"]][did] = per[r["Kernel_Name"]].get(did, 0.0) + float(r["Counter_Value"])
    return {k: [v[d] for d in sorted(v)] for k, v in per.items()}


def _copy_dispatches(rows: List[dict], counter: str) -> List[float]:
    """The counter's value for each device-copy dispatch, in dispatch order."""
    per: Dict[int, float] = {}
    for r in rows:
        if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower():
            did = int(r["Dispatch_Id"])
            per[did] = per.get(did, 0.0) + float(r["Counter_Value"])
    return [per[d] for d in sorted(per)]


def calibration_scales(fetch_rows: List[dict], write_rows: List[dict],
                       known_kib: float = CALIBRATION_BYTES / 1024) -> tuple:
    """(fetch_scale, write_scale) from the calibration copy: of the device copies
    of the run (the same, in the same order, in both passes), the one whose
    WRITE_SIZE is nearest its known 1 GiB; each scale is the known KiB over what
    the counter read for that dispatch."""
    fc, wc = _copy_dispatches(fetch_rows, "FETCH_SIZE"), _copy_dispatches(write_rows, "WRITE_SIZE")
    if not wc or len(fc) != len(wc):
        raise ValueError(f"calibration copy not found (copies counted: fetch {len(fc)}, write {len(wc)})")
    i = min(range(len(wc)), key=lambda j: abs(wc[j] - known_kib))
    if not (0.5 * known_kib < wc[i] < 2.0 * known_kib) or fc[i] <= 0:
        raise ValueError(f"no copy near {known_kib:.0f} KiB among the counted dispatches")
    return known_kib / fc[i], known_kib / wc[i]


def mfma_busy(busy_cycles: float, grbm_active: float, simds: int = SIMDS, xcds: int = XCDS) -> float:
    return busy_cycles / (simds * grbm_active / xcds) if grbm_active > 0 else 0.0


# -- reports -----------------------------------------------------------------

def _mean(v: List[float]) -> float:
    return sum(v) / len(v) if v else 0.0


def summarize(out: str) -> dict:
    """Everything the report needs, from the CSV files of the passes under out/."""
    res: dict = {"trace": trace_stats(_csv_rows(os.path.join(out, "trace"), "kernel_trace.csv"))}
    fetch_rows = _csv_rows(os.path.join(out, "fetch"), "counter_collection.csv")
    write_rows = _csv_rows(os.path.join(out, "write"), "counter_collection.csv")
    if fetch_rows and write_rows:
        f, w = counter_values(fetch_rows, "FETCH_SIZE"), counter_values(write_rows, "WRITE_SIZE")
        fs, ws = calibration_scales(fetch_rows, write_rows)
        res["traffic"] = {"fetch_scale": fs, "write_scale": ws, "kernels": {
            k: {"dispatches": len(f[k]), "fetch_kib": _mean(f[k]), "write_kib": _mean(w.get(k, [])),
                "read_bytes": _mean(f[k]) * 1024 * fs, "write_bytes": _mean(w.get(k, [])) * 1024 * ws}
            for k in f if is_library_kernel(k)}}
    mrows = _csv_rows(os.path.join(out, "mfma"), "counter_collection.csv")
    if mrows:
        busy = counter_values(mrows, "SQ_VALU_MFMA_BUSY_CYCLES")
        insts = counter_values(mrows, "SQ_INSTS_MFMA")
        grbm = counter_values(mrows, "GRBM_GUI_ACTIVE")
        res["mfma"] = {}
        for k in busy:
            if not is_library_kernel(k):
                continue
            g = _mean(grbm.get(k, []))
            med = res["trace"].get(k, {}).get("median_us")
            res["mfma"][k] = {"insts_mfma": _mean(insts.get(k, [])), "busy": mfma_busy(_mean(busy[k]), g),
                              "clock_ghz": (g / XCDS) / (med * 1e3) if med and med > 50 else None}
    srows = _csv_rows(os.path.join(out, "stalls"), "counter_collection.csv")
    if srows:
        vals = {c: counter_values(srows, c) for c in STALL_COUNTERS}
        res["stalls"] = {}
        for k, cyc in vals["SQ_WAVE_CYCLES"].items():
            if not is_library_kernel(k) or _mean(cyc) <= 0:
                continue
            w = _mean(cyc)
            res["stalls"][k] = {"wave_cycles": w, **{c: _mean(vals[c].get(k, [])) / w for c in STALL_COUNTERS[1:]}}
    return res


def _fmt(x: Optional[float], spec: str) -> str:
    return "-" if x is None else format(x, spec)


def write_markdown(suite: str, out: str, res: dict, path: str) -> None:
    cmds = [" ".join(shlex.quote(c) for c in pass_command(suite, w, "<out>", "python3")) for w in PASSES]
    cmds = [c.replace(os.path.join(ROOT, "bench.py"), "bench.py") for c in cmds]
    lib = {k: v for k, v in res["trace"].items() if is_library_kernel(k)}
    L = [f"# rocprofv3 summary: {TITLES[suite]} (MI355X, gfx950)", "", f"Workload: {WORKLOADS[suite]}", "",
         "Made by `python -m global_attention_mimo_amd.prof run --suite " + suite + " --out <out>` and "
         "`python -m global_attention_mimo_amd.prof report --suite " + suite + " --out <out>`, run from the "
         "repository root on the GPU box after `cd /tmp && export TMPDIR=/tmp`; the passes it runs:", "", "```",
         *cmds, "```", "", "## Kernel durations (kernel trace, every dispatch of the run)", "",
         "| kernel | dispatches | median us | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|---|"]
    for k, v in sorted(lib.items(), key=lambda kv: -kv[1]["total_ms"]):
        L.append(f"| `{short_name(k)}` | {v['dispatches']} | {v['median_us']:.2f} | {v['avg_us']:.2f} | "
                 f"{v['min_us']:.2f} | {v['max_us']:.2f} | {v['total_ms']:.2f} |")
    if "traffic" in res:
        t = res["traffic"]
        L += ["", "## HBM-side bytes per dispatch (mean over the dispatches of the FETCH_SIZE and WRITE_SIZE passes)",
              "", f"Calibration: the 1 GiB device copy scales FETCH_SIZE by {t['fetch_scale']:.4f} and WRITE_SIZE "
              f"by {t['write_scale']:.4f} (bytes per counted KiB / 1024).", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read GB | scaled write GB |",
              "|---|---|---|---|---|---|"]
        for k, v in sorted(t["kernels"].items(), key=lambda kv: -kv[1]["read_bytes"]):
            L.append(f"| `{short_name(k)}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | "
                     f"{v['read_bytes'] / 1e9:.3f} | {v['write_bytes'] / 1e9:.3f} |")
    if "mfma" in res:
        L += ["", "## Matrix-core activity per dispatch", "",
              f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GRBM_GUI_ACTIVE / {XCDS} XCDs); effective "
              "clock = (GRBM_GUI_ACTIVE / 8) / the kernel's median duration above (kernels under 50 us: -).", "",
              "| kernel | SQ_INSTS_MFMA | MFMA busy | effective clock GHz |", "|---|---|---|---|"]
        for k, v in sorted(res["mfma"].items(), key=lambda kv: -kv[1]["insts_mfma"]):
            L.append(f"| `{short_name(k)}` | {v['insts_mfma']:.0f} | {100 * v['busy']:.1f}% | "
                     f"{_fmt(v['clock_ghz'], '.2f')} |")
    if res.get("stalls"):
        L += ["", "## Where the waves' cycles go (fractions of SQ_WAVE_CYCLES per dispatch)", "",
              "Per-wave cycles (several waves share a SIMD, so these are not SIMD time): waiting on dependencies "
              "(SQ_WAIT_ANY: loads, LDS, barriers), ready but not issued (SQ_WAIT_INST_ANY: the unit it needs is "
              "busy -- the matrix core, the memory pipeline -- or another wave issues), and issuing "
              "(SQ_ACTIVE_INST_ANY), the last split by kind (VALU includes MFMA).", "",
              "| kernel | waiting on data | ready, not issued | issuing | VALU+MFMA | LDS | VMEM | other |",
              "|---|---|---|---|---|---|---|---|"]
        for k, v in sorted(res["stalls"].items(), key=lambda kv: -kv[1]["wave_cycles"]):
            L.append(f"| `{short_name(k)}` | {100 * v['SQ_WAIT_ANY']:.1f}% | {100 * v['SQ_WAIT_INST_ANY']:.1f}% | "
                     f"{100 * v['SQ_ACTIVE_INST_ANY']:.1f}% | {100 * v['SQ_ACTIVE_INST_VALU']:.1f}% | "
                     f"{100 * v['SQ_ACTIVE_INST_LDS']:.1f}% | {100 * v['SQ_ACTIVE_INST_VMEM']:.1f}% | "
                     f"{100 * v['SQ_ACTIVE_INST_MISC']:.1f}% |")
    with open(path, "w") as f:
        f.write("\n".join(L) + "\n")


def write_traffic_record(res: dict, path: str, suite: str = "step") -> Optional[dict]:
    """The GA prefill launch's calibrated HBM bytes, keyed by the digest of its sources."""
    kern = next((k for k in res.get("traffic", {}).get("kernels", {}) if is_ga_prefill(short_name(k))), None)
    if kern is None:
        return None
    t = res["traffic"]
    v = t["kernels"][kern]
    cmds = [" ".join(shlex.quote(c) for c in pass_command(suite, w, "<out>", "python3")).replace(
        os.path.join(ROOT, "bench.py"), "bench.py") for w in ("fetch", "write")]
    rec = {"kernel": "prefill_kernel<GA> (GA prefill, 1 x 32768 tokens, 64q/4kv heads, d 192/128)",
           "sources": TRAFFIC_SOURCES, "code_sha256": code_digest(TRAFFIC_SOURCES),
           "fetch_kib": v["fetch_kib"], "write_kib": v["write_kib"], "fetch_scale": t["fetch_scale"],
           "write_scale": t["write_scale"], "read_bytes": v["read_bytes"], "write_bytes": v["write_bytes"],
           "commands": cmds}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


REPORTS = {"step": "profiles/hot_path_bench_step.md", "hybrid": "profiles/hybrid_stack_48_layers.md",
           "next-rows": "profiles/next_rows_chunk_paged_fp8_backward.md"}


def report(suite: str, out: str, md: Optional[str] = None) -> dict:
    res = summarize(out)
    write_markdown(suite, out, res, md or os.path.join(ROOT, REPORTS[suite]))
    if suite == "step":
        write_traffic_record(res, os.path.join(ROOT, "profiles/prefill_ga_1x32768_traffic.json"))
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("action", choices=("run", "report", "all"))
    ap.add_argument("--suite", choices=tuple(SUITES), default="step")
    ap.add_argument("--out", required=True, help="directory for the profiler output (e.g. under gpurun_out/)")
    ap.add_argument("--passes", default="trace,fetch,write,mfma,stalls")
    ap.add_argument("--md", default=None, help="markdown summary path (default: the suite's file under profiles/)")
    a = ap.parse_args(argv)
    if a.action in ("run", "all"):
        run(a.suite, a.out, [p for p in a.passes.split(",") if p])
    if a.action in ("report", "all"):
        report(a.suite, a.out, a.md)
        print(f"[prof] wrote {a.md or REPORTS[a.suite]}", flush=True)


if __name__ == "__main__":
    main()
