"""rocprofv3 harness for bench.py: kernel times, HBM bytes and MFMA utilisation per kernel.

For each workload it runs bench.py under rocprofv3 in separate passes (this
process never touches the GPU itself):

    trace   --kernel-trace --stats              steady-state time per kernel
    fetch   --pmc FETCH_SIZE                    HBM bytes read (KiB per dispatch)
    write   --pmc WRITE_SIZE                    HBM bytes written
    mfma    --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16
                                                MFMA busy cycles over GPU-active
                                                cycles x SIMDs (%), bf16 MFMA flops

The fetch and write passes also time a 1 GiB device copy (bench.py
--calib-copy-mib 1024); each counter is scaled by the ratio of the copy's known
bytes to what the counter reads for it.  Per kernel, the last dispatches of the
run count: as many as bench.py times (one per step of the stream and append
workloads, every call of the CLCES workload), so a stream pass reads the full
72-frame cache only.  The summary goes to profiles/kernels_<workload>.json
(and beside the raw output), which bench.py reads for the traffic and MFMA
fields of its roofline (only while the kernel sources still hash as
recorded).

The CLCES workload gets the trace pass only, with the rank history (clces)
and with every window layer ranked in every step (clces_rerank): its
FETCH_SIZE pass went silent for minutes where every other pass ends in
seconds, with no cause found, so no counter pass is run on it.  The diversity
and token-budget stacks also get the trace pass only, over every dispatch of
their last 10 frames (found from a kernel that runs a fixed number of times
per frame).

    python profile_bench.py [--workloads stream,append,clces,clces_rerank,diversity,budget] [--out gpurun_out/prof]
    python profile_bench.py --parse-only ...    # rebuild the summaries from existing output
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "bounded_kv_cache_stream_amd", "csrc")
SOURCES = ["attend.hip", "pages.hip", "clces.hip", "diversity.hip"]
CALIB_MIB = 1024
COPY_KERNEL = "__amd_rocclr_copyBuffer"

WORKLOADS = {
    # bench.py arguments of each workload; steps None: bench.py's fixed call count (all dispatches count).
    # The MFMA pass is taken where MFMA kernels run.
    "stream": {"args": ["--no-cpu-baseline"], "trace_steps": 30, "pmc_steps": 10, "pmc": True, "mfma": True},
    "append": {"args": ["--workload", "append", "--no-cpu-baseline"], "trace_steps": 30, "pmc_steps": 10,
               "pmc": True, "mfma": False},
    "clces": {"args": ["--workload", "clces", "--no-cpu-baseline", "--reuse-ranks"], "trace_steps": None, "pmc_steps": None,
              "pmc": False, "mfma": False},
    # the same calls with every window layer ranked in every step
    "clces_rerank": {"args": ["--workload", "clces", "--no-cpu-baseline", "--no-reuse-ranks"], "trace_steps": None,
                     "pmc_steps": None, "pmc": False, "mfma": False},
    # the stacks: every dispatch from the start of the last trace_steps frames (found from a kernel that runs
    # `per_step` times a frame) counts
    "diversity": {"args": ["--workload", "diversity", "--no-cpu-baseline"], "trace_steps": 10, "pmc_steps": None,
                  "pmc": False, "mfma": False, "marker": "append_layers_kernel", "per_step": 1},
    "budget": {"args": ["--workload", "budget", "--no-cpu-baseline"], "trace_steps": 10, "pmc_steps": None,
               "pmc": False, "mfma": False, "marker": "append_kernel", "per_step": 24},
}


def source_hashes() -> dict:
    out = {}
    for s in SOURCES:
        with open(os.path.join(CSRC, s), "rb") as f:
            out[s] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


def run_pass(name: str, out_dir: str, prof_args: list, bench_args: list, limit: int, parse_only: bool) -> str:
    """One rocprofv3 run (its output goes straight to <name>.log); returns its output directory."""
    d = os.path.join(out_dir, name)
    if parse_only:
        return d
    cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *prof_args, "-T", "-f", "csv", "-d", d, "-o", "run",
           "--", sys.executable, "-u", os.path.join(ROOT, "bench.py"), *bench_args]
    print("[profile]", " ".join(cmd), flush=True)
    t0 = time.time()
    with open(d + ".log", "w") as log:
        r = subprocess.run(cmd, cwd="/tmp", stdout=log, stderr=subprocess.STDOUT)
    # rocprofv3 may end with a signal of its own after the program's last line; the CSVs decide
    if not glob.glob(os.path.join(d, "**", "*.csv"), recursive=True):
        raise RuntimeError(f"{name}: no rocprofv3 output (exit {r.returncode}); see {d}.log")
    print(f"[profile] {name} done in {time.time() - t0:.1f} s (exit {r.returncode})", flush=True)
    return d


def read_csv(d: str, suffix: str) -> list:
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    rows = []
    for fn in files:
        with open(fn) as f:
            rows.extend(csv.DictReader(f))
    return rows


def last(values: list, n) -> list:
    """The last n values (all of them for n None)."""
    return values if n is None else values[-n:]


def kernel_times(d: str, n, marker=None, per_step=1) -> dict:
    """Per kernel name: mean and min/max duration (us) over its last n dispatches, from the kernel trace; with a
    marker kernel, over every dispatch that starts at or after the marker's (n * per_step)-th last dispatch."""
    by = {}
    for r in read_csv(d, "kernel_trace.csv"):
        by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    t_from = None
    if marker:
        starts = sorted(s for k, v in by.items() if marker in k for s, _ in v)
        t_from = starts[-n * per_step] if len(starts) >= n * per_step else starts[0]
    out = {}
    for k, v in by.items():
        v.sort()
        sel = [x for x in v if x[0] >= t_from] if t_from is not None else last(v, n)
        if not sel:
            continue
        dur = [(e - s) / 1e3 for s, e in sel]
        out[k] = {"dispatches": len(v), "used": len(dur), "avg_us": sum(dur) / len(dur), "min_us": min(dur),
                  "max_us": max(dur)}
    return out


def counter_means(d: str, n) -> dict:
    """Per kernel name and counter: mean over its last n dispatches."""
    by = {}
    for r in read_csv(d, "counter_collection.csv"):
        by.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(
            (int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    out = {}
    for (k, c), v in by.items():
        v.sort()
        vals = [x for _, x in last(v, n)]
        out.setdefault(k, {})[c] = sum(vals) / len(vals)
    return out


def profile(workload: str, out_dir: str, parse_only: bool = False) -> dict:
    w = WORKLOADS[workload]
    steps = lambda n: ["--steps", str(n)] if n else []  # noqa: E731
    base = [*w["args"]]
    commands = []
    targs = base + steps(w["trace_steps"])
    t = run_pass(f"{workload}_trace", out_dir, ["--kernel-trace", "--stats"], targs, 600, parse_only)
    commands.append("rocprofv3 --kernel-trace --stats -- python3 bench.py " + " ".join(targs))
    times = kernel_times(t, w["trace_steps"], w.get("marker"), w.get("per_step", 1))
    f, wr, m, calib = {}, {}, {}, None
    n = w["pmc_steps"]
    if w["pmc"]:
        pmc_args = base + steps(n) + ["--calib-copy-mib", str(CALIB_MIB)]
        f = counter_means(run_pass(f"{workload}_fetch", out_dir, ["--pmc", "FETCH_SIZE"], pmc_args, 300, parse_only), n)
        commands.append("rocprofv3 --pmc FETCH_SIZE -- python3 bench.py " + " ".join(pmc_args))
        wr = counter_means(run_pass(f"{workload}_write", out_dir, ["--pmc", "WRITE_SIZE"], pmc_args, 300, parse_only),
                           n)
        commands.append("rocprofv3 --pmc WRITE_SIZE -- python3 bench.py " + " ".join(pmc_args))
        calib_bytes = CALIB_MIB * 1024 * 1024
        calib = {"copy_bytes": calib_bytes,
                 "fetch_factor": calib_bytes / (f[COPY_KERNEL]["FETCH_SIZE"] * 1024),
                 "write_factor": calib_bytes / (wr[COPY_KERNEL]["WRITE_SIZE"] * 1024),
                 "fetch_kib_raw": f[COPY_KERNEL]["FETCH_SIZE"], "write_kib_raw": wr[COPY_KERNEL]["WRITE_SIZE"]}
    if w["mfma"]:
        margs = base + steps(n)
        m = counter_means(run_pass(f"{workload}_mfma", out_dir, ["--pmc", "MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16"],
                                   margs, 300, parse_only), n)
        commands.append("rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 -- python3 bench.py " + " ".join(margs))
    kernels = {}
    for k, tv in times.items():
        if k == COPY_KERNEL or "elementwise" in k:
            continue  # the calibration copy and torch's input generators
        e = dict(tv)
        if k in f:
            e["fetch_kib_raw"] = f[k]["FETCH_SIZE"]
            e["fetch_bytes"] = f[k]["FETCH_SIZE"] * 1024 * calib["fetch_factor"]
        if k in wr:
            e["write_kib_raw"] = wr[k]["WRITE_SIZE"]
            e["write_bytes"] = wr[k]["WRITE_SIZE"] * 1024 * calib["write_factor"]
        if k in m:
            e["mfma_util_pct"] = m[k].get("MfmaUtil")
            mops = m[k].get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
            e["mfma_flops_bf16"] = None if mops is None else mops * 512
        kernels[k] = e
    return {"workload": workload, "source_sha256_16": source_hashes(), "commands": commands,
            "dispatches_used": ("every dispatch of the last %d frames" % w["trace_steps"]) if w.get("marker") else
            "last %s per kernel" % (w["trace_steps"] or "all") if not w["pmc"] else
            "last %s per kernel (trace), last %s (counters)" % (w["trace_steps"], n),
            "calibration": calib, "counters": "not collected" if not w["pmc"] else "FETCH_SIZE, WRITE_SIZE"
            + (", MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16" if w["mfma"] else ""), "kernels": kernels}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="stream,append,clces")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--parse-only", action="store_true", help="summarise existing output; run nothing")
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)
    for wl in args.workloads.split(","):
        rec = profile(wl, args.out, args.parse_only)
        for path in (os.path.join(args.profiles, f"kernels_{wl}.json"), os.path.join(args.out, f"kernels_{wl}.json")):
            with open(path, "w") as fh:
                json.dump(rec, fh, indent=1, sort_keys=True)
            print(f"[profile] wrote {path}", flush=True)
        print(f"| kernel | dispatches | steady avg (us) | fetch (MB) | write (MB) | MFMA busy (%) |")
        for k, e in sorted(rec["kernels"].items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["used"]):
            fb = e.get("fetch_bytes")
            wb = e.get("write_bytes")
            mu = e.get("mfma_util_pct")
            print(f"| {k[:60]} | {e['dispatches']} | {e['avg_us']:.2f} | "
                  f"{'' if fb is None else f'{fb / 1e6:.1f}'} | {'' if wb is None else f'{wb / 1e6:.1f}'} | "
                  f"{'' if mu is None else f'{mu:.1f}'} |", flush=True)


if __name__ == "__main__":
    main()
