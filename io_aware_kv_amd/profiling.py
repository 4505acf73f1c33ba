"""Summaries of rocprofv3 output for the committed profile records.

Reads the CSV files that ``rocprofv3 --output-format csv`` writes (kernel
statistics of a ``--kernel-trace --stats`` run, per-dispatch counters of a
``--pmc`` run) and turns them into the short text summaries kept in
``profiles/`` and into ``profiles/counters.json``, which bench.py reads to
report measured HBM traffic next to the algorithmic bytes.

  python -m io_aware_kv_amd.profiling stats DIR --command "..." --out FILE
  python -m io_aware_kv_amd.profiling counters --workload NAME --fetch DIR --write DIR \
      --copy-fetch DIR --copy-write DIR --copy-bytes N
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = {
    "attn_mfma": os.path.join(ROOT, "io_aware_kv_amd", "csrc", "attn_mfma.hip"),
    "attn_combine": os.path.join(ROOT, "io_aware_kv_amd", "csrc", "attn_mfma.hip"),
    "proj_mfma": os.path.join(ROOT, "io_aware_kv_amd", "csrc", "proj_mfma.hip"),
    "attn_generic": os.path.join(ROOT, "io_aware_kv_amd", "csrc", "generic_kernels.hip"),
    "proj_generic": os.path.join(ROOT, "io_aware_kv_amd", "csrc", "generic_kernels.hip"),
}


def src_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _find(dirpath: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, dirpath))
    return hits[0]


def kernel_stats(dirpath: str):
    """Rows of the kernel statistics: name, calls, average/min/max in us."""
    rows = []
    with open(_find(dirpath, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3,
                         "percent": float(r.get("Percentage", 0.0))})
    return rows


def counter_per_kernel(dirpath: str, counter: str):
    """Mean value of one counter per kernel name over its dispatches."""
    acc = defaultdict(list)
    with open(_find(dirpath, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def short_name(name: str) -> str:
    name = name.replace("fdllm::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(fdllm::")[0]


def write_stats_summary(dirpath: str, command: str, out: str, title: str):
    rows = kernel_stats(dirpath)
    lines = ["# %s" % title, "",
             "Command (from the repository root on one MI355X):", "", "    " + command, "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.1f |" % (short_name(r["name"]), r["calls"], r["avg_us"],
                                                                    r["min_us"], r["max_us"], r["percent"]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_workload_summary(workload: str, title: str, trace_dir: str, trace_cmd: str, fetch_dir: str,
                           write_dir: str, pmc_cmd: str, out: str):
    """One workload's kernel times and per-launch HBM traffic (calibrated)."""
    with open(COUNTERS_JSON) as f:
        cal = json.load(f)["calibration"]
    rows = kernel_stats(trace_dir)
    fetch = counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = counter_per_kernel(write_dir, "WRITE_SIZE")
    lines = ["# %s" % title, "",
             "Kernel trace (`rocprofv3 --kernel-trace --stats`), from the repository root on one MI355X:", "",
             "    " + trace_cmd, "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f |" % (short_name(r["name"]), r["calls"], r["avg_us"],
                                                              r["min_us"], r["max_us"]))
    if any(r["name"].startswith("__amd_rocclr") for r in rows):
        lines += ["", "`__amd_rocclr_*` are the runtime's own copy and fill kernels that load the seeded "
                      "inputs and caches into the buffer sets, outside the timed steps."]
    lines += ["", "HBM traffic per launch from two counter passes (`FETCH_SIZE`, then `WRITE_SIZE`, KiB per "
              "dispatch), each scaled by what the same counter reads for a plain 1 GiB device copy "
              "(fetch x%.4f, write x%.4f):" % (cal["fetch_factor"], cal["write_factor"]), "",
              "    " + pmc_cmd.replace("COUNTER", "FETCH_SIZE"), "    " + pmc_cmd.replace("COUNTER", "WRITE_SIZE"), "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated MB read | calibrated MB written |",
              "|---|---|---|---|---|---|"]
    for k, (v, n) in sorted(fetch.items()):
        if "fdllm" not in k:
            continue
        wv = write.get(k, (0.0, 0))[0]
        lines.append("| `%s` | %d | %.0f | %.0f | %.2f | %.2f |" % (short_name(k), n, v, wv,
                                                                    v * 1024 * cal["fetch_factor"] / 1e6,
                                                                    wv * 1024 * cal["write_factor"] / 1e6))
    lines += ["", "Workload key in counters.json: `%s`." % workload]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def update_counters(workload: str, fetch_dir: str, write_dir: str, copy_fetch: str, copy_write: str,
                    copy_bytes: int, commands: dict):
    cf = counter_per_kernel(copy_fetch, "FETCH_SIZE")
    cw = counter_per_kernel(copy_write, "WRITE_SIZE")
    # the copy kernel is the largest reader of the calibration run
    copy_kib_f = max(v for v, _ in cf.values())
    copy_kib_w = max(v for v, _ in cw.values())
    cal = {"copy_bytes": copy_bytes,
           "copy_fetch_kib": copy_kib_f, "copy_write_kib": copy_kib_w,
           "fetch_factor": copy_bytes / 1024.0 / copy_kib_f,
           "write_factor": copy_bytes / 1024.0 / copy_kib_w}
    data = {"calibration": cal, "kernels": {}, "commands": {}}
    if os.path.exists(COUNTERS_JSON):
        with open(COUNTERS_JSON) as f:
            old = json.load(f)
        data["kernels"] = old.get("kernels", {})
        data["commands"] = old.get("commands", {})
    data["calibration"] = cal
    fetch = counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = counter_per_kernel(write_dir, "WRITE_SIZE")
    for key, path in KERNEL_SOURCES.items():
        # the step's launches of this kernel (the prefill launch of the
        # projection uses another tile and appears under its own name)
        names = [n for n in fetch if key + "_kernel" in n]
        if key == "proj_mfma" and len(names) > 1:
            names = [n for n in names if fetch[n][1] == max(fetch[m][1] for m in names)]
        if not names:
            continue
        name = max(names, key=lambda n: fetch[n][1])
        ent = {"kernel": short_name(name), "fetch_kib": fetch[name][0], "write_kib": write.get(name, (0.0, 0))[0],
               "dispatches": fetch[name][1], "src_hash": src_hash(path)}
        data["kernels"].setdefault(key, {})[workload] = ent
    data["commands"].update(commands)
    with open(COUNTERS_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command", action="append", default=[], help="name=command, recorded with the figures")
    w = sub.add_parser("summary")
    w.add_argument("--workload", required=True)
    w.add_argument("--title", required=True)
    w.add_argument("--trace", required=True)
    w.add_argument("--trace-cmd", required=True)
    w.add_argument("--fetch", required=True)
    w.add_argument("--write", required=True)
    w.add_argument("--pmc-cmd", required=True)
    w.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.cmd == "stats":
        write_stats_summary(a.dir, a.command, a.out, a.title)
    elif a.cmd == "summary":
        write_workload_summary(a.workload, a.title, a.trace, a.trace_cmd, a.fetch, a.write, a.pmc_cmd, a.out)
    else:
        cmds = dict(x.split("=", 1) for x in a.command)
        update_counters(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, cmds)


if __name__ == "__main__":
    main()
