"""Summaries of rocprofv3 output for the block's kernels.

    python -m video_diffusion_transformer_03_amd.profile_summary \
        --ktrace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --workload block_l16384 --steps 5 --cmd "..." --out profiles

Reads the CSV files rocprofv3 writes (`--output-format csv`):
  - kernel-trace (`*_kernel_stats.csv`): per-kernel count and average duration;
  - `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of the same command (`*_counter_collection.csv`,
    KiB per dispatch);
  - the same two counters on a plain device copy of known size (bench.py --copy-calibration: 2 x 1 GiB),
    which gives the factor each counter's KiB must be scaled by to read true bytes.
Writes `profiles/kernels_<workload>.txt` (durations, HBM bytes per launch) and
`profiles/traffic.json` (per-kernel HBM bytes per launch, with a hash of the kernel sources
so a later change to a kernel marks its numbers stale).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))

# kernel kind -> (source file, substring of the mangled kernel name, extra selector)
KINDS = {
    "attention": ("k_attn.hip", "attn_bf16_kernel"),
    "gemm": ("k_gemm.hip", "gemm_pp_kernel"),
    "rows": ("k_rows.hip", "row_kernel"),
    "adaln": ("k_rows.hip", "adaln_kernel"),
}


def source_hash(fname: str) -> str:
    data = open(os.path.join(HERE, "csrc", fname), "rb").read()
    return hashlib.sha256(data).hexdigest()[:16]


def short_name(name: str) -> str:
    m = re.search(r"h3k::(\w+)<([^>]*)>", name)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.search(r"h3k::(\w+)", name)
    return m.group(1) if m else name[:60]


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(d: str):
    out = {}
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))):
        out[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"]))
    return out


def counter_by_kernel(d: str, counter: str):
    """{(kernel name, grid size): mean counter value per dispatch}"""
    acc = defaultdict(list)
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] == counter:
            acc[(r["Kernel_Name"], r["Grid_Size"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def copy_factor(d: str, counter: str, bytes_per_copy: float) -> float:
    vals = [v for (k, _), v in counter_by_kernel(d, counter).items() if "copyBuffer" in k or "copy" in k.lower()]
    if not vals:
        raise RuntimeError(f"no copy kernel found in {d}")
    return bytes_per_copy / (max(vals) * 1024.0)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--ktrace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--workload", required=True)
    ap.add_argument("--steps", type=int, required=True, help="timed steps of the profiled run")
    ap.add_argument("--cmd", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", default="profiles")
    a = ap.parse_args()

    stats = kernel_stats(a.ktrace)
    fetch = counter_by_kernel(a.fetch, "FETCH_SIZE")
    write = counter_by_kernel(a.write, "WRITE_SIZE")
    ff = copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    fw = copy_factor(a.copy_write, "WRITE_SIZE", a.copy_bytes)

    lines = [f"# Kernel durations and HBM traffic per launch, workload {a.workload}", "",
             "Commands:", *[f"    {c}" for c in a.cmd.split(" ;; ")], "",
             f"Copy calibration (plain 1 GiB device copy): FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f}", "",
             f"{'kernel':58s} {'calls':>6s} {'avg us':>10s} {'read MB':>9s} {'write MB':>9s}"]
    traffic = {"workload": a.workload, "copy_factor": {"fetch": ff, "write": fw},
               "sources": {f: source_hash(f) for f, _ in KINDS.values()}, "kernels": {}}
    rows = []
    for name, (calls, avg_ns, tot_ns) in stats.items():
        if "h3k::" not in name:
            continue
        f_kib = [v for (k, _), v in fetch.items() if k == name]
        w_kib = [v for (k, _), v in write.items() if k == name]
        rd = max(f_kib) * 1024 * ff if f_kib else float("nan")
        wr = max(w_kib) * 1024 * fw if w_kib else float("nan")
        rows.append((tot_ns, name, calls, avg_ns, rd, wr))
    for tot_ns, name, calls, avg_ns, rd, wr in sorted(rows, reverse=True):
        lines.append(f"{short_name(name)[:58]:58s} {calls:6d} {avg_ns / 1e3:10.1f} {rd / 1e6:9.1f} {wr / 1e6:9.1f}")
        for kind, (src, key) in KINDS.items():
            if key in name:
                traffic["kernels"].setdefault(short_name(name), {"kind": kind, "source": src,
                                                                 "read_bytes": rd, "write_bytes": wr,
                                                                 "avg_us": avg_ns / 1e3})
    os.makedirs(a.out, exist_ok=True)
    open(os.path.join(a.out, f"kernels_{a.workload}.txt"), "w").write("\n".join(lines) + "\n")
    json.dump(traffic, open(os.path.join(a.out, "traffic.json"), "w"), indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
