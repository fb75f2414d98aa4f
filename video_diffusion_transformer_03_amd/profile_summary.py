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
Writes `profiles/kernels_<name>.txt` (durations, time per step, HBM bytes per launch;
<name> defaults to the workload) and, unless --no-traffic, `profiles/traffic.json` (per-kernel HBM bytes per launch, with a hash of the kernel sources
so a later change to a kernel marks its numbers stale).

With --sq DIR (a `--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY
SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE` run of the same command)
it also writes `profiles/sq_<name>.txt`: per kernel the fraction of SIMD cycles the matrix
cores were busy, the fraction of wave time spent waiting, LDS bank-conflict cycles per LDS
instruction and LDS-active cycles per CU cycle.
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
    "attention": ("k_attn.hip", "attn_v2_kernel"),
    "gemm": ("k_gemm.hip", "gemm_"),
    "rows": ("k_rows.hip", "row_kernel"),
    "adaln": ("k_rows.hip", "adaln_kernel"),
}


def source_hash(fname: str) -> str:
    data = open(os.path.join(HERE, "csrc", fname), "rb").read()
    return hashlib.sha256(data).hexdigest()[:16]


# template arguments in mangled names the profiler leaves undemangled (it does not know
# _Float16, "DF16_"): integer literals, bool literals and the types used here
_MANGLED_ARGS = [(r"Li(-?\d+)E", r"\1"), (r"Lb0E", "false"), (r"Lb1E", "true"),
                 (r"DF16_", "_Float16"), (r"^t", "unsigned short"), (r"^f", "float")]


def _demangle_args(args: str) -> str:
    out = []
    while args:
        for pat, rep in _MANGLED_ARGS:
            m = re.match(pat if pat.startswith("^") else "^" + pat, args)
            if m:
                out.append(m.expand(rep))
                args = args[m.end():]
                break
        else:
            out.append(args)
            break
    return ", ".join(out)


def short_name(name: str) -> str:
    m = re.search(r"h3k::(\w+)<([^>]*)>", name)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.match(r"_ZN3h3k\d+(\w+?)I(.*?)EEEv", name)
    if m:  # a mangled h3k kernel
        return f"{m.group(1)}<{_demangle_args(m.group(2) + 'E')}>"
    m = re.search(r"h3k::(\w+)", name)
    return m.group(1) if m else name[:60]


def is_ours(name: str) -> bool:
    return "h3k::" in name or name.startswith("_ZN3h3k")


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(d: str, steps: int, warmup: int):
    """{(kernel, grid threads): (calls, mean ns over the timed dispatches, total ns, outside
    the steps?)} from the per-dispatch trace (one kernel launched on several grid sizes,
    such as a row quantiser used on weights and on activations, counts once per size).
    The profiled bench runs `warmup` untimed steps, then `steps` plain steps and `steps`
    steps with event records (2 * steps timed steps in all); every step starts with the
    AdaLN kernel. A kernel launched k times per step (k * (warmup + 2 * steps) dispatches
    from the first AdaLN launch on) is averaged over its last k * 2 * steps dispatches; any
    other kernel (set-up work such as weight quantisation) over all of its dispatches,
    flagged True."""
    per = defaultdict(list)
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_trace.csv")))):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        per[(r["Kernel_Name"], str(grid))].append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    starts = [t for (name, _), v in per.items() if "adaln_kernel" in name for t, _ in v]
    t0 = min(starts) if starts else -1
    per_cmd = warmup + 2 * steps
    out = {}
    for key, v in per.items():
        v.sort()
        n = len(v)
        n_in = sum(1 for t, _ in v if t >= t0)
        whole = n_in == 0 or n_in % per_cmd != 0
        timed = n if whole else n_in // per_cmd * 2 * steps
        durs = [t for _, t in v[n - timed:]]
        out[key] = (n_in if not whole else n, sum(durs) / len(durs), float(sum(t for _, t in v)), whole)
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
    ap.add_argument("--steps", type=int, required=True, help="--steps of the profiled bench run")
    ap.add_argument("--warmup", type=int, default=2, help="untimed steps before them")
    ap.add_argument("--cmd", required=True, help="the command lines that produced the inputs")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--name", default=None,
                    help="file-name tag of the summaries (default: the workload name)")
    ap.add_argument("--no-traffic", action="store_true",
                    help="do not write traffic.json (a variant of the measured workload)")
    ap.add_argument("--sq", default=None, help="directory of the SQ counter run (optional)")
    ap.add_argument("--sq-cmd", default="", help="the command line of the SQ counter run")
    a = ap.parse_args()
    a.name = a.name or a.workload

    stats = kernel_stats(a.ktrace, a.steps, a.warmup)
    fetch = counter_by_kernel(a.fetch, "FETCH_SIZE")
    write = counter_by_kernel(a.write, "WRITE_SIZE")
    ff = copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    fw = copy_factor(a.copy_write, "WRITE_SIZE", a.copy_bytes)

    lines = [f"# Kernel durations and HBM traffic per launch, workload {a.workload}", "",
             "Commands:", *[f"    {c}" for c in a.cmd.split(" ;; ")], "",
             f"Copy calibration (plain 1 GiB device copy): FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {fw:.3f}", "",
             f"Durations: mean over the dispatches of the bench's 2 x {a.steps} timed steps (plain and event-timed "
             f"loops; its {a.warmup} warm-up steps excluded); * = launched outside the steps, mean of all dispatches.", "",
             f"{'kernel':58s} {'calls':>6s} {'avg us':>10s} {'ms/step':>9s} {'read MB':>9s} {'write MB':>9s}"]
    traffic = {"workload": a.workload, "copy_factor": {"fetch": ff, "write": fw},
               "sources": {f: source_hash(f) for f, _ in KINDS.values()}, "kernels": {}}
    rows = []
    grids = defaultdict(int)
    for name, _ in stats:
        grids[name] += 1
    for (name, grid), (calls, avg_ns, tot_ns, whole) in stats.items():
        if not is_ours(name):
            continue
        rd = fetch.get((name, grid), float("nan")) * 1024 * ff
        wr = write.get((name, grid), float("nan")) * 1024 * fw
        rows.append((tot_ns, name, grid, calls, avg_ns, rd, wr, whole))
    for tot_ns, name, grid, calls, avg_ns, rd, wr, whole in sorted(rows, reverse=True):
        sfx = (f" [{grid}]" if grids[name] > 1 else "") + (" *" if whole else "")
        label = short_name(name)[:58 - len(sfx)] + sfx
        # launches per step x mean duration (kernels launched outside the steps: blank)
        per_step = "" if whole else f"{calls / (a.warmup + 2 * a.steps) * avg_ns / 1e6:9.3f}"
        lines.append(f"{label:58s} {calls:6d} {avg_ns / 1e3:10.1f} {per_step:>9s} {rd / 1e6:9.1f} {wr / 1e6:9.1f}")
        for kind, (src, key) in KINDS.items():
            if key in name:
                traffic["kernels"].setdefault(short_name(name), {"kind": kind, "source": src,
                                                                 "read_bytes": rd, "write_bytes": wr,
                                                                 "avg_us": avg_ns / 1e3})
    os.makedirs(a.out, exist_ok=True)
    open(os.path.join(a.out, f"kernels_{a.name}.txt"), "w").write("\n".join(lines) + "\n")
    if not a.no_traffic:
        json.dump(traffic, open(os.path.join(a.out, "traffic.json"), "w"), indent=1)
    print("\n".join(lines))
    if a.sq:
        sq_summary(a)


def sq_summary(a):
    """MFMA-busy and LDS figures per kernel from one SQ counter run (means over dispatches).
    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so cycles per XCD = value / 8; the machine
    has 256 CUs, 1024 SIMDs; SQ_WAVE_CYCLES and SQ_WAIT_ANY count quad-cycles."""
    acc = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(_one(os.path.join(a.sq, "**", "*counter_collection.csv")))):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# Matrix-core and LDS activity per launch, workload {a.workload}", "",
             "Command:", f"    {a.sq_cmd}", "",
             f"{'kernel':58s} {'MFMA busy':>10s} {'wait/wave':>10s} {'LDS confl/inst':>15s} {'LDS active':>11s}"]
    rows = []
    for name, cs in acc.items():
        if not is_ours(name):
            continue
        d = {c: sum(v) / len(v) for c, v in cs.items()}
        cyc = d.get("GRBM_GUI_ACTIVE", 0) / 8
        if cyc <= 0:
            continue
        mfma = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (cyc * 1024)
        wait = d.get("SQ_WAIT_ANY", 0) / max(d.get("SQ_WAVE_CYCLES", 1), 1)
        confl = d.get("SQ_LDS_BANK_CONFLICT", 0) / max(d.get("SQ_INSTS_LDS", 1), 1)
        ldsa = d.get("SQ_LDS_IDX_ACTIVE", 0) / (cyc * 256)
        rows.append((cyc, name, mfma, wait, confl, ldsa))
    for cyc, name, mfma, wait, confl, ldsa in sorted(rows, reverse=True):
        lines.append(f"{short_name(name)[:58]:58s} {mfma:10.3f} {wait:10.3f} {confl:15.3f} {ldsa:11.3f}")
    open(os.path.join(a.out, f"sq_{a.name}.txt"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
