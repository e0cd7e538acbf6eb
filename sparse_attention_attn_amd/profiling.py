"""Summaries of rocprofv3 output for the kernels of libattn.so.

Turns the CSV files that `rocprofv3 --kernel-trace --stats` and `rocprofv3 --pmc FETCH_SIZE`
/ `--pmc WRITE_SIZE` write into the short text summaries kept with the sources, and into the
per-launch HBM traffic record that bench.py attaches to its roofline figure.

HBM traffic calibration. FETCH_SIZE and WRITE_SIZE count memory requests leaving the L2 in
KiB; how a request is sized depends on the chip, so the raw counts are scaled by what the same
counter reads for a plain device-to-device copy of known size (bench.py --copy-calib-mib N
runs one such copy, which the runtime executes as `__amd_rocclr_copyBuffer` dispatches):
factor = bytes the copy must move / bytes the counter reports for it.

Usage (after the three rocprofv3 runs, see the header of each summary for the commands):

    python -m sparse_attention_attn_amd.profiling summary --stats DIR --fetch DIR --write DIR \
        --calib-mib 1024 --kernel "fwd_dense_kernel<128, 1, 8, false>" --workload gqa_prefill_8k \
        --command "..." --out profiles/fwd_dense_kernel_gqa_prefill_8k.md [--traffic-json F]

MFMA work and clock. One `rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE
SQ_VALU_MFMA_BUSY_CYCLES` run gives, per dispatch, the bf16 MFMA flops the kernel executed
(MOPS x 512), the GPU cycles it was active and the SIMD cycles its matrix cores were busy; the
`mfma` subcommand sets the flops against the algorithmic count and divides the active cycles
by the dispatch's own duration (its start and end timestamps) to give the shader clock.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_hash(files):
    """First 16 hex digits of the SHA-256 of the named csrc files, concatenated in order."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def read_kernel_stats(stats_dir):
    """Rows of *_kernel_stats.csv as dicts with numeric fields."""
    path = _one(os.path.join(stats_dir, "**", "*kernel_stats.csv"))
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            out.append({"name": r["Name"], "calls": int(r["Calls"]),
                        "total_ns": float(r["TotalDurationNs"]), "avg_ns": float(r["AverageNs"]),
                        "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                        "pct": float(r["Percentage"])})
    return out


def read_counter(counter_dir, counter):
    """(kernel name, value) per dispatch, in dispatch order, for one counter."""
    path = _one(os.path.join(counter_dir, "**", "*counter_collection.csv"))
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(n, v) for _, n, v in rows]


def copy_factor(dispatches, calib_mib, moved_per_mib=1.0):
    """Scale factor from the first run of copy dispatches (the calibration copy)."""
    total = 0.0
    seen = False
    for name, v in dispatches:
        if COPY_KERNEL in name:
            total += v
            seen = True
        elif seen:
            break
    if not seen or total <= 0:
        raise ValueError("no calibration copy dispatch found")
    return calib_mib * 1024.0 * moved_per_mib / total


def read_counter_rows(counter_dir, counter):
    """(kernel name, value, duration ns) per dispatch, in dispatch order, for one counter."""
    path = _one(os.path.join(counter_dir, "**", "*counter_collection.csv"))
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]),
                             dur))
    rows.sort()
    return [(n, v, d) for _, n, v, d in rows]


def mfma_summary(counter_dir, kernel, workload, command, algorithmic_flops, simds=1024, xcds=8):
    """Per-dispatch averages of the MFMA and clock counters for `kernel` (see module doc)."""
    def avg(counter):
        rows = [(v, d) for n, v, d in read_counter_rows(counter_dir, counter) if kernel in n]
        if not rows:
            raise ValueError(f"kernel {kernel!r} not found for {counter}")
        return (sum(v for v, _ in rows) / len(rows), sum(d for _, d in rows) / len(rows),
                len(rows))
    mops, dur, n = avg("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    gui, dur_g, _ = avg("GRBM_GUI_ACTIVE")
    busy, _, _ = avg("SQ_VALU_MFMA_BUSY_CYCLES")
    flops = mops * 512.0
    gui /= xcds  # the CSV sums GRBM_GUI_ACTIVE over the XCDs, each of which counts every cycle
    rec = {"workload": workload, "kernel": kernel, "command": command, "dispatches": n,
           "mfma_flops_per_dispatch": flops, "algorithmic_flops": algorithmic_flops,
           "executed_over_algorithmic": flops / algorithmic_flops if algorithmic_flops else None,
           "gpu_active_cycles": gui, "dispatch_ns": dur_g,
           "shader_clock_ghz": gui / dur_g if dur_g > 0 else None,
           "mfma_busy_pct": 100.0 * busy / (gui * simds) if gui > 0 else None}
    return rec


def render_mfma_md(rec):
    lines = [f"# {rec['kernel']} — {rec['workload']}: MFMA work and clock", "",
             "Counter run (run from the repository root):", "", "```", rec["command"], "```", "",
             f"- dispatches averaged: {rec['dispatches']}",
             f"- bf16 MFMA flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): "
             f"{rec['mfma_flops_per_dispatch']:,.0f}",
             f"- algorithmic flops (2 (Dqk + Dv) per visible pair): {rec['algorithmic_flops']:,}",
             f"- executed / algorithmic: {rec['executed_over_algorithmic']:.4f} (masked parts of "
             "the diagonal tiles are computed, then discarded)",
             f"- GPU active cycles (GRBM_GUI_ACTIVE, per XCD): {rec['gpu_active_cycles']:,.0f} over "
             f"{rec['dispatch_ns'] / 1e3:.1f} us of dispatch: shader clock "
             f"{rec['shader_clock_ghz']:.3f} GHz",
             f"- MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over active cycles x 1024 SIMDs): "
             f"{rec['mfma_busy_pct']:.1f}%", ""]
    return "\n".join(lines)


def per_dispatch(dispatches, kernel):
    vals = [v for n, v in dispatches if kernel in n]
    if not vals:
        raise ValueError(f"kernel {kernel!r} not found")
    return sum(vals) / len(vals), len(vals)


def step_rate(stats, kernels, work, unit, peak):
    """Per-step rate from the kernel trace: `kernels` run once per step each; their average
    durations add up to the step time. work: algorithmic flops (unit TFLOP/s) or bytes (unit
    GB/s) of one step; peak in the same unit."""
    ns = 0.0
    parts = []
    for k in kernels:
        mine = [s for s in stats if k in s["name"]]
        if not mine:
            raise ValueError(f"kernel {k!r} not in the trace")
        ns += mine[0]["avg_ns"]
        parts.append({"kernel": k, "avg_us": round(mine[0]["avg_ns"] / 1e3, 2),
                      "calls": mine[0]["calls"]})
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    rate = work / (ns * 1e-9) / scale
    return {"kernels": parts, "step_us": round(ns / 1e3, 2), "work": work, "unit": unit,
            "achieved": round(rate, 3), "peak": peak, "frac": round(rate / peak, 4)}


def summary(stats_dir, fetch_dir, write_dir, calib_mib, kernel, workload, command,
            algorithmic_bytes=None):
    stats = read_kernel_stats(stats_dir)
    rec = {"workload": workload, "kernel": kernel, "command": command}
    mine = [s for s in stats if kernel in s["name"]]
    if mine:
        rec["avg_ns"] = mine[0]["avg_ns"]
        rec["calls"] = mine[0]["calls"]
    if fetch_dir and write_dir:
        fd = read_counter(fetch_dir, "FETCH_SIZE")
        wd = read_counter(write_dir, "WRITE_SIZE")
        ff = copy_factor(fd, calib_mib)
        wf = copy_factor(wd, calib_mib)
        fk, nf = per_dispatch(fd, kernel)
        wk, nw = per_dispatch(wd, kernel)
        rec.update({"fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_factor": ff,
                    "write_factor": wf, "dispatches_counted": min(nf, nw),
                    "hbm_bytes_per_launch": int(round((fk * ff + wk * wf) * 1024.0))})
        if algorithmic_bytes:
            rec["algorithmic_bytes"] = int(algorithmic_bytes)
            rec["traffic_over_algorithmic"] = rec["hbm_bytes_per_launch"] / algorithmic_bytes
    return rec, stats


def render_md(rec, stats, stats_cmd, fetch_cmd, write_cmd):
    lines = [f"# {rec['kernel']} — {rec['workload']}", ""]
    lines += ["Kernel-trace statistics command (run from the repository root):", "",
              "```", stats_cmd, "```", ""]
    if "rate" in rec:
        r = rec["rate"]
        names = " + ".join(f"`{p['kernel']}` {p['avg_us']} µs" for p in r["kernels"])
        lines += [f"- step time from the trace: {names} = {r['step_us']} µs",
                  f"- algorithmic work per step: {r['work']:,} ({'flop' if r['unit'] == 'TFLOP/s' else 'B'})",
                  f"- rate: {r['achieved']} {r['unit']} = {r['frac']:.4f} of the {r['peak']} "
                  f"{r['unit']} peak", ""]
    lines += ["| kernel | calls | avg µs | min µs | max µs | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for s in stats:
        name = s["name"] if len(s["name"]) <= 160 else s["name"][:157] + "..."
        lines.append(f"| `{name}` | {s['calls']} | {s['avg_ns'] / 1e3:.1f} | "
                     f"{s['min_ns'] / 1e3:.1f} | {s['max_ns'] / 1e3:.1f} | {s['pct']:.2f} |")
    lines.append("")
    if "hbm_bytes_per_launch" in rec:
        lines += ["Counter runs (one counter per run):", "", "```", fetch_cmd, write_cmd, "```", "",
                  f"- FETCH_SIZE per dispatch (raw): {rec['fetch_kib_raw']:.1f} KiB, copy "
                  f"calibration factor {rec['fetch_factor']:.4f}",
                  f"- WRITE_SIZE per dispatch (raw): {rec['write_kib_raw']:.1f} KiB, copy "
                  f"calibration factor {rec['write_factor']:.4f}",
                  f"- HBM-side traffic per launch: {rec['hbm_bytes_per_launch']:,} B"]
        if "algorithmic_bytes" in rec:
            lines.append(f"- algorithmic bytes per launch: {rec['algorithmic_bytes']:,} B "
                         f"(traffic / algorithmic = {rec['traffic_over_algorithmic']:.3f})")
        lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m sparse_attention_attn_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summary")
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--calib-mib", type=int, default=1024)
    s.add_argument("--kernel", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--algorithmic-bytes", type=float, default=None)
    s.add_argument("--stats-command", required=True)
    s.add_argument("--fetch-command", default="")
    s.add_argument("--write-command", default="")
    s.add_argument("--source-files", default="",
                   help="comma list of csrc files whose hash tags the traffic record")
    s.add_argument("--out", required=True)
    s.add_argument("--traffic-json")
    s.add_argument("--step-kernel", action="append", default=[],
                   help="kernel run once per step (repeat for several); with --work, --unit "
                        "and --peak the summary states the step's rate and fraction of peak")
    s.add_argument("--work", type=float, default=None)
    s.add_argument("--unit", default="TFLOP/s")
    s.add_argument("--peak", type=float, default=None)
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--algorithmic-flops", type=int, required=True)
    m.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "mfma":
        rec = mfma_summary(a.dir, a.kernel, a.workload, a.command, a.algorithmic_flops)
        with open(a.out, "w") as fh:
            fh.write(render_mfma_md(rec))
        print(json.dumps({k: v for k, v in rec.items() if k != "command"}))
        return
    rec, stats = summary(a.stats, a.fetch, a.write, a.calib_mib, a.kernel, a.workload,
                         a.stats_command, a.algorithmic_bytes)
    if a.work is not None and a.peak is not None:
        rec["rate"] = step_rate(stats, a.step_kernel or [a.kernel], int(a.work), a.unit, a.peak)
    with open(a.out, "w") as fh:
        fh.write(render_md(rec, stats, a.stats_command, a.fetch_command, a.write_command))
    if a.traffic_json:
        if a.source_files:
            rec["kernel_source_sha256_16"] = kernel_source_hash(a.source_files.split(","))
        rec["counter_commands"] = [a.fetch_command, a.write_command]
        with open(a.traffic_json, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
    print(json.dumps({k: v for k, v in rec.items() if k != "command"}))


if __name__ == "__main__":
    main()
