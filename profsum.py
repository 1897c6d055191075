#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

  ktrace: --kernel-trace --stats output -> per-kernel call count and
          average / min / max duration.
  pmc:    four --pmc runs (FETCH_SIZE and WRITE_SIZE of one kernel, the same
          two counters of a plain copy of known size) -> HBM bytes per launch
          of that kernel, each counter scaled by what it reads for the copy.
  counters: several --pmc runs of shader counters plus a kernel trace ->
          per-dispatch averages, MFMA busy share, shader clock, LDS / VALU
          activity of one kernel.

Reads CSV files only; runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def ktrace(args):
    path = _one(os.path.join(args.dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    out = [f"# rocprofv3 kernel trace: {args.title}",
           f"command: {args.cmd}", "",
           f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = re.sub(r"\(.*", "", r["Name"])[:90]
        out.append(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                   f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                   f"{float(r['Percentage']):>6.2f}  {name}")
    text = "\n".join(out) + "\n"
    open(args.out, "w").write(text)
    print(text)


def _counter(dirname, counter, match):
    """Per-dispatch values of one counter for kernels whose name matches."""
    path = _one(os.path.join(dirname, "**", "*counter_collection.csv"))
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or not re.search(match, r["Kernel_Name"]):
            continue
        key = r["Dispatch_Id"]
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"{counter}: no dispatch of /{match}/ in {path}")
    return list(vals.values())


def pmc(args):
    from bench import algorithmic_bytes, kernel_source_sha
    from swiglu_mlp_rmsnorm_amd import synth
    w = synth.WORKLOADS[args.workload]
    alg = algorithmic_bytes(args.kernel, args.M, w.d, w.ff, w.wtype)
    copy_f = statistics.median(_counter(args.copy_fetch, "FETCH_SIZE", args.copy_match))
    copy_w = statistics.median(_counter(args.copy_write, "WRITE_SIZE", args.copy_match))
    k_f = _counter(args.fetch, "FETCH_SIZE", args.match)
    k_w = _counter(args.write, "WRITE_SIZE", args.match)
    # counters are KiB per dispatch; the copy moves copy_bytes each way. A
    # kernel kind may dispatch more than once per forward step: traffic is
    # summed over the run's dispatches and divided by its steps.
    for n, name in ((len(k_f), "FETCH_SIZE"), (len(k_w), "WRITE_SIZE")):
        if n % args.steps:
            raise SystemExit(f"{name}: {n} dispatches of /{args.match}/ is not a multiple of "
                             f"the run's {args.steps} steps (a run with extra timing windows?)")
    fetch_scale = args.copy_bytes / (copy_f * 1024.0)
    write_scale = args.copy_bytes / (copy_w * 1024.0)
    fetch_b = sum(k_f) * 1024.0 * fetch_scale / args.steps
    write_b = sum(k_w) * 1024.0 * write_scale / args.steps
    traffic = fetch_b + write_b
    sha = kernel_source_sha(args.kernel)
    lines = [
        f"# HBM traffic of {args.kernel} on {args.workload}, M={args.M}",
        f"kernel: {args.kernel}",
        f"kernel_match: {args.match}",
        f"source_sha: {sha}",
        f"traffic_bytes_per_step: {traffic:.0f}",
        f"fetch_bytes_per_step: {fetch_b:.0f}",
        f"write_bytes_per_step: {write_b:.0f}",
        f"algorithmic_bytes_per_step: {alg}",
        f"steps_in_run: {args.steps}",
        f"traffic_over_algorithmic: {traffic / alg:.4f}",
        f"dispatches_fetch: {len(k_f)}",
        f"dispatches_write: {len(k_w)}",
        f"fetch_kib_per_dispatch: {' '.join(f'{v:.0f}' for v in k_f)}",
        f"write_kib_per_dispatch: {' '.join(f'{v:.0f}' for v in k_w)}",
        f"copy_bytes: {args.copy_bytes}",
        f"copy_fetch_kib: {copy_f:.1f}",
        f"copy_write_kib: {copy_w:.1f}",
        f"fetch_scale: {fetch_scale:.4f}",
        f"write_scale: {write_scale:.4f}",
        "",
        "commands:",
        f"  kernel FETCH_SIZE: {args.cmd_fetch}",
        f"  kernel WRITE_SIZE: {args.cmd_write}",
        f"  copy FETCH_SIZE:   {args.cmd_copy_fetch}",
        f"  copy WRITE_SIZE:   {args.cmd_copy_write}",
    ]
    text = "\n".join(l for l in lines if l is not None) + "\n"
    open(args.out, "w").write(text)
    print(text)


def _dispatch_values(dirname, match):
    """{counter: [per-dispatch value]} for kernels whose name matches (each
    dispatch's value summed over the counter's dimensions), plus
    "_DURATION_NS": the dispatches' own durations in that run."""
    path = _one(os.path.join(dirname, "**", "*counter_collection.csv"))
    per = {}
    for r in csv.DictReader(open(path)):
        if not re.search(match, r["Kernel_Name"]):
            continue
        key = (r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        dk = ("_DURATION_NS", r["Dispatch_Id"])
        per[dk] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for (c, _), v in sorted(per.items(), key=lambda kv: int(kv[0][1])):
        out.setdefault(c, []).append(v)
    if not out:
        raise SystemExit(f"no dispatch of /{match}/ in {path}")
    return out


def _trace_avg_ns(dirname, match):
    path = _one(os.path.join(dirname, "**", "*kernel_stats.csv"))
    calls, total = 0, 0.0
    for r in csv.DictReader(open(path)):
        if re.search(match, r["Name"]):
            calls += int(r["Calls"])
            total += float(r["TotalDurationNs"])
    if not calls:
        raise SystemExit(f"no kernel /{match}/ in {path}")
    return total / calls, calls


def counters(args):
    """Hardware counters of one kernel (several --pmc passes, one directory
    each) with the kernel's average duration from a --kernel-trace run:
    per-dispatch averages and the derived utilisations."""
    vals = {}
    for d in args.dirs:
        for c, v in _dispatch_values(d, args.match).items():
            vals[c] = v
    avg = {c: statistics.mean(v) for c, v in vals.items()}
    dur_ns, calls = _trace_avg_ns(args.trace, args.match)
    simds, cus = args.cus * 4, args.cus
    # GRBM counters arrive summed over the XCDs (one GRBM each): per-XCD
    # cycles are the sum over args.xcds; SQ counters are sums over all CUs
    gui_x = avg["GRBM_GUI_ACTIVE"] / args.xcds if "GRBM_GUI_ACTIVE" in avg else None
    lines = [f"# hardware counters of {args.kernel} ({args.title})",
             f"kernel_match: {args.match}",
             f"avg_duration_us: {dur_ns / 1e3:.2f}  (kernel trace, {calls} dispatches)"]
    gui = gui_x
    if gui:
        cdur = avg.get("_DURATION_NS", dur_ns)
        clk = gui / cdur
        if clk <= 2.45:
            lines.append(f"shader_clock_ghz: {clk:.3f}  (GRBM_GUI_ACTIVE / {args.xcds} XCDs"
                         " / the dispatch's duration in the counter run)")
        else:  # the GRBM window outlasts a short dispatch: no clock from it
            lines.append(f"shader_clock_ghz: not derived (GRBM_GUI_ACTIVE / {args.xcds} XCDs"
                         f" over the dispatch's duration gives {clk:.2f}, above the 2.4 GHz"
                         " peak: the counting window is longer than the dispatch)")
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        lines.append(f"mfma_busy_pct: {100 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * simds):.1f}"
                     f"  (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * {simds} SIMDs))")
    if "SQ_INSTS_VALU_MFMA_MOPS_F16" in avg:
        fl = avg["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
        lines.append(f"mfma_f16_flop_per_dispatch: {fl:.4g}  (SQ_INSTS_VALU_MFMA_MOPS_F16 * 512)")
        lines.append(f"mfma_tflop_per_s: {fl / dur_ns / 1e3:.1f}")
        if gui:
            peak_at_clock = 2500.0 * (gui / dur_ns) / 2.4
            lines.append(f"mfma_peak_at_measured_clock_tflop_per_s: {peak_at_clock:.0f}"
                         "  (2.5 PFLOP/s scaled from 2.4 GHz)")
    if gui:
        for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                  "SQ_ACTIVE_INST_MISC", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                  "SQ_ACTIVE_INST_ANY", "SQ_VALU_MFMA_COEXEC_CYCLES"):
            if c in avg and "SQ_WAVE_CYCLES" in avg:
                lines.append(f"{c.lower()}_per_wave_cycle: {avg[c] / avg['SQ_WAVE_CYCLES']:.3f}")
        if "SQ_LDS_IDX_ACTIVE" in avg:
            lines.append(f"lds_active_pct: {100 * avg['SQ_LDS_IDX_ACTIVE'] / (gui * cus):.1f}"
                         f"  (SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE * {cus} CUs))")
        if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg:
            lines.append(f"lds_bank_conflict_ratio: "
                         f"{avg['SQ_LDS_BANK_CONFLICT'] / max(avg['SQ_LDS_IDX_ACTIVE'], 1):.4f}")
        if "TA_TA_BUSY_sum" in avg:
            lines.append(f"ta_busy_pct: {100 * avg['TA_TA_BUSY_sum'] / (gui * cus):.1f}")
    if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
        lines.append(f"valu_insts_per_mfma: {avg['SQ_INSTS_VALU'] / max(avg['SQ_INSTS_MFMA'], 1):.2f}")
    lines += ["", "per-dispatch averages:"]
    lines += [f"  {c}: {avg[c]:.6g}" for c in sorted(avg)]
    lines += ["", "commands:"] + [f"  {c}" for c in args.cmds]
    text = "\n".join(lines) + "\n"
    open(args.out, "w").write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    k = sub.add_parser("ktrace")
    k.add_argument("--dir", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--cmd", required=True)
    k.add_argument("--out", required=True)
    p = sub.add_parser("pmc")
    for a in ("fetch", "write", "copy_fetch", "copy_write", "match", "kernel", "workload",
              "out", "cmd_fetch", "cmd_write", "cmd_copy_fetch", "cmd_copy_write"):
        p.add_argument("--" + a.replace("_", "-"), dest=a, required=True)
    p.add_argument("--copy-match", default=".")
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--M", type=int, required=True)
    p.add_argument("--steps", type=int, required=True,
                   help="forward steps in the counted run (bench.py warmup + steps)")
    c = sub.add_parser("counters")
    c.add_argument("--dirs", nargs="+", required=True, help="one directory per --pmc pass")
    c.add_argument("--trace", required=True, help="directory of a --kernel-trace --stats run")
    for a in ("match", "kernel", "title", "out"):
        c.add_argument("--" + a, required=True)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--cmds", nargs="+", default=[])
    args = ap.parse_args()
    {"ktrace": ktrace, "pmc": pmc, "counters": counters}[args.mode](args)


if __name__ == "__main__":
    main()
