#!/usr/bin/env python3
"""Benchmark of the fused gated-MLP forward on one MI355X.

One step = one fmlp_forward call (RMSNorm -> interleaved gate/up matmul ->
SiLU*mul -> down projection) on one layer, the weight set rotating every
step through `sets` distinct layers so the 256 MB Infinity Cache cannot serve
repeats. Inputs are resident in HBM before timing starts.

Prints ONE JSON line (stdout). Default workload: Phi-3-mini-shaped decode,
d=3072, ff=8192, M=1, 32 weight sets. `--workload`/`--M` select another
configuration; `--all` prints one line per (workload, M).
"""
from __future__ import annotations

import argparse
import functools
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MLP tokens/s + % HBM roofline (decode M=1) / % MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
DEFAULT_WORKLOAD = "phi3mini_decode_d3072_ff8192"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--all", action="store_true", help="every (workload, M); one line each")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the five repeat windows and the graph-captured timing")
    ap.add_argument("--path", choices=sorted(PATHS), default="auto",
                    help="kernel path (fmlp_forward_path); auto is fmlp_forward's own choice")
    ap.add_argument("--activation", choices=sorted(ACTS), default="silu",
                    help="gate activation; other than silu runs fmlp_forward_ex")
    ap.add_argument("--residual", action="store_true",
                    help="add a residual input before the norm (fmlp_forward_ex)")
    ap.add_argument("--weights", choices=("stored", "f16"), default="stored",
                    help="f16: run bf16 workloads on their weights converted to fp16 "
                         "(fmlp_convert_f16, the FMLP_W_F16 weight type)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "known-size reference for the HBM byte counters) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- bytes / flops

PATHS = {"auto": 0, "decode": 1, "prefill": 2, "single_pass": 3}
ACTS = {"silu": 0, "gelu_tanh": 1, "gelu_erf": 2}


def weight_bytes(d, ff, wtype):
    """(W_gu bytes, W_down bytes), scales included for int4."""
    if wtype == "int4":
        return 2 * ff * d // 2 + 2 * ff * (d // 32) * 2, d * ff // 2 + d * (ff // 32) * 2
    return 2 * ff * d * 2, d * ff * 2


def step_bytes(M, d, ff, wtype):
    """Algorithmic bytes of one step: weights (+ scales) + x + gamma + y."""
    gu, dn = weight_bytes(d, ff, wtype)
    return gu + dn + M * d * 2 + d * 2 + M * d * 2


def kernel_bytes(kernel, M, d, ff, wtype, f16=None):
    """Algorithmic bytes of one launch of a decode kernel: its weights
    (+ scales), its activation inputs and its outputs. bf16 path: gate/up
    reads x and gamma and writes the SiLU*mul product as a bf16 hi + lo pair
    (4 bytes per element), which down reads back. int4 path, and the bf16
    path at larger M (f16: a prep kernel ran): gate/up reads the prepared
    fp16 n, the product is fp16 (2 bytes per element).
    Single-pass decode: one kernel reads both matrices, x and gamma and
    writes fp32 partial sums per 32-feature slice of ff, which the reduce
    kernel reads back to write y."""
    gu, dn = weight_bytes(d, ff, wtype)
    f16 = wtype == "int4" if f16 is None else f16
    a_elem = 2 if f16 else 4
    partials = (ff // 32) * M * d * 4  # single-pass decode: fp32 per 32-feature slice
    if kernel == "decode_fused_bf16":
        return gu + dn + M * d * 2 + d * 2 + partials
    if kernel == "partial_reduce":
        return partials + M * d * 2
    if "gateup" in kernel:
        act_in = M * d * 2 + (0 if f16 else d * 2)
        return gu + act_in + M * ff * a_elem
    if kernel == "act_prep":
        return M * d * 2 + d * 2 + M * d * 2
    return dn + M * ff * a_elem + M * d * 2


def gemm_bytes(kernel, M, d, ff):
    """Algorithmic bytes of one prefill GEMM launch: bf16 weights, fp16
    activations in, its output (fp16 SiLU*mul product, or bf16 y)."""
    if kernel == "gemm_gateup_silu_f16":
        return 2 * ff * d * 2 + M * d * 2 + M * ff * 2
    return d * ff * 2 + M * ff * 2 + M * d * 2


def algorithmic_bytes(kernel, M, d, ff, wtype):
    if kernel.startswith("gemm"):
        return gemm_bytes(kernel, M, d, ff)
    return kernel_bytes(kernel, M, d, ff, wtype)


def step_flops(M, d, ff):
    return 6.0 * M * ff * d


# ----------------------------------------------------------------------------- traffic

def kernel_source_sha(kernel):
    """Hash of the HIP source that defines a kernel kind (to expire counter data)."""
    src = {
        "decode_gateup_bf16": "decode.hip", "decode_down_bf16": "decode.hip",
        "decode_gateup_int4": "decode.hip", "decode_down_int4": "decode.hip",
        "gemm_gateup_silu_f16": "prefill.hip", "gemm_down_f16": "prefill.hip",
        "act_prep": "decode.hip", "decode_fused_bf16": "decode.hip",
        "partial_reduce": "decode.hip",
    }.get(kernel)
    if src is None:
        return None
    h = hashlib.sha256()
    for f in (src, "device_common.hpp"):
        h.update(open(os.path.join(ROOT, "swiglu_mlp_rmsnorm_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, M):
    """HBM bytes per forward step of one kernel kind, from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE of its dispatches,
    scaled by the copy-kernel calibration), or None when there is none or the
    kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}_M{M}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^(\w+):\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_sha") != kernel_source_sha(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_step"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(w, M, host_layer, host_inputs, budget_s):
    """Time the fp64 CPU oracle on a bounded sample of the same workload
    (weight set 0; the seeded row-major weights, or for int4 the seeded tiled
    buffers expanded by the oracle's own layout code)."""
    from oracle import oracle
    x, g = host_inputs
    if w.wtype == "int4":
        q_gu, s_gu, q_d, s_d = host_layer
        host_layer = (*oracle.untile_int4(q_gu, s_gu, 2 * w.ff, w.d),
                      *oracle.untile_int4(q_d, s_d, w.d, w.ff))
    # rows are independent: for large M, run row subsets until the budget is spent
    rows_per_call = M if M <= 32 else 1
    done_rows, calls = 0, 0
    t0 = time.perf_counter()
    while True:
        r0 = (calls * rows_per_call) % M
        xs = x[r0:r0 + rows_per_call]
        if w.wtype == "int4":
            q_gu, s_gu, q_d, s_d = host_layer
            oracle.forward_int4(xs, g, w_eps(), q_gu, s_gu, q_d, s_d)
        else:
            wg, wu, wd = host_layer
            oracle.forward_unfused(xs, g, w_eps(), wg, wu, wd)
        done_rows += xs.shape[0]
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {
        "value": done_rows / el, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
        "sample": (f"{calls} oracle forward call(s) of {rows_per_call} row(s) on weight set 0 of "
                   f"{w.name} (fp64, {el:.1f} s)"),
    }


def w_eps():
    from swiglu_mlp_rmsnorm_amd import synth
    return synth.EPS


# ----------------------------------------------------------------------------- run

def run_one(wname, M, steps, warmup, args):
    import torch
    from swiglu_mlp_rmsnorm_amd import fmlp as F
    from swiglu_mlp_rmsnorm_amd import synth

    w = synth.WORKLOADS[wname]
    dev = torch.device("cuda:0")
    d, ff = w.d, w.ff
    w16 = args.weights == "f16"
    if w16 and w.wtype != "bf16":
        raise SystemExit(f"--weights f16 converts bf16 weights; {wname} holds {w.wtype}")
    path = args.path if args.path != "auto" else ("decode" if M <= 32 else "prefill")
    pcode = None if args.path == "auto" else PATHS[args.path]  # None: fmlp_forward itself
    ex = args.activation != "silu" or args.residual  # the variants run fmlp_forward_ex
    log(f"[bench] {wname} M={M}: building {w.sets} weight set(s)")
    layers, xs = [], []
    host0 = None  # row-major / untiled copies of set 0 for the CPU baseline
    for l in range(w.sets):
        if w.wtype == "int4":
            layers.append(synth.layer_int4(w, l, dev))
            if l == 0 and not args.no_cpu_baseline:
                host0 = tuple(synth.bits(t) for t in layers[0])
        else:
            wg, wu, wd = synth.layer_bf16(w, l, dev)
            L = (F.fmlp_pack_interleaved(wg, wu), F.fmlp_pack_matrix(wd))
            if w16:  # (2 bytes per weight either way)
                L = (F.fmlp_convert_f16(L[0]), F.fmlp_convert_f16(L[1]))
            layers.append(L)
            if l == 0 and not args.no_cpu_baseline:
                host0 = (synth.bits(wg), synth.bits(wu), synth.bits(wd))
            del wg, wu, wd
        xs.append(synth.inputs(w, M, dev, layer=l))
    torch.cuda.synchronize()
    y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    wt = F.FMLP_W_INT4_G32 if w.wtype == "int4" else F.FMLP_W_F16 if w16 else F.FMLP_W_BF16
    ws = torch.empty(F.fmlp_workspace_size(M, d, ff, wt),
                     dtype=torch.uint8, device=dev)
    res = synth.activations(M, d, 977, dev) if args.residual else None
    hout = torch.empty((M, d), dtype=torch.bfloat16, device=dev) if args.residual else None

    def step(i):
        L = layers[i % w.sets]
        x, g = xs[i % w.sets]
        if ex:
            fwd = functools.partial(F.fmlp_forward_ex, path=pcode or 0,
                                    activation=ACTS[args.activation], residual=res, h_out=hout)
        elif pcode is None:
            fwd = F.fmlp_forward
        else:
            fwd = functools.partial(F.fmlp_forward_path, path=pcode)
        if w.wtype == "int4":
            fwd(x, g, synth.EPS, L[0], L[2], L[1], L[3], y=y, workspace=ws, ff=ff)
        else:
            fwd(x, g, synth.EPS, L[0], L[1], y=y, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {warmup} done; timing {steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = e0.elapsed_time(e1) / steps
    wall_ms_per_step = (t1 - t0) * 1e3 / steps
    tokens_per_s = M / (ms_per_step * 1e-3)
    sb = step_bytes(M, d, ff, w.wtype) + (4 * M * d if args.residual else 0)  # + r in, h out
    log(f"[bench] {ms_per_step*1e3:.2f} us/step (host wall {wall_ms_per_step*1e3:.2f}), "
        f"{sb / ms_per_step / 1e6:.1f} GB/s step")

    # Spread: five more windows of the same length, after the timed region
    # (median, p10, p90 of their us/step); and the same steps captured once as
    # a HIP graph (one rotation of weight sets) and replayed, which shows what
    # host launch overhead the plain loop carries.
    spread = None
    if not args.no_spread:
        win = []
        for r in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(steps):
                step(i)
            b.record()
            torch.cuda.synchronize()
            win.append(a.elapsed_time(b) * 1e3 / steps)
        win.sort()
        spread = {"windows": 5, "steps_per_window": steps,
                  "us_per_step_p10": round(win[0] + 0.4 * (win[1] - win[0]), 3),
                  "us_per_step_median": round(win[2], 3),
                  "us_per_step_p90": round(win[3] + 0.6 * (win[4] - win[3]), 3)}
        spread["graph_us_per_step"] = graph_us_per_step(step, w.sets, steps)
        log(f"[bench] spread {json.dumps(spread)}")

    # per-kernel durations from HIP events recorded by the library on its launch stream
    kernels = {}
    if not args.no_profile:
        F.fmlp_profile_enable(True)
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        for name, (n, ms) in F.fmlp_profile_read().items():
            # a kernel kind may launch more than once per step (the gate/up
            # GEMM's tail launch): rates below use its time per step
            kernels[name] = {"launches": n, "avg_us": ms * 1e3 / n,
                             "launches_per_step": n / steps, "us_per_step": ms * 1e3 / steps}
        F.fmlp_profile_enable(False)
        log(f"[bench] kernels: {json.dumps(kernels)}")

    if "decode_fused_bf16" in kernels:
        path = "single_pass"
    if path == "single_pass":
        dom = "decode_fused_bf16"
        dom_units = kernel_bytes(dom, M, d, ff, w.wtype)
        unit, peak, bound = "GB/s", HBM_PEAK_GBS, "hbm"
    elif path == "decode":
        dom = "decode_gateup_int4" if w.wtype == "int4" else "decode_gateup_bf16"
        # fp16 activations: int4, or a bf16 step that ran the prep kernel
        f16 = w.wtype == "int4" or "act_prep" in kernels
        dom_units = kernel_bytes(dom, M, d, ff, w.wtype, f16)
        unit, peak, bound = "GB/s", HBM_PEAK_GBS, "hbm"
    else:
        dom = "gemm_gateup_silu_f16"
        dom_units = 2.0 * M * (2 * ff) * d
        unit, peak, bound = "TFLOP/s", MFMA_PEAK_TFLOPS, "mfma"
    # the dominant kernel's algorithmic units and time per step (its launches
    # in one step together: one for decode, one or two for the gate/up GEMM)
    roofline = None
    if dom in kernels:
        step_s = kernels[dom]["us_per_step"] * 1e-6
        achieved = dom_units / step_s / (1e9 if unit == "GB/s" else 1e12)
        roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": unit, "frac": round(achieved / peak, 4),
                    "units_per_step": dom_units,
                    "launches_per_step": kernels[dom]["launches_per_step"],
                    # (the committed counter runs are of the stored weight types)
                    "traffic": None if w16 else measured_traffic(dom, wname, M)}
    for name, k in kernels.items():
        t = k["us_per_step"]
        if name.startswith("decode") or name in ("act_prep", "partial_reduce"):
            k["gb_per_s"] = round(kernel_bytes(name, M, d, ff, w.wtype,
                                               w.wtype == "int4" or "act_prep" in kernels)
                                  / (t * 1e3), 1)
        elif name == "gemm_gateup_silu_f16":
            k["tflop_per_s"] = round(2.0 * M * 2 * ff * d / (t * 1e6), 1)
        elif name == "gemm_down_f16":
            k["tflop_per_s"] = round(2.0 * M * ff * d / (t * 1e6), 1)

    # The HBM read rate a plain streaming kernel reaches on exactly the bytes
    # the dominant decode kernel streams (the gate/up weights of each rotated
    # set, read once per launch): the practical ceiling its roofline fraction
    # should be read against.
    ceiling = None
    if path == "decode" and not args.no_profile:
        ceiling = read_ceiling([L[0] for L in layers], steps)
        if roofline is not None and ceiling:
            ceiling["dominant_kernel_frac_of_ceiling"] = round(
                roofline["achieved"] / ceiling["gb_per_s"], 4)

    cpu = None
    if not args.no_cpu_baseline and not ex:  # the oracle baseline times the plain Eq(1) step
        host_inputs = (synth.bits(xs[0][0]), synth.bits(xs[0][1]))
        log(f"[bench] CPU oracle baseline ({args.cpu_seconds:.0f} s budget)")
        cpu = cpu_baseline(w, M, host0, host_inputs, args.cpu_seconds)

    step_gbs = sb / (ms_per_step * 1e-3) / 1e9
    step_tflops = step_flops(M, d, ff) / (ms_per_step * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4-bf16" if w.wtype == "int4" else "f16-bf16" if w16 else "bf16",
        "data": "synthetic",
        "config": {"workload": wname, "M": M, "d": d, "ff": ff, "weight_sets": w.sets,
                   "wtype": "f16" if w16 else w.wtype, "path": path, "activation": args.activation,
                   "residual": bool(args.residual), "parallelism": "none (1 GPU)"},
        "step_gb_per_s": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_tflop_per_s": round(step_tflops, 2),
        "step_mfma_frac": round(step_tflops / MFMA_PEAK_TFLOPS, 4),
        "host_wall_ms_per_step": round(wall_ms_per_step, 6),
        "roofline": roofline,
        "read_ceiling": ceiling,
        "spread": spread,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    del layers, xs
    torch.cuda.empty_cache()
    return rec


def graph_us_per_step(step, period, steps):
    """Capture `period` consecutive steps (one rotation of the weight sets) in
    a HIP graph, replay it to cover about `steps` steps, and return the GPU
    time per step; None if capture fails."""
    import torch
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(period):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
    except RuntimeError as e:
        log(f"[bench] graph capture failed: {e}")
        return None
    reps = max(1, steps // period)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * period)
    del g
    return round(us, 3)


def read_ceiling(buffers, steps):
    """Streaming-read probe (fmlp_read_probe) over the rotated weight buffers,
    timed with the library's dispatch-stamped events; the best of three grid
    sizes."""
    import torch
    from swiglu_mlp_rmsnorm_amd import fmlp as F
    nbytes = buffers[0].numel() * buffers[0].element_size()
    best = None
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=buffers[0].device)
    for wgs in (512, 1024, 2048):
        for i in range(2 * len(buffers)):
            F.fmlp_read_probe(buffers[i % len(buffers)], sink, wgs)
        torch.cuda.synchronize()
        F.fmlp_profile_enable(True)
        for i in range(steps):
            F.fmlp_read_probe(buffers[i % len(buffers)], sink, wgs)
        torch.cuda.synchronize()
        n, ms = F.fmlp_profile_read().get("read_probe", (0, 0.0))
        F.fmlp_profile_enable(False)
        if n:
            gbs = nbytes * n / (ms * 1e-3) / 1e9
            if best is None or gbs > best["gb_per_s"]:
                best = {"bytes_per_launch": nbytes, "workgroups": wgs,
                        "us_per_launch": round(ms * 1e3 / n, 3), "gb_per_s": round(gbs, 1)}
    return best


def default_steps(w, M):
    # ~1 s of timed GPU work per line, a whole number of rotations
    if M > 32:
        return 200, 20
    return 100 * w.sets, 4 * w.sets


def copy_calibration(mib):
    """Five plain copies of `mib` MiB between two fresh device buffers: each
    reads and writes exactly mib * 2^20 bytes, which makes it the yardstick
    for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the fused MLP here "
              "has no multi-GPU path, and every workload runs on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from swiglu_mlp_rmsnorm_amd import synth
    jobs = []
    if args.all:
        for wname, w in synth.WORKLOADS.items():
            for M in w.Ms:
                jobs.append((wname, M))
    else:
        w = synth.WORKLOADS[args.workload]
        jobs.append((args.workload, args.M if args.M is not None else w.Ms[0]))
    for wname, M in jobs:
        w = synth.WORKLOADS[wname]
        s, wu = default_steps(w, M)
        steps = args.steps if args.steps is not None else s
        warmup = args.warmup if args.warmup is not None else wu
        rec = run_one(wname, M, steps, warmup, args)
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
