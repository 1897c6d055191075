#!/usr/bin/env python3
"""Benchmark of the fused gated-MLP forward on one MI355X.

One step = one fmlp_forward call (RMSNorm -> interleaved gate/up matmul ->
SiLU*mul -> down projection) on one layer, the weight set rotating every
step through `sets` distinct layers so the 256 MB Infinity Cache cannot serve
repeats. Inputs are resident in HBM before timing starts.

Prints ONE JSON line (stdout). Default: the Llama-3.1-8B-shaped prefill,
d=4096, ff=14336, M=2048 tokens (the MFMA half of the metric), with the
three decode M=1 workloads (Phi-3-mini-, Llama-3.1-8B- and 70B-int4-shaped;
the HBM half) measured in the same run and reported inside the same line
under "decode_m1". `--workload`/`--M` select one configuration alone;
`--all` prints one line per (workload, M), the 70B-shaped int4 layer also at
512 and 2048 tokens (its int4 weights through the prefill GEMMs).
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
DEFAULT_WORKLOAD = "llama8b_prefill_d4096_ff14336"
DEFAULT_M = 2048
DECODE_M1 = ("phi3mini_decode_d3072_ff8192", "llama8b_decode_d4096_ff14336",
             "llama70b_int4_decode_d8192_ff28672")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None,
                    help=f"one workload alone (default: {DEFAULT_WORKLOAD} M={DEFAULT_M} with the "
                         "decode M=1 lines)")
    ap.add_argument("--M", type=int, default=None)
    ap.add_argument("--all", action="store_true",
                    help="every (workload, M), prefill sizes included; one line each")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU-oracle baseline sample (all threads; the "
                         "one-thread figure takes a third of it)")
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
    writes y (its fp32 partial sums per 32-feature slice of ff are scratch
    traffic inside the launch, not counted, like the decode intermediate)."""
    gu, dn = weight_bytes(d, ff, wtype)
    f16 = wtype == "int4" if f16 is None else f16
    a_elem = 2 if f16 else 4
    if kernel == "decode_fused_bf16":
        return gu + dn + M * d * 2 + d * 2 + M * d * 2
    if "gateup" in kernel:
        act_in = M * d * 2 + (0 if f16 else d * 2)
        return gu + act_in + M * ff * a_elem
    if kernel == "act_prep":
        return M * d * 2 + d * 2 + M * d * 2
    return dn + M * ff * a_elem + M * d * 2


def gemm_bytes(kernel, M, d, ff, wtype="bf16"):
    """Algorithmic bytes of one prefill GEMM launch: its weights (bf16, or
    int4 codes and scales), fp16 activations in, its output (fp16 SiLU*mul
    product, or bf16 y)."""
    gu, dn = weight_bytes(d, ff, wtype)
    if kernel == "gemm_gateup_silu_f16":
        return gu + M * d * 2 + M * ff * 2
    return dn + M * ff * 2 + M * d * 2


def algorithmic_bytes(kernel, M, d, ff, wtype):
    if kernel.startswith("gemm"):
        return gemm_bytes(kernel, M, d, ff, wtype)
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
    }.get(kernel)
    if src is None:
        return None
    h = hashlib.sha256()
    for f in (src, "device_common.hpp"):
        text = open(os.path.join(ROOT, "swiglu_mlp_rmsnorm_amd", "csrc", f)).read()
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def code_only(text):
    """A C++ source without its comments and blank lines, so that editing a
    comment does not expire a measurement of the code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


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

# the accuracy bar of the forward (max |y - y_ref| over rms(y_ref), and the
# mean relative error sum |y - y_ref| / sum |y_ref|)
PARITY_BAR = {"max_over_rms": 2e-2, "l1_rel": 3e-3}


def parity_rows(M, n=16):
    """n token rows spread evenly over the M (all of them when M <= n)."""
    if M <= n:
        return list(range(M))
    return sorted({round(k * (M - 1) / (n - 1)) for k in range(n)})


def cpu_baseline(w, M, host_layer, host_inputs, budget_s, rows=None, y_rows=None):
    """Time the fp64 CPU oracle, as it stands, on a bounded sample of the same
    workload (weight set 0, the same seeded row-major weights and inputs):
    rows are independent, so it runs calls on consecutive row subsets until
    the budget is spent, first with every OpenMP thread, then with one.
    With `rows` and the GPU's y of those rows (`y_rows`, from the measured
    launch on the full input), the oracle's y of the same rows also gives the
    parity of the measured configuration on that sample: (record, parity)."""
    import numpy as np
    from oracle import oracle
    x, g = host_inputs
    if w.wtype == "int4":
        qg, sg, qu, su, qd, sd = host_layer
        q_gu, s_gu = oracle.pack_interleaved_int4(qg, sg, qu, su)

        def call(xs):
            return oracle.forward_int4(xs, g, w_eps(), q_gu, s_gu, qd, sd)
    else:
        wg, wu, wd = host_layer

        def call(xs):
            return oracle.forward_unfused(xs, g, w_eps(), wg, wu, wd)

    parity = None
    if rows is not None:
        y_ref = call(np.ascontiguousarray(x[rows]))
        err = np.abs(y_rows - y_ref)
        parity = {"rows": len(rows), "of_tokens": M,
                  "max_over_rms": float(err.max() / np.sqrt(np.mean(y_ref ** 2))),
                  "l1_rel": float(err.sum() / np.abs(y_ref).sum()), "bar": PARITY_BAR,
                  "note": "oracle (fp64) against the GPU's y of the measured launch, "
                          "weight set 0, rows spread evenly over the input"}

    def timed(rows_per_call, budget):
        done, calls = 0, 0
        t0 = time.perf_counter()
        while True:
            r0 = (calls * rows_per_call) % M
            xs = x[r0:r0 + rows_per_call]
            call(xs)
            done += xs.shape[0]
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return done, calls, el

    threads = oracle.threads()
    rows_per_call = min(M, 16)
    done, calls, el = timed(rows_per_call, budget_s)
    oracle.set_threads(1)
    try:
        done1, calls1, el1 = timed(1, budget_s / 3)
    finally:
        oracle.set_threads(threads)
    return {
        "value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "nproc": os.cpu_count(), "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
        "value_1core": done1 / el1,
        "sample": (f"{calls} oracle forward call(s) of {rows_per_call} row(s) of the {M}-token "
                   f"input on weight set 0 of {w.name} (fp64, {threads} threads, {el:.1f} s); "
                   f"then {calls1} call(s) of 1 row on 1 thread ({el1:.1f} s)"),
    }, parity


def w_eps():
    from swiglu_mlp_rmsnorm_amd import synth
    return synth.EPS


# ----------------------------------------------------------------------------- run

def build_layers(w, dev, w16, keep_host):
    """The rotated weight sets, packed by the library; with keep_host, also
    the host bits of set 0's row-major tensors (for the CPU baseline)."""
    from swiglu_mlp_rmsnorm_amd import fmlp as F
    from swiglu_mlp_rmsnorm_amd import synth
    layers, host0 = [], None
    for l in range(w.sets):
        if w.wtype == "int4":
            qg, sg, qu, su, qd, sd = synth.layer_int4(w, l, dev)
            layers.append((*F.fmlp_pack_int4_interleaved(qg, sg, qu, su),
                           *F.fmlp_pack_int4_matrix(qd, sd)))
            if l == 0 and keep_host:
                host0 = tuple(synth.bits(t) for t in (qg, sg, qu, su, qd, sd))
            del qg, sg, qu, su, qd, sd
        else:
            wg, wu, wd = synth.layer_bf16(w, l, dev)
            L = (F.fmlp_pack_interleaved(wg, wu), F.fmlp_pack_matrix(wd))
            if w16:  # (2 bytes per weight either way)
                L = (F.fmlp_convert_f16(L[0]), F.fmlp_convert_f16(L[1]))
            layers.append(L)
            if l == 0 and keep_host:
                host0 = (synth.bits(wg), synth.bits(wu), synth.bits(wd))
            del wg, wu, wd
    return layers, host0


def run_one(wname, M, steps, warmup, args, *, cpu=True, spread=True):
    """Measure one (workload, M): W warmup steps, then K timed steps with
    nothing but the forward calls between two stream events; then the same K
    steps again with the library's per-launch HIP events (dispatch start and
    end stamps on the launch stream), for the per-kernel durations. The
    events are kept out of the timed region: they add idle time between the
    launches (microseconds per launch), though not to the
    kernels' own durations, which agree with a rocprofv3 kernel trace."""
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
    cpu = cpu and not args.no_cpu_baseline and not ex  # the baseline times the plain Eq(1) step
    log(f"[bench] {wname} M={M}: building {w.sets} weight set(s)")
    layers, host0 = build_layers(w, dev, w16, cpu)
    xs = [synth.inputs(w, M, dev, layer=l) for l in range(w.sets)]
    torch.cuda.synchronize()
    y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    wt = F.FMLP_W_INT4_G32 if w.wtype == "int4" else F.FMLP_W_F16 if w16 else F.FMLP_W_BF16
    ws = torch.empty(F.fmlp_workspace_size(M, d, ff, wt), dtype=torch.uint8, device=dev)
    res = synth.activations(M, d, 977, dev) if args.residual else None
    hout = torch.empty((M, d), dtype=torch.bfloat16, device=dev) if args.residual else None
    if ex:
        fwd = functools.partial(F.fmlp_forward_ex, path=pcode or 0,
                                activation=ACTS[args.activation], residual=res, h_out=hout)
    elif pcode is None:
        fwd = F.fmlp_forward
    else:
        fwd = functools.partial(F.fmlp_forward_path, path=pcode)

    def step(i):
        L = layers[i % w.sets]
        x, g = xs[i % w.sets]
        if w.wtype == "int4":
            fwd(x, g, synth.EPS, L[0], L[2], L[1], L[3], y=y, workspace=ws, ff=ff)
        else:
            fwd(x, g, synth.EPS, L[0], L[1], y=y, workspace=ws)

    def collect_kernels(nsteps):
        out = {}
        for name, (n, ms) in F.fmlp_profile_read().items():
            # a kernel kind may launch more than once per step (the gate/up
            # GEMM's tail launch): rates below use its time per step
            out[name] = {"launches": n, "avg_us": ms * 1e3 / n,
                         "launches_per_step": n / nsteps, "us_per_step": ms * 1e3 / nsteps}
        return out

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
    kernels = {}
    ms_per_step = e0.elapsed_time(e1) / steps
    wall_ms_per_step = (t1 - t0) * 1e3 / steps
    tokens_per_s = M / (ms_per_step * 1e-3)
    sb = step_bytes(M, d, ff, w.wtype) + (4 * M * d if args.residual else 0)  # + r in, h out
    log(f"[bench] {ms_per_step*1e3:.2f} us/step (host wall {wall_ms_per_step*1e3:.2f}), "
        f"{sb / ms_per_step / 1e6:.1f} GB/s step")

    # per-kernel durations from HIP events recorded by the library on its launch stream
    if not args.no_profile:
        F.fmlp_profile_enable(True)
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        kernels = collect_kernels(steps)
        F.fmlp_profile_enable(False)
    # Spread: five more windows of the same length, after the timed region
    # (median, p10, p90 of their us/step); and the same steps captured once as
    # a HIP graph (one rotation of weight sets) and replayed, which shows what
    # host launch overhead the plain loop carries.
    spr = None
    if spread and not args.no_spread:
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
        spr = {"windows": 5, "steps_per_window": steps,
               "us_per_step_p10": round(win[0] + 0.4 * (win[1] - win[0]), 3),
               "us_per_step_median": round(win[2], 3),
               "us_per_step_p90": round(win[3] + 0.6 * (win[4] - win[3]), 3)}
        spr["graph_us_per_step"] = graph_us_per_step(step, w.sets, steps)
        log(f"[bench] spread {json.dumps(spr)}")

    if kernels:
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
    # The dominant kernel's algorithmic units per step over its time per step
    # (its launches in one step together: one for decode, one or two for the
    # gate/up GEMM), i.e. units per launch over the average launch duration
    # when it launches once per step.
    roofline = None
    if dom in kernels:
        step_s = kernels[dom]["us_per_step"] * 1e-6
        achieved = dom_units / step_s / (1e9 if unit == "GB/s" else 1e12)
        roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": unit, "frac": round(achieved / peak, 4),
                    "units_per_step": dom_units,
                    "launches_per_step": kernels[dom]["launches_per_step"],
                    "us_per_step": round(kernels[dom]["us_per_step"], 3),
                    "events": "the same K steps run again right after the timed region",
                    # (the committed counter runs are of the stored weight types)
                    "traffic": None if w16 else measured_traffic(dom, wname, M)}
    for name, k in kernels.items():
        t = k["us_per_step"]
        if name.startswith("decode") or name == "act_prep":
            k["gb_per_s"] = round(kernel_bytes(name, M, d, ff, w.wtype,
                                               w.wtype == "int4" or "act_prep" in kernels)
                                  / (t * 1e3), 1)
        elif name == "gemm_gateup_silu_f16":
            k["tflop_per_s"] = round(2.0 * M * 2 * ff * d / (t * 1e6), 1)
        elif name == "gemm_down_f16":
            k["tflop_per_s"] = round(2.0 * M * ff * d / (t * 1e6), 1)

    # The HBM read rate a plain streaming kernel reaches on exactly the bytes
    # the dominant decode kernel streams (the gate/up weights of each rotated
    # set, read once per launch), and on the whole step's weight bytes (both
    # matrices of each set read back to back): the practical ceilings the
    # roofline fractions should be read against.
    ceiling = None
    if path == "decode" and not args.no_profile:
        ceiling = read_ceiling([L[0] for L in layers], steps)
        whole = read_ceiling_step(layers, w.wtype, steps)
        if ceiling is not None:
            ceiling["step_weights"] = whole
        if roofline is not None and ceiling:
            ceiling["dominant_kernel_frac_of_ceiling"] = round(
                roofline["achieved"] / ceiling["gb_per_s"], 4)

    cpu_rec = parity = None
    if cpu:
        host_inputs = (synth.bits(xs[0][0]), synth.bits(xs[0][1]))
        # the GPU's y of weight set 0 from the measured launch (full input)
        step(0)
        torch.cuda.synchronize()
        rows = parity_rows(M)
        y_rows = y[rows].double().cpu().numpy()
        log(f"[bench] CPU oracle baseline ({args.cpu_seconds:.0f} s budget)")
        cpu_rec, parity = cpu_baseline(w, M, host0, host_inputs, args.cpu_seconds, rows, y_rows)

    step_gbs = sb / (ms_per_step * 1e-3) / 1e9
    step_tflops = step_flops(M, d, ff) / (ms_per_step * 1e-3) / 1e12
    # the whole step against the roofline of its bound (what the metric names)
    if bound == "mfma":
        step_roof = {"bound": "mfma", "achieved": round(step_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(step_tflops / MFMA_PEAK_TFLOPS, 4)}
    else:
        step_roof = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4)}
    dtype = ("int4-f16" if w.wtype == "int4" else
             "f16" if (w16 or path == "prefill" or "act_prep" in kernels) else "bf16")
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
        "dtype": dtype,
        "dtype_detail": ("MFMA operands: " + {
            "bf16": "bf16 weights x bf16 hi+lo activations",
            "f16": "fp16 (bf16 weights converted exactly in registers)",
            "int4-f16": "fp16 from int4 codes and fp16 group scales"}[dtype]
            + "; fp32 accumulation; bf16 x, gamma and y"),
        "data": "synthetic",
        "seeds": ("1_000_003 * workload + 1_009 * layer + tensor id (x 0, gamma 1, W_gate 2, "
                  f"W_up 3, W_down 4; int4 codes and scales 5-10); workload {w.index}"),
        "env": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                "gpu": torch.cuda.get_device_name(0),
                "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None)},
        "config": {"workload": wname, "M": M, "d": d, "ff": ff, "weight_sets": w.sets,
                   "wtype": "f16" if w16 else w.wtype, "path": path, "activation": args.activation,
                   "residual": bool(args.residual), "parallelism": "none (1 GPU)"},
        "step_gb_per_s": round(step_gbs, 1),
        "step_tflop_per_s": round(step_tflops, 2),
        "step_roofline": step_roof,
        "host_wall_ms_per_step": round(wall_ms_per_step, 6),
        "roofline": roofline,
        "read_ceiling": ceiling,
        "spread": spr,
        "kernels": kernels,
        "cpu_baseline": cpu_rec,
        "parity_sample": parity,
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


def _probe(buffers, steps, wgs_list):
    """fmlp_read_probe over each buffer list entry in turn (each entry a list
    of tensors read back to back), best rate over the grid sizes."""
    import torch
    from swiglu_mlp_rmsnorm_amd import fmlp as F
    nbytes = sum(t.numel() * t.element_size() for t in buffers[0])
    best = None
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=buffers[0][0].device)
    for wgs in wgs_list:
        for i in range(2 * len(buffers)):
            for t in buffers[i % len(buffers)]:
                F.fmlp_read_probe(t, sink, wgs)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            for t in buffers[i % len(buffers)]:
                F.fmlp_read_probe(t, sink, wgs)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        if best is None or gbs > best["gb_per_s"]:
            best = {"bytes_per_step": nbytes, "launches_per_step": len(buffers[0]),
                    "workgroups": wgs, "us_per_step": round(us, 3), "gb_per_s": round(gbs, 1)}
    return best


def read_ceiling(buffers, steps):
    """Streaming-read probe (fmlp_read_probe) over the rotated gate/up weight
    buffers, timed with the library's dispatch-stamped events; the best of
    three grid sizes."""
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


def read_ceiling_step(layers, wtype, steps):
    """The same probe over a whole step's weight bytes: each rotated set's
    W_gu and W_down (and int4 scales) read back to back, as one step's two
    launches read them, timed over the whole sequence with stream events (so
    the gaps between the launches count, as they do in a step)."""
    bufs = [list(L) for L in layers]  # bf16: (w_gu, w_down); int4: codes and scales
    return _probe(bufs, steps, (1024, 2048))


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


def all_pairs(workloads):
    """(workload, M) of every `--all` line: each workload's configured token
    counts, then those it also runs through the prefill GEMMs."""
    return [(name, M) for name, w in workloads.items() for M in w.Ms + w.prefill_Ms]


def decode_summary(rec):
    """The fields of a decode M=1 record that the default line nests."""
    keep = ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "step_gb_per_s",
            "step_roofline", "roofline", "read_ceiling", "spread", "kernels")
    out = {k: rec[k] for k in keep}
    out["config"] = rec["config"]
    return out


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

    def steps_for(wname, M):
        s, wu = default_steps(synth.WORKLOADS[wname], M)
        return (args.steps if args.steps is not None else s,
                args.warmup if args.warmup is not None else wu)

    if args.all:
        for wname, M in all_pairs(synth.WORKLOADS):
            st, wu = steps_for(wname, M)
            print(json.dumps(run_one(wname, M, st, wu, args)), flush=True)
        return
    if args.workload is not None:
        w = synth.WORKLOADS[args.workload]
        M = args.M if args.M is not None else w.Ms[0]
        st, wu = steps_for(args.workload, M)
        print(json.dumps(run_one(args.workload, M, st, wu, args)), flush=True)
        return
    # default: the prefill headline, then the decode M=1 workloads (their own
    # default step counts: whole rotations of their weight sets), one line
    M = args.M if args.M is not None else DEFAULT_M
    st, wu = steps_for(DEFAULT_WORKLOAD, M)
    rec = run_one(DEFAULT_WORKLOAD, M, st, wu, args)
    dec = {}
    for wname in DECODE_M1:
        s, wu2 = default_steps(synth.WORKLOADS[wname], 1)
        dec[wname] = decode_summary(run_one(wname, 1, s, wu2, args, cpu=False))
    rec["decode_m1"] = dec
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
