"""Host-side checks of bench.py (no GPU): the byte and flop counts behind
its roofline figures against the figures worked out independently for the
workloads (the per-step table of the measurement plan, in decimal MB and
GFLOP), the lines `--all` prints, the refusal of more than one GPU, and the
comment-blind source hash that expires a committed traffic summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("d,ff,wtype,M,mb", [
    (3072, 8192, "bf16", 1, 151.01), (3072, 8192, "bf16", 8, 151.10),
    (4096, 14336, "bf16", 1, 352.35), (4096, 14336, "bf16", 32, 352.85),
    (4096, 14336, "bf16", 512, 360.72), (4096, 14336, "bf16", 2048, 385.88),
    (8192, 28672, "int4", 1, 396.41), (8192, 28672, "int4", 16, 396.90)])
def test_step_bytes_match_the_workload_table(d, ff, wtype, M, mb):
    assert round(bench.step_bytes(M, d, ff, wtype) / 1e6, 2) == mb


@pytest.mark.parametrize("d,ff,M,gflop", [(4096, 14336, 512, 180.39), (4096, 14336, 2048, 721.55),
                                          (8192, 28672, 16, 22.55)])
def test_step_flops_match_the_workload_table(d, ff, M, gflop):
    assert round(bench.step_flops(M, d, ff) / 1e9, 2) == gflop


def test_kernel_bytes_add_up_to_the_weights():
    # the two decode kernels of a step read each weight byte once between them
    for d, ff, wt in ((3072, 8192, "bf16"), (8192, 28672, "int4")):
        gu, dn = bench.weight_bytes(d, ff, wt)
        assert gu == 2 * dn  # gate and up rows against down, same element count
        M = 1
        total = (bench.kernel_bytes("decode_gateup_" + wt, M, d, ff, wt) +
                 bench.kernel_bytes("decode_down_" + wt, M, d, ff, wt))
        a_elem = 2 if wt == "int4" else 4
        # x (+ gamma), the intermediate written and read back, y
        act = M * d * 2 + (0 if wt == "int4" else d * 2) + 2 * M * ff * a_elem + M * d * 2
        assert total == gu + dn + act
    # int4: half a byte per weight plus one fp16 scale per 32
    gu, dn = bench.weight_bytes(8192, 28672, "int4")
    assert dn == 8192 * 28672 // 2 + 8192 * (28672 // 32) * 2


def test_gemm_bytes_follow_the_weight_type():
    d, ff, M = 8192, 28672, 512
    for wt in ("bf16", "int4"):
        gu, dn = bench.weight_bytes(d, ff, wt)
        assert bench.gemm_bytes("gemm_gateup_silu_f16", M, d, ff, wt) == gu + M * d * 2 + M * ff * 2
        assert bench.gemm_bytes("gemm_down_f16", M, d, ff, wt) == dn + M * ff * 2 + M * d * 2
    # int4 GEMMs read a quarter of the bf16 weight bytes plus one fp16 scale per 32
    assert (bench.gemm_bytes("gemm_down_f16", 0, d, ff, "int4") ==
            d * ff // 2 + d * (ff // 32) * 2)


def test_all_lines_cover_every_configuration():
    from swiglu_mlp_rmsnorm_amd import synth
    pairs = bench.all_pairs(synth.WORKLOADS)
    assert len(pairs) == len(set(pairs))
    for name, w in synth.WORKLOADS.items():
        assert all((name, M) in pairs for M in w.Ms)
    # int4 weights through the prefill GEMMs, at the prefill token counts
    assert ("llama70b_int4_decode_d8192_ff28672", 512) in pairs
    assert ("llama70b_int4_decode_d8192_ff28672", 2048) in pairs


def test_parity_rows_span_the_input():
    assert bench.parity_rows(5) == [0, 1, 2, 3, 4]
    rows = bench.parity_rows(2048)
    assert len(rows) == 16 and rows[0] == 0 and rows[-1] == 2047
    # one row in each of the eight 256-token tiles at least
    assert {r // 256 for r in rows} == set(range(8))
    assert rows == sorted(set(rows))


def test_cpu_leg_parity_of_the_oracle_own_rounded_output():
    # the CPU leg's parity on the tiny layer, fed the oracle's own y rounded
    # to bf16 for the sampled rows: only y's rounding remains (at most half a
    # bf16 ulp: 2^-8 relative, 8 significand bits), and the record carries
    # the bar
    import numpy as np
    import torch
    from oracle import oracle
    from swiglu_mlp_rmsnorm_amd import synth
    w = synth.WORKLOADS["tiny_d256_ff704"]
    M = 40
    host = tuple(synth.bits(t) for t in synth.layer_bf16(w, 0))
    x, g = (synth.bits(t) for t in synth.inputs(w, M))
    rows = bench.parity_rows(M)
    ref = oracle.forward_unfused(x[rows], g, synth.EPS, *host)
    y_rows = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    rec, par = bench.cpu_baseline(w, M, host, (x, g), 0.2, rows, y_rows)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["value_1core"] > 0
    assert par["rows"] == 16 and par["of_tokens"] == M and par["bar"] == bench.PARITY_BAR
    rel = np.abs(y_rows - ref) / np.maximum(np.abs(ref), 1e-30)
    assert rel.max() <= 2.0 ** -8
    assert 0 < par["l1_rel"] < 2e-3 and 0 < par["max_over_rms"] < 2e-2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no result line


def test_source_hash_ignores_comments_only():
    code = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    recommented = "/* helper */\nint f(int a) {\n\n  // add one\n  return a + 1;\n}\n"
    changed = "int f(int a) {\n  return a + 2;  // one more\n}\n"
    assert bench.code_only(code) == bench.code_only(recommented)
    assert bench.code_only(code) != bench.code_only(changed)
    assert "one more" not in bench.code_only(code)
