"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (fmlp_forward, automatic path choice, weight set 0 of each workload).
Rows are independent, so the oracle runs on a sample of rows and the error
bar is evaluated over those rows."""
import numpy as np
import pytest
import torch

from oracle import oracle
from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import assert_parity

pytestmark = pytest.mark.gpu

CASES = [
    ("phi3mini_decode_d3072_ff8192", 1), ("phi3mini_decode_d3072_ff8192", 8),
    ("llama8b_decode_d4096_ff14336", 1), ("llama8b_decode_d4096_ff14336", 4),
    ("llama8b_decode_d4096_ff14336", 16), ("llama8b_decode_d4096_ff14336", 32),
    ("llama8b_prefill_d4096_ff14336", 512), ("llama8b_prefill_d4096_ff14336", 2048),
    ("llama70b_int4_decode_d8192_ff28672", 1), ("llama70b_int4_decode_d8192_ff28672", 16),
    # int4 weights on the prefill path (beyond the workload's own M values)
    ("llama70b_int4_decode_d8192_ff28672", 64),
]


def sample_rows(M, n):
    if M <= n:
        return list(range(M))
    return sorted(set(int(r) for r in np.linspace(0, M - 1, n)))


# the last of each decode workload's rotated weight sets as well as the first
LAST_SET_CASES = [(n, 1, synth.WORKLOADS[n].sets - 1) for n in (
    "phi3mini_decode_d3072_ff8192", "llama8b_decode_d4096_ff14336",
    "llama70b_int4_decode_d8192_ff28672")]


@pytest.mark.parametrize("wname,M,layer", [(n, M, 0) for n, M in CASES] + LAST_SET_CASES)
def test_full_size_parity(wname, M, layer):
    w = synth.WORKLOADS[wname]
    x, g = synth.inputs(w, M, "cuda", layer=layer)
    b = synth.bits
    if w.wtype == "int4":
        q_gu, s_gu, q_d, s_d = synth.layer_int4(w, layer, "cuda")
        y = F.fmlp_forward(x, g, synth.EPS, q_gu, q_d, s_gu, s_d, ff=w.ff)
        rows = sample_rows(M, 2)
        host = (*oracle.untile_int4(b(q_gu), b(s_gu), 2 * w.ff, w.d),
                *oracle.untile_int4(b(q_d), b(s_d), w.d, w.ff))
        ref = oracle.forward_int4(b(x)[rows], b(g), synth.EPS, *host)
    else:
        wg, wu, wd = synth.layer_bf16(w, layer, "cuda")
        y = F.fmlp_forward(x, g, synth.EPS, F.fmlp_pack_interleaved(wg, wu), F.fmlp_pack_matrix(wd))
        rows = sample_rows(M, 8 if M <= 32 else 4)
        ref = oracle.forward_unfused(b(x)[rows], b(g), synth.EPS, b(wg), b(wu), b(wd))
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(y.float()))
    mx, l1 = assert_parity(y[rows], ref, f"{wname} M={M} set {layer}")
    print(f"{wname} M={M} set {layer} rows={rows}: max/rms={mx:.3e} L1={l1:.3e}")


@pytest.mark.parametrize("wname,M", [("phi3mini_decode_d3072_ff8192", 1),
                                     ("phi3mini_decode_d3072_ff8192", 8),
                                     ("llama8b_decode_d4096_ff14336", 1),
                                     ("llama8b_decode_d4096_ff14336", 4)])
def test_full_size_single_pass(wname, M):
    w = synth.WORKLOADS[wname]
    x, g = synth.inputs(w, M, "cuda")
    b = synth.bits
    wg, wu, wd = synth.layer_bf16(w, 0, "cuda")
    y = F.fmlp_forward_path(x, g, synth.EPS, F.fmlp_pack_interleaved(wg, wu),
                            F.fmlp_pack_matrix(wd), path=F.FMLP_PATH_SINGLE_PASS)
    rows = sample_rows(M, 8)
    ref = oracle.forward_unfused(b(x)[rows], b(g), synth.EPS, b(wg), b(wu), b(wd))
    torch.cuda.synchronize()
    mx, l1 = assert_parity(y[rows], ref, f"single pass {wname} M={M}")
    print(f"single pass {wname} M={M}: max/rms={mx:.3e} L1={l1:.3e}")
