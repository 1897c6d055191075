"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (fmlp_forward, automatic path choice, a workspace of
fmlp_workspace_size bytes, weight sets 0 and the last rotated one).

The accuracy bar is evaluated over the whole [M, d] output of every case:
the oracle (OpenMP over outputs, tokens in chunks that share each weight
row's decoding) runs on all rows on the host once the GPU result has been
copied back. Besides every configured (workload, M), int4 weights on the
prefill path run at the 70B shape at M = 64, 512 and 2048."""
import numpy as np
import pytest
import torch

from oracle import oracle
from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import assert_parity

pytestmark = pytest.mark.gpu

# every (workload, M) the workloads configure, on weight set 0
CASES = [(name, M, 0) for name, w in synth.WORKLOADS.items() for M in w.Ms]
# the last of each decode workload's rotated weight sets as well
CASES += [(n, 1, synth.WORKLOADS[n].sets - 1) for n in (
    "phi3mini_decode_d3072_ff8192", "llama8b_decode_d4096_ff14336",
    "llama70b_int4_decode_d8192_ff28672")]
# int4 weights on the prefill path at the 70B shape, all rows
CASES += [("llama70b_int4_decode_d8192_ff28672", M, 0) for M in (64, 512, 2048)]


class FullLayer:
    """One weight set of a workload: device copies packed by the library, and
    the host bits of the same seeded tensors for the oracle."""

    def __init__(self, w, layer):
        self.w = w
        b = synth.bits
        if w.wtype == "int4":
            qg, sg, qu, su, qd, sd = synth.layer_int4(w, layer, "cuda")
            self.dev = (*F.fmlp_pack_int4_interleaved(qg, sg, qu, su),
                        *F.fmlp_pack_int4_matrix(qd, sd))
            q_gu, s_gu = oracle.pack_interleaved_int4(b(qg), b(sg), b(qu), b(su))
            self.host = (q_gu, s_gu, b(qd), b(sd))
        else:
            wg, wu, wd = synth.layer_bf16(w, layer, "cuda")
            self.dev = (F.fmlp_pack_interleaved(wg, wu), F.fmlp_pack_matrix(wd))
            self.host = (b(wg), b(wu), b(wd))

    def forward(self, x, g):
        w = self.w
        wt = F.FMLP_W_INT4_G32 if w.wtype == "int4" else F.FMLP_W_BF16
        ws = torch.empty(F.fmlp_workspace_size(x.shape[0], w.d, w.ff, wt), dtype=torch.uint8,
                         device="cuda")
        if w.wtype == "int4":
            q_gu, s_gu, q_d, s_d = self.dev
            return F.fmlp_forward(x, g, synth.EPS, q_gu, q_d, s_gu, s_d, ff=w.ff, workspace=ws)
        return F.fmlp_forward(x, g, synth.EPS, *self.dev, workspace=ws)

    def oracle(self, xb, gb):
        if self.w.wtype == "int4":
            return oracle.forward_int4(xb, gb, synth.EPS, *self.host)
        return oracle.forward_unfused(xb, gb, synth.EPS, *self.host)


@pytest.mark.parametrize("wname,M,layer", CASES)
def test_full_size_parity_all_rows(wname, M, layer):
    w = synth.WORKLOADS[wname]
    print(f"[fullsize] {wname} M={M} set {layer}: GPU forward", flush=True)
    L = FullLayer(w, layer)
    x, g = synth.inputs(w, M, "cuda", layer=layer)
    y = L.forward(x, g)
    torch.cuda.synchronize()
    print(f"[fullsize] {wname} M={M}: oracle on all {M} rows", flush=True)
    ref = L.oracle(synth.bits(x), synth.bits(g))
    mx, l1 = assert_parity(y, ref, f"{wname} M={M} set {layer} (all rows)")
    print(f"[fullsize] {wname} M={M} set {layer}: max/rms={mx:.3e} L1={l1:.3e}", flush=True)


@pytest.mark.parametrize("wname,M", [("phi3mini_decode_d3072_ff8192", 1),
                                     ("phi3mini_decode_d3072_ff8192", 8),
                                     ("llama8b_decode_d4096_ff14336", 1),
                                     ("llama8b_decode_d4096_ff14336", 4),
                                     ("llama8b_tp8_shard_decode_d4096_ff1792", 1)])
def test_full_size_single_pass_all_rows(wname, M):
    w = synth.WORKLOADS[wname]
    L = FullLayer(w, 0)
    x, g = synth.inputs(w, M, "cuda")
    y = F.fmlp_forward_path(x, g, synth.EPS, *L.dev, path=F.FMLP_PATH_SINGLE_PASS)
    torch.cuda.synchronize()
    mx, l1 = assert_parity(y, L.oracle(synth.bits(x), synth.bits(g)), f"single pass {wname} M={M}")
    print(f"[fullsize] single pass {wname} M={M}: max/rms={mx:.3e} L1={l1:.3e}", flush=True)
