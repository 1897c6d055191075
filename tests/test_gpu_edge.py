"""Edge cases of Eq(1) on the GPU, against the oracle, on every path:

* an all-zero input row with eps = 0: mean(x^2) + eps = 0, the normalisation
  divides zero by zero and the row is NaN, as the closed form is (the
  oracle's own row is NaN too); every other row is unaffected;
* an input row whose SiLU*mul intermediate exceeds the fp16 range: the paths
  that carry the intermediate in fp16 (prefill, decode above 16 tokens,
  int4 decode, fp16 weights) turn that row of y non-finite (inf or NaN),
  never into a finite wrong value; the bf16 decode path up to 16 tokens
  (bf16 hi + lo intermediate, the range of fp32) returns the oracle's
  values. Other rows stay within the accuracy bar on every path.
All buffers carry guard regions (parity_util.guarded_call)."""
import numpy as np
import pytest
import torch

from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import Bf16Layer, F16Layer, Int4Layer, assert_parity, bf16_inputs

pytestmark = pytest.mark.gpu
D, FF = 256, 704
SP = F.FMLP_PATH_SINGLE_PASS
DEC, PRE = F.FMLP_PATH_DECODE, F.FMLP_PATH_PREFILL


@pytest.fixture(scope="module")
def layers():
    return {"bf16": Bf16Layer(D, FF, 110), "int4": Int4Layer(D, FF, 111),
            "f16": F16Layer(D, FF, 112)}


def _rows_except(y, ref, bad, what):
    keep = [m for m in range(y.shape[0]) if m not in bad]
    if keep:
        assert_parity(y[keep], ref[keep], what)


@pytest.mark.parametrize("wt,path,M", [("bf16", DEC, 5), ("bf16", DEC, 20), ("bf16", PRE, 40),
                                       ("bf16", SP, 3), ("int4", DEC, 3), ("int4", DEC, 20),
                                       ("int4", PRE, 40), ("f16", DEC, 4), ("f16", PRE, 40)])
def test_zero_row_with_zero_eps_is_nan(layers, wt, path, M):
    L = layers[wt]
    x, g = bf16_inputs(M, D, 120 + M)
    x[2] = 0
    y = L.forward(x, g, 0.0, path=path)
    ref = L.oracle(x, g, 0.0)
    assert np.all(np.isnan(ref[2])), "the closed form gives NaN for this row"
    assert torch.all(torch.isnan(y[2].float())), f"{wt} path={path}: row 2 not NaN"
    _rows_except(y, ref, {2}, f"{wt} path={path} M={M}, zero row 2, eps=0")


def _overflow_layer(kind):
    """Weights whose gate/up feature 0 rows are 2 * sign(x row 0): for x row 0
    (all entries +-1, so r = 1 at eps = 0) the gate and up sums reach
    2 * sum(gamma) ~ 512 and their product ~ 2.6e5, past fp16's 65504; for
    random rows they stay ~ 2 * sqrt(d) = 32 (products ~ 1e3)."""
    L = {"bf16": Bf16Layer, "f16": F16Layer}[kind](D, FF, 113)
    return L


def _overflow_inputs(M):
    x, g = bf16_inputs(M, D, 130 + M)
    sign = torch.where(torch.arange(D, device="cuda") % 3 == 0, -1.0, 1.0)
    x[0] = sign.to(torch.bfloat16)
    return x, g, sign


def _plant(L, sign):
    L.wg[0] = (2 * sign).to(torch.bfloat16)
    L.wu[0] = (2 * sign).to(torch.bfloat16)
    L.wgu_t = F.fmlp_pack_interleaved(L.wg, L.wu)
    L.host = tuple(synth.bits(t) for t in (L.wg, L.wu, L.wd))
    if isinstance(L, F16Layer):
        from oracle import oracle
        L.hgu_t = F.fmlp_convert_f16(L.wgu_t)
        hgu, bad = oracle.bf16_to_f16_trunc(oracle.pack_interleaved(*L.host[:2]))
        assert bad == 0
        L.host16 = (hgu, L.host16[1])


def _a_row_max(L, x, g):
    """max |SiLU(g_i) u_i| per row, in float64 (test-side, from the same bits)."""
    xv = x.double()
    n = xv / xv.pow(2).mean(dim=1, keepdim=True).sqrt() * g.double()
    gg, uu = n @ L.wg.double().T, n @ L.wu.double().T
    return (torch.nn.functional.silu(gg) * uu).abs().max(dim=1).values


@pytest.mark.parametrize("kind,path,M,row0_finite", [
    ("bf16", DEC, 4, True), ("bf16", DEC, 16, True),      # bf16 hi + lo intermediate
    ("bf16", SP, 4, True),
    ("bf16", DEC, 20, False), ("bf16", PRE, 40, False),  # fp16 intermediate
    ("bf16", PRE, 4, False), ("f16", DEC, 4, False), ("f16", PRE, 40, False)])
def test_intermediate_beyond_fp16_range(kind, path, M, row0_finite):
    L = _overflow_layer(kind)
    x, g, sign = _overflow_inputs(M)
    _plant(L, sign)
    amax = _a_row_max(L, x, g)
    assert amax[0] > 2 * 65504 and torch.all(amax[1:] < 32768), amax
    y = L.forward(x, g, 0.0, path=path)
    ref = L.oracle(x, g, 0.0)
    if row0_finite:
        assert_parity(y, ref, f"{kind} path={path} M={M}, large intermediate")
    else:
        assert not torch.any(torch.isfinite(y[0].float())), "row 0 must be non-finite"
        _rows_except(y, ref, {0}, f"{kind} path={path} M={M}, other rows")


@pytest.mark.parametrize("path,M", [(DEC, 1), (DEC, 20), (PRE, 40)])
def test_int4_intermediate_beyond_fp16_range(path, M):
    # int4 codes of feature 0 set to +-7 along sign(x row 0), scale 0.25:
    # gate and up sums ~ 1.75 * sum(gamma), product ~ 2e5; int4 carries n and
    # a in fp16 on every path, so row 0 is non-finite there
    L = Int4Layer(D, FF, 114)
    x, g, sign = _overflow_inputs(M)
    code = torch.where(sign > 0, 7, 9).to(torch.uint8)  # 9 = -7 in two's complement
    packed = (code[0::2] | (code[1::2] << 4)).to(torch.uint8)
    for q, s in ((L.q_g, L.s_g), (L.q_u, L.s_u)):
        q[0] = packed
        s[0] = 0.25
    L.q_gu, L.s_gu = F.fmlp_pack_int4_interleaved(L.q_g, L.s_g, L.q_u, L.s_u)
    from oracle import oracle
    b = synth.bits
    L.host = (*oracle.pack_interleaved_int4(b(L.q_g), b(L.s_g), b(L.q_u), b(L.s_u)),
              *L.host[2:])
    y = L.forward(x, g, 0.0, path=path)
    ref = L.oracle(x, g, 0.0)
    assert np.abs(ref[0]).max() > 0  # the oracle's row is finite
    assert not torch.any(torch.isfinite(y[0].float())), "row 0 must be non-finite"
    _rows_except(y, ref, {0}, f"int4 path={path} M={M}, other rows")
