"""fmlp_forward_noalloc (the entry point that allocates nothing; its scratch
is the library's fixed device array) against fmlp_forward on the same
inputs, through the C ABI: two calls in a row on each weight type, the
second on a smaller problem, each compared bit for bit with fmlp_forward
(same kernels, same path) and with the oracle to the accuracy bar."""
import ctypes

import pytest
import torch

from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import Bf16Layer, F16Layer, Int4Layer, assert_parity, bf16_inputs

pytestmark = pytest.mark.gpu
EPS = synth.EPS


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(layer, x, g):
    """The new entry point, called through ctypes on the C ABI directly."""
    M, d = x.shape
    y = torch.full((M, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    if isinstance(layer, Int4Layer):
        args = (F.FMLP_W_INT4_G32, layer.q_gu, layer.s_gu, layer.q_d, layer.s_d)
    elif isinstance(layer, F16Layer):
        args = (F.FMLP_W_F16, layer.hgu_t, None, layer.hd_t, None)
    else:
        args = (F.FMLP_W_BF16, layer.wgu_t, None, layer.wd_t, None)
    wt, wgu, sgu, wd, sd = args
    st = F.lib().fmlp_forward_noalloc(_ptr(x), _ptr(g), EPS, wt, _ptr(wgu), _ptr(sgu), _ptr(wd),
                                      _ptr(sd), _ptr(y), M, d, layer.ff,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == F.FMLP_OK, F.fmlp_status_string(st)
    return y


@pytest.mark.parametrize("kind", ["bf16", "int4", "f16"])
@pytest.mark.parametrize("big,small", [((1024, 2048, 17), (256, 704, 3)),   # decode, split down
                                       ((256, 704, 70), (256, 704, 1)),     # prefill, then decode
                                       ((3072, 8192, 8), (3072, 8192, 1))])  # Phi-3 shape
def test_noalloc_matches_forward_twice(kind, big, small):
    cls = {"bf16": Bf16Layer, "int4": Int4Layer, "f16": F16Layer}[kind]
    for i, (d, ff, M) in enumerate((big, small)):
        layer = cls(d, ff, 200 + d + i)
        x, g = bf16_inputs(M, d, 210 + M + i)
        y_na = _noalloc(layer, x, g)
        torch.cuda.synchronize()
        y_ref = layer.forward(x, g, EPS)
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), \
            f"{kind} d={d} ff={ff} M={M}: differs from fmlp_forward"
        assert_parity(y_na, layer.oracle(x, g, EPS), f"noalloc {kind} d={d} ff={ff} M={M}")


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    # Llama-8B-shaped prefill at 2048 tokens needs far more than the scratch
    d, ff, M = 4096, 14336, 2048
    assert F.fmlp_workspace_size(M, d, ff) > F.FMLP_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    g = torch.ones((d,), dtype=torch.bfloat16, device="cuda")
    wgu = torch.zeros((2 * ff, d), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((d, ff), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FmlpError) as e:
        F.fmlp_forward_noalloc(x, g, EPS, wgu, wd)
    assert e.value.status == F.FMLP_ERR_WORKSPACE
    # and the entry point still works after the rejection
    layer = Bf16Layer(256, 704, 230)
    x, g = bf16_inputs(5, 256, 231)
    y = F.fmlp_forward_noalloc(x, g, EPS, layer.wgu_t, layer.wd_t)
    assert torch.equal(y.view(torch.int16), layer.forward(x, g, EPS).view(torch.int16))
