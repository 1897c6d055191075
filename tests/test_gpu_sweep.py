"""GPU parity over a grid of layer shapes and token counts that crosses the
launch planners' thresholds, on the automatic path (decode up to 32 tokens,
prefill above), bf16 and int4 weights, every case against the oracle at the
accuracy bar of parity_util.

The grid: d of one 32-column block, of one 256-row down tile, and of eight
tiles plus a 32-row remainder (2, 16 and 130 down row blocks of 16 for the
decode kernels, all split along K); ff of 224, 2048 and 4352 (28, 256 and
544 gate/up row blocks of 16, and a part-filled 256-row band for the prefill
GEMMs); token counts at both sides of the decode settings' switches (1, 2, 5,
17 and 32 tokens), of the decode/prefill crossover (33) and of the prefill
planner's 128-token bands (130, 257). Over this grid the down GEMM's plan
takes all three tile shapes (256 x 256, 256 x 128, 128 x 128) and 1-, 4- and
8-way K splits (the 2-way split is the Llama-8B M=2048 plan of the full-size
tests)."""
import itertools

import pytest

from swiglu_mlp_rmsnorm_amd import synth

from parity_util import Bf16Layer, Int4Layer, assert_parity, bf16_inputs

pytestmark = pytest.mark.gpu
EPS = synth.EPS

D = (32, 256, 2080)
FF = (224, 2048, 4352)
M_BF16 = (1, 2, 5, 17, 32, 33, 130, 257)
D_INT4 = (128, 2080)
FF_INT4 = (224, 2048)
M_INT4 = (1, 5, 17, 33, 130)


@pytest.mark.parametrize("d,ff", list(itertools.product(D, FF)))
def test_sweep_bf16(d, ff):
    layer = Bf16Layer(d, ff, 900 + d + ff)
    for M in M_BF16:
        x, g = bf16_inputs(M, d, 1000 + M)
        assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS),
                      f"bf16 d={d} ff={ff} M={M}")


@pytest.mark.parametrize("d,ff", list(itertools.product(D_INT4, FF_INT4)))
def test_sweep_int4(d, ff):
    layer = Int4Layer(d, ff, 950 + d + ff)
    for M in M_INT4:
        x, g = bf16_inputs(M, d, 1100 + M)
        assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS),
                      f"int4 d={d} ff={ff} M={M}")
