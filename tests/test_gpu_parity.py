"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact for packing, quantisation and dequantisation; within the accuracy
bar of parity_util for the forward pass, on both kernel paths, ragged token
counts, both int4 and bf16 weights, and the degenerate cases of Eq(1)."""
import numpy as np
import pytest
import torch

from oracle import oracle
from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import assert_parity, bf16_inputs, bf16_layer, oracle_bf16, oracle_int4

pytestmark = pytest.mark.gpu
EPS = synth.EPS
TINY_D, TINY_FF = 256, 704


@pytest.fixture(scope="module")
def tiny_layer():
    wg, wu, wd = bf16_layer(TINY_D, TINY_FF, 10)
    return wg, wu, F.fmlp_pack_interleaved(wg, wu), wd


# ----------------------------------------------------------------- packing

@pytest.mark.parametrize("ff,d", [(704, 256), (32, 32), (14336, 4096)])
def test_pack_bit_exact(ff, d):
    wg = synth.bf16_weight(ff, d, 1, "cuda")
    wu = synth.bf16_weight(ff, d, 2, "cuda")
    got = F.fmlp_pack_interleaved(wg, wu)
    torch.cuda.synchronize()
    ref = oracle.pack_interleaved(synth.bits(wg), synth.bits(wu))
    assert np.array_equal(synth.bits(got), ref)


# ----------------------------------------------------------------- int4

def test_quantize_bit_exact_random_and_ties():
    w = synth.bf16_weight(96, 704, 5, "cuda")
    # plant groups with exact ties (w/s = +-k.5) and an all-zero group
    ties = torch.tensor([0.875, 0.3125, -0.3125, 0.1875, -0.875, 0.0625] + [0.0] * 26)
    w[3, 0:32] = ties.to(torch.bfloat16).cuda()
    w[4, 32:64] = 0
    w[5, 64:96] = torch.linspace(-3, 3, 32).to(torch.bfloat16).cuda()
    q, s = F.fmlp_quantize_int4(w)
    st, q_ref, s_ref = oracle.quantize_int4(synth.bits(w))
    assert st == 0
    assert np.array_equal(synth.bits(q), q_ref)
    assert np.array_equal(synth.bits(s), s_ref)


def test_quantize_commutes_with_pack():
    wg = synth.bf16_weight(64, 256, 6, "cuda")
    wu = synth.bf16_weight(64, 256, 7, "cuda")
    q1, s1 = F.fmlp_quantize_int4(F.fmlp_pack_interleaved(wg, wu))
    qg, sg = F.fmlp_quantize_int4(wg)
    qu, su = F.fmlp_quantize_int4(wu)
    assert torch.equal(q1[0::2], qg) and torch.equal(q1[1::2], qu)
    assert torch.equal(s1[0::2], sg) and torch.equal(s1[1::2], su)


def test_quantize_range_error():
    w = torch.full((2, 64), 1e6, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FmlpError) as e:
        F.fmlp_quantize_int4(w)
    assert e.value.status == F.FMLP_ERR_RANGE
    w = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    w[1, 5] = float("nan")
    with pytest.raises(F.FmlpError):
        F.fmlp_quantize_int4(w)
    # a later valid call still works (the flag is reset per call)
    q, s = F.fmlp_quantize_int4(torch.ones((2, 64), dtype=torch.bfloat16, device="cuda"))
    assert torch.all(s == torch.tensor(1.0 / 7).half().cuda())


@pytest.mark.parametrize("rows,K", [(48, 256), (8192, 1024)])
def test_dequant_bit_exact(rows, K):
    q, s = synth.int4_weight(rows, K, 11, 12, "cuda")
    got = F.fmlp_dequant_int4(q, s)
    ref = oracle.dequant_int4(synth.bits(q), synth.bits(s))
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ----------------------------------------------------------------- forward bf16

@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32])
def test_decode_bf16_ragged(tiny_layer, M):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 100 + M)
    y = F.fmlp_forward(x, g, EPS, wgu, wd)
    assert_parity(y, oracle_bf16(x, g, EPS, wgu, wd), f"decode M={M}")


@pytest.mark.parametrize("M", [33, 63, 65, 127, 129, 200, 257])
def test_prefill_bf16_ragged(tiny_layer, M):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 200 + M)
    y = F.fmlp_forward(x, g, EPS, wgu, wd)
    assert_parity(y, oracle_bf16(x, g, EPS, wgu, wd), f"prefill M={M}")


@pytest.mark.parametrize("M,path", [(1, F.FMLP_PATH_PREFILL), (17, F.FMLP_PATH_PREFILL),
                                    (32, F.FMLP_PATH_PREFILL), (32, F.FMLP_PATH_DECODE),
                                    (33, F.FMLP_PATH_PREFILL)])
def test_both_paths_at_the_crossover(tiny_layer, M, path):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 300 + M)
    y = F.fmlp_forward_path(x, g, EPS, wgu, wd, path=path)
    assert_parity(y, oracle_bf16(x, g, EPS, wgu, wd), f"path={path} M={M}")


@pytest.mark.parametrize("d,ff,M", [(32, 32, 1), (64, 96, 3), (96, 160, 40), (512, 1376, 5),
                                    (512, 1376, 70)])
def test_odd_shapes(d, ff, M):
    wg, wu, wd = bf16_layer(d, ff, 20 + d)
    wgu = F.fmlp_pack_interleaved(wg, wu)
    x, g = bf16_inputs(M, d, 400 + M)
    y = F.fmlp_forward(x, g, EPS, wgu, wd)
    assert_parity(y, oracle_bf16(x, g, EPS, wgu, wd), f"d={d} ff={ff} M={M}")


def test_unfused_oracle_agrees_with_packed_gpu(tiny_layer):
    # the GPU result from the packed matrix matches Eq(1) on separate matrices
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(4, TINY_D, 77)
    y = F.fmlp_forward(x, g, EPS, wgu, wd)
    b = synth.bits
    ref = oracle.forward_unfused(b(x), b(g), EPS, b(wg), b(wu), b(wd))
    assert_parity(y, ref, "unfused")


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 5), (F.FMLP_PATH_PREFILL, 70)])
def test_zero_weight_and_zero_input_cases(tiny_layer, path, M):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 9)
    zero_gate = wgu.clone()
    zero_gate[0::2] = 0
    for args in ((x, zero_gate, wd), (x, wgu, torch.zeros_like(wd)),
                 (torch.zeros_like(x), wgu, wd)):
        y = F.fmlp_forward_path(args[0], g, EPS, args[1], args[2], path=path)
        assert torch.all(y == 0)


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 9), (F.FMLP_PATH_PREFILL, 100)])
def test_every_output_written_and_deterministic(tiny_layer, path, M):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 55)
    y1 = torch.full((M, TINY_D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((F.fmlp_workspace_size(M, TINY_D, TINY_FF),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    F.fmlp_forward_path(x, g, EPS, wgu, wd, y=y1, workspace=ws, path=path)
    assert torch.all(torch.isfinite(y1.float()))
    y2 = F.fmlp_forward_path(x, g, EPS, wgu, wd, path=path)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 6), (F.FMLP_PATH_PREFILL, 80)])
def test_nan_row_stays_in_its_row(tiny_layer, path, M):
    wg, wu, wgu, wd = tiny_layer
    x, g = bf16_inputs(M, TINY_D, 66)
    x[2, 7] = float("nan")
    y = F.fmlp_forward_path(x, g, EPS, wgu, wd, path=path).float()
    assert torch.all(torch.isnan(y[2]))
    keep = [m for m in range(M) if m != 2]
    assert torch.all(torch.isfinite(y[keep]))


def test_eps_zero_and_large_eps(tiny_layer):
    wg, wu, wgu, wd = tiny_layer
    for eps, M in ((0.0, 3), (0.5, 3), (0.0, 40)):
        x, g = bf16_inputs(M, TINY_D, 88)
        y = F.fmlp_forward(x, g, eps, wgu, wd)
        assert_parity(y, oracle_bf16(x, g, eps, wgu, wd), f"eps={eps} M={M}")


# ----------------------------------------------------------------- forward int4

@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 17, 32])
def test_decode_int4_ragged(M):
    d, ff = 256, 704
    q_gu, s_gu = synth.int4_weight(2 * ff, d, 30, 31, "cuda")
    q_d, s_d = synth.int4_weight(d, ff, 32, 33, "cuda")
    x, g = bf16_inputs(M, d, 500 + M)
    y = F.fmlp_forward(x, g, EPS, q_gu, q_d, s_gu, s_d)
    assert_parity(y, oracle_int4(x, g, EPS, q_gu, s_gu, q_d, s_d), f"int4 M={M}")


def test_int4_from_quantised_bf16_layer(tiny_layer):
    # end to end: quantise a bf16 layer with the library, run int4 forward,
    # compare with the oracle on the same codes
    wg, wu, wgu, wd = tiny_layer
    q_gu, s_gu = F.fmlp_quantize_int4(wgu)
    q_d, s_d = F.fmlp_quantize_int4(wd)
    x, g = bf16_inputs(3, TINY_D, 600)
    y = F.fmlp_forward(x, g, EPS, q_gu, q_d, s_gu, s_d)
    assert_parity(y, oracle_int4(x, g, EPS, q_gu, s_gu, q_d, s_d), "int4 quantised")
