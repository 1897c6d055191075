"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact for packing/tiling, quantisation and dequantisation; within the
accuracy bar of parity_util for the forward pass, on both kernel paths,
ragged token counts, bf16 and int4 weights, and the degenerate cases of
Eq(1). The oracle only ever sees the seeded inputs (host copies)."""
import numpy as np
import pytest
import torch

from oracle import oracle
from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

from parity_util import Bf16Layer, Int4Layer, assert_parity, bf16_inputs

pytestmark = pytest.mark.gpu
EPS = synth.EPS
TINY_D, TINY_FF = 256, 704


@pytest.fixture(scope="module")
def tiny():
    return Bf16Layer(TINY_D, TINY_FF, 10)


# ----------------------------------------------------------------- packing / tiling

@pytest.mark.parametrize("ff,d", [(704, 256), (32, 32), (64, 96), (14336, 4096)])
def test_pack_interleaved_bit_exact(ff, d):
    wg = synth.bf16_weight(ff, d, 1, "cuda")
    wu = synth.bf16_weight(ff, d, 2, "cuda")
    got = F.fmlp_pack_interleaved(wg, wu)
    torch.cuda.synchronize()
    b = synth.bits
    ref = oracle.tile_bf16(oracle.pack_interleaved(b(wg), b(wu)))
    assert np.array_equal(b(got).reshape(-1), ref)


@pytest.mark.parametrize("R,K", [(256, 704), (16, 32), (4096, 14336)])
def test_pack_matrix_bit_exact(R, K):
    w = synth.bf16_weight(R, K, 3, "cuda")
    got = F.fmlp_pack_matrix(w)
    assert np.array_equal(synth.bits(got).reshape(-1), oracle.tile_bf16(synth.bits(w)))


# ----------------------------------------------------------------- int4

@pytest.mark.parametrize("R,K", [(96, 704), (16, 128), (64, 4096), (5, 64), (1, 32)])
def test_quantize_bit_exact(R, K):
    # row-major in and out (the exchange format), any row count
    w = synth.bf16_weight(R, K, 5, "cuda")
    if R > 5:
        # exact ties (w/s = +-k.5), an all-zero group, a ramp
        ties = torch.tensor([0.875, 0.3125, -0.3125, 0.1875, -0.875, 0.0625] + [0.0] * 26)
        w[3, 0:32] = ties.to(torch.bfloat16).cuda()
        w[4, 32:64] = 0
        w[5, 64:96] = torch.linspace(-3, 3, 32).to(torch.bfloat16).cuda()
    q, s = F.fmlp_quantize_int4(w)
    st, q_ref, s_ref = oracle.quantize_int4(synth.bits(w))
    assert st == 0
    assert np.array_equal(synth.bits(q), q_ref)
    assert np.array_equal(synth.bits(s), s_ref)


def test_quantize_commutes_with_interleave():
    # quantising the row-interleaved matrix = interleaving the quantised rows
    wg = synth.bf16_weight(64, 256, 6, "cuda")
    wu = synth.bf16_weight(64, 256, 7, "cuda")
    w_il = torch.empty((128, 256), dtype=torch.bfloat16, device="cuda")
    w_il[0::2], w_il[1::2] = wg, wu
    q1, s1 = F.fmlp_quantize_int4(w_il)
    (qg, sg), (qu, su) = F.fmlp_quantize_int4(wg), F.fmlp_quantize_int4(wu)
    assert torch.equal(q1[0::2], qg) and torch.equal(q1[1::2], qu)
    assert torch.equal(s1[0::2].view(torch.int16), sg.view(torch.int16))
    assert torch.equal(s1[1::2].view(torch.int16), su.view(torch.int16))
    # and the tiled forms agree: pack_int4_interleaved(gate, up) == pack_int4_matrix(interleaved)
    a = F.fmlp_pack_int4_interleaved(qg, sg, qu, su)
    b = F.fmlp_pack_int4_matrix(q1, s1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


def test_quantize_range_error():
    w = torch.full((16, 64), 1e6, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FmlpError) as e:
        F.fmlp_quantize_int4(w)
    assert e.value.status == F.FMLP_ERR_RANGE
    w = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    w[1, 5] = float("nan")
    with pytest.raises(F.FmlpError):
        F.fmlp_quantize_int4(w)
    # a later valid call works again (the flag is reset per call)
    q, s = F.fmlp_quantize_int4(torch.ones((16, 128), dtype=torch.bfloat16, device="cuda"))
    assert torch.all(s == torch.tensor(1.0 / 7).half().cuda())


@pytest.mark.parametrize("R,K", [(48, 704), (8192, 1024), (3, 96)])
def test_dequant_bit_exact(R, K):
    q, s = synth.int4_weight(R, K, 11, 12, "cuda")
    got = F.fmlp_dequant_int4(q, s)
    ref = oracle.dequant_int4(synth.bits(q), synth.bits(s))
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("R,K", [(16, 32), (48, 704), (64, 4096), (8192, 28672)])
def test_pack_int4_matrix_bit_exact(R, K):
    # K = 704 and 32 leave padding groups in the last super-tile: zero codes and scales
    q, s = synth.int4_weight(R, K, 13, 14, "cuda")
    qt, st = F.fmlp_pack_int4_matrix(q, s)
    qt_ref, st_ref = oracle.tile_int4(synth.bits(q), synth.bits(s))
    assert np.array_equal(synth.bits(qt), qt_ref)
    assert np.array_equal(synth.bits(st), st_ref)


@pytest.mark.parametrize("ff,d", [(32, 32), (704, 256), (28672, 8192)])
def test_pack_int4_interleaved_bit_exact(ff, d):
    qg, sg = synth.int4_weight(ff, d, 15, 16, "cuda")
    qu, su = synth.int4_weight(ff, d, 17, 18, "cuda")
    qt, st = F.fmlp_pack_int4_interleaved(qg, sg, qu, su)
    b = synth.bits
    q_il, s_il = oracle.pack_interleaved_int4(b(qg), b(sg), b(qu), b(su))
    qt_ref, st_ref = oracle.tile_int4(q_il, s_il)
    assert np.array_equal(synth.bits(qt), qt_ref)
    assert np.array_equal(synth.bits(st), st_ref)


# ----------------------------------------------------------------- forward bf16

@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32])
def test_decode_bf16_ragged(tiny, M):
    x, g = bf16_inputs(M, TINY_D, 100 + M)
    assert_parity(tiny.forward(x, g, EPS), tiny.oracle(x, g, EPS), f"decode M={M}")


@pytest.mark.parametrize("M", [33, 63, 65, 127, 129, 200, 257])
def test_prefill_bf16_ragged(tiny, M):
    x, g = bf16_inputs(M, TINY_D, 200 + M)
    assert_parity(tiny.forward(x, g, EPS), tiny.oracle(x, g, EPS), f"prefill M={M}")


@pytest.mark.parametrize("M,path", [(1, F.FMLP_PATH_PREFILL), (17, F.FMLP_PATH_PREFILL),
                                    (32, F.FMLP_PATH_PREFILL), (32, F.FMLP_PATH_DECODE),
                                    (33, F.FMLP_PATH_PREFILL)])
def test_both_paths_at_the_crossover(tiny, M, path):
    x, g = bf16_inputs(M, TINY_D, 300 + M)
    assert_parity(tiny.forward(x, g, EPS, path=path), tiny.oracle(x, g, EPS), f"path={path} M={M}")


@pytest.mark.parametrize("d,ff,M", [(32, 32, 1), (64, 96, 3), (96, 160, 40), (512, 1376, 5),
                                    (512, 1376, 70), (160, 224, 17), (256, 4096, 100),
                                    (288, 2048, 33), (256, 38400, 33),
                                    # d past 8192: the prefill RMSNorm stores each token
                                    # row without staging the workgroup's rows in LDS
                                    (8224, 512, 40),
                                    # >= 768 gate/up workgroups: the 4-wave gate/up launch
                                    (256, 6144, 1), (96, 6176, 3),
                                    # staged gate/up activations with more chunks than
                                    # the staging registers hold
                                    (4096, 1024, 3),
                                    # a K split of the down projection whose equal
                                    # slices would leave the last one empty
                                    (32, 3104, 1),
                                    # 2ff/16 = 1032 row blocks: the eight-block gate/up
                                    # workgroups at two token blocks (M > 16)
                                    (64, 8256, 17), (64, 8256, 32), (64, 8256, 9),
                                    # more than 256 four-block gate/up workgroups: the
                                    # large-M gate/up settings from two tokens on
                                    (64, 8256, 2), (64, 8256, 4)])
def test_odd_shapes(d, ff, M):
    layer = Bf16Layer(d, ff, 20 + d)
    x, g = bf16_inputs(M, d, 400 + M)
    assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS), f"d={d} ff={ff} M={M}")


@pytest.mark.parametrize("M", [1, 3, 17, 32])
def test_decode_split_down(M):
    # d/16 = 64 row blocks on 256 CUs: the down projection splits K four ways
    # across workgroups and the last slice to arrive sums the partials
    layer = Bf16Layer(1024, 2048, 77)
    x, g = bf16_inputs(M, 1024, 700 + M)
    y1 = layer.forward(x, g, EPS)
    assert_parity(y1, layer.oracle(x, g, EPS), f"split down M={M}")
    assert torch.equal(y1.view(torch.int16), layer.forward(x, g, EPS).view(torch.int16))


SP = F.FMLP_PATH_SINGLE_PASS


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8])
def test_single_pass_ragged(tiny, M):
    # ff = 704: 22 slices of 32 features; d = 256: 16 down row blocks over 8 waves
    x, g = bf16_inputs(M, TINY_D, 150 + M)
    assert_parity(tiny.forward(x, g, EPS, path=SP), tiny.oracle(x, g, EPS), f"single pass M={M}")


@pytest.mark.parametrize("d,ff,M", [(32, 32, 1), (64, 96, 3), (96, 160, 8), (512, 1376, 5),
                                    (1024, 2048, 2), (288, 2048, 1), (4128, 64, 1),
                                    (3072, 8192, 1)])
def test_single_pass_shapes(d, ff, M):
    # d = 32: most waves own no down row block; d = 4128: 258 row blocks,
    # more down tiles per wave than it keeps in flight
    layer = Bf16Layer(d, ff, 30 + d)
    x, g = bf16_inputs(M, d, 450 + M)
    y1 = layer.forward(x, g, EPS, path=SP)
    assert_parity(y1, layer.oracle(x, g, EPS), f"single pass d={d} ff={ff} M={M}")
    assert torch.equal(y1.view(torch.int16), layer.forward(x, g, EPS, path=SP).view(torch.int16))


def test_single_pass_matches_two_kernel_path_closely(tiny):
    # same operand precision (bf16 hi + lo activations, fp32 accumulation):
    # the two decode variants differ only in summation order
    x, g = bf16_inputs(4, TINY_D, 160)
    y1 = tiny.forward(x, g, EPS, path=SP).float()
    y2 = tiny.forward(x, g, EPS, path=F.FMLP_PATH_DECODE).float()
    rms = float(y2.pow(2).mean().sqrt())
    assert float((y1 - y2).abs().max()) <= 2 ** -7 * rms


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 5), (F.FMLP_PATH_PREFILL, 70), (SP, 3)])
def test_zero_weight_and_zero_input_cases(tiny, path, M):
    x, g = bf16_inputs(M, TINY_D, 9)
    zero_gate = F.fmlp_pack_interleaved(torch.zeros_like(tiny.wg), tiny.wu)
    zero_up = F.fmlp_pack_interleaved(tiny.wg, torch.zeros_like(tiny.wu))
    zero_down = torch.zeros_like(tiny.wd_t)
    for xx, wgu, wd in ((x, zero_gate, tiny.wd_t), (x, zero_up, tiny.wd_t),
                        (x, tiny.wgu_t, zero_down), (torch.zeros_like(x), tiny.wgu_t, tiny.wd_t)):
        y = F.fmlp_forward_path(xx, g, EPS, wgu, wd, path=path)
        assert torch.all(y == 0)


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 9), (F.FMLP_PATH_DECODE, 32),
                                    (F.FMLP_PATH_PREFILL, 100), (SP, 1), (SP, 8)])
def test_every_output_written_and_deterministic(tiny, path, M):
    x, g = bf16_inputs(M, TINY_D, 55)
    y1 = torch.full((M, TINY_D), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((F.fmlp_workspace_size(M, TINY_D, TINY_FF),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    tiny.forward(x, g, EPS, y=y1, workspace=ws, path=path)
    assert torch.all(torch.isfinite(y1.float()))
    y2 = tiny.forward(x, g, EPS, path=path)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 6), (F.FMLP_PATH_PREFILL, 80), (SP, 6)])
def test_nan_row_stays_in_its_row(tiny, path, M):
    x, g = bf16_inputs(M, TINY_D, 66)
    x[2, 7] = float("nan")
    y = tiny.forward(x, g, EPS, path=path).float()
    assert torch.all(torch.isnan(y[2]))
    keep = [m for m in range(M) if m != 2]
    assert torch.all(torch.isfinite(y[keep]))


def test_eps_zero_and_large_eps(tiny):
    for eps, M in ((0.0, 3), (0.5, 3), (0.0, 40)):
        x, g = bf16_inputs(M, TINY_D, 88)
        assert_parity(tiny.forward(x, g, eps), tiny.oracle(x, g, eps), f"eps={eps} M={M}")


# ----------------------------------------------------------------- forward int4

@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 17, 32])
def test_decode_int4_ragged(M):
    layer = Int4Layer(TINY_D, TINY_FF, 30)
    x, g = bf16_inputs(M, TINY_D, 500 + M)
    assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS), f"int4 M={M}")


@pytest.mark.parametrize("d,ff,M", [(128, 128, 1), (384, 640, 7), (256, 1024, 32), (1024, 2048, 1),
                                    (1024, 2048, 20),
                                    # activations staged in LDS (M <= 4) with more chunks
                                    # than the staging registers hold: gate/up at d=8192,
                                    # and a 4-way K-split down projection at ff=20480
                                    (8192, 256, 3), (1024, 20480, 4), (1024, 20480, 2),
                                    (4096, 1056, 1),
                                    # a K split of the down projection whose equal
                                    # slices would leave the last one empty (25 K units
                                    # over 6 slices): the split count is recomputed
                                    (32, 3104, 1), (32, 3104, 3)])
def test_decode_int4_shapes(d, ff, M):
    layer = Int4Layer(d, ff, 40 + d)
    x, g = bf16_inputs(M, d, 550 + M)
    assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS), f"int4 d={d} ff={ff} M={M}")


@pytest.mark.parametrize("M,path", [(33, F.FMLP_PATH_AUTO), (70, F.FMLP_PATH_AUTO),
                                    (200, F.FMLP_PATH_AUTO), (1, F.FMLP_PATH_PREFILL),
                                    (32, F.FMLP_PATH_PREFILL)])
def test_prefill_int4(M, path):
    # int4 on the MFMA path: the GEMMs dequantise the codes in their operand path
    layer = Int4Layer(TINY_D, TINY_FF, 31)
    x, g = bf16_inputs(M, TINY_D, 800 + M)
    assert_parity(layer.forward(x, g, EPS, path=path), layer.oracle(x, g, EPS),
                  f"int4 prefill M={M}")


@pytest.mark.parametrize("d,ff,M", [(512, 1376, 70), (256, 4096, 100)])
def test_prefill_int4_shapes(d, ff, M):
    layer = Int4Layer(d, ff, 50 + d)
    x, g = bf16_inputs(M, d, 850 + M)
    assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS), f"int4 prefill d={d} ff={ff}")


@pytest.mark.parametrize("M", [512, 2048])
def test_prefill_int4_large_m(M):
    # the int4 prefill path at the token counts of the prefill workload, all
    # rows, on a layer small enough for the oracle (8 x 28 weight row bands)
    layer = Int4Layer(1024, 3584, 57)
    x, g = bf16_inputs(M, 1024, 860 + M)
    assert_parity(layer.forward(x, g, EPS), layer.oracle(x, g, EPS), f"int4 prefill M={M}")


@pytest.mark.parametrize("d,ff,M", [(256, 704, 70), (1024, 3584, 512), (8192, 1024, 40),
                                    (96, 160, 33)])
def test_int4_prefill_equals_fp16_weights_of_s_times_q(d, ff, M):
    # The int4 GEMMs expand each weight to fp16(s * q) (the exact product,
    # rounded once to nearest even) inside their operand path. The same
    # values stored as fp16 weights (dequantised exactly, rounded by torch,
    # tiled) through the fp16-weight GEMMs must give y bit for bit.
    layer = Int4Layer(d, ff, 70 + d)
    q_il = torch.empty((2 * ff, d // 2), dtype=torch.uint8, device="cuda")
    s_il = torch.empty((2 * ff, d // 32), dtype=torch.float16, device="cuda")
    q_il[0::2], q_il[1::2] = layer.q_g, layer.q_u
    s_il[0::2], s_il[1::2] = layer.s_g, layer.s_u

    def tiled_f16(q, s):
        w16 = F.fmlp_dequant_int4(q, s).half()
        return F.fmlp_pack_matrix(w16.view(torch.bfloat16)).view(torch.float16)

    wgu16, wd16 = tiled_f16(q_il, s_il), tiled_f16(layer.q_dn, layer.s_dn)
    x, g = bf16_inputs(M, d, 870 + M)
    for path in (F.FMLP_PATH_PREFILL, F.FMLP_PATH_AUTO):
        y4 = layer.forward(x, g, EPS, path=path)
        y16 = F.fmlp_forward_path(x, g, EPS, wgu16, wd16, path=F.FMLP_PATH_PREFILL)
        if path == F.FMLP_PATH_PREFILL or M > 32:
            assert torch.equal(y4.view(torch.int16), y16.view(torch.int16))


def test_int4_end_to_end_from_bf16(tiny):
    # quantise gate, up and down with the library in the exchange format,
    # pack, run; the oracle quantises the same seeded bf16 weights itself
    # and runs Eq(1) on its own codes
    (qg, sg), (qu, su) = F.fmlp_quantize_int4(tiny.wg), F.fmlp_quantize_int4(tiny.wu)
    qd, sd = F.fmlp_quantize_int4(tiny.wd)
    q_gu, s_gu = F.fmlp_pack_int4_interleaved(qg, sg, qu, su)
    q_d, s_d = F.fmlp_pack_int4_matrix(qd, sd)
    wg, wu, wd = tiny.host
    _, qg_o, sg_o = oracle.quantize_int4(oracle.pack_interleaved(wg, wu))
    _, qd_o, sd_o = oracle.quantize_int4(wd)
    x, g = bf16_inputs(3, TINY_D, 600)
    y = F.fmlp_forward(x, g, EPS, q_gu, q_d, s_gu, s_d, ff=TINY_FF)
    b = synth.bits
    assert_parity(y, oracle.forward_int4(b(x), b(g), EPS, qg_o, sg_o, qd_o, sd_o), "int4 e2e")


# ----------------------------------------------------------------- variants
# Gate activation (SiLU / GELU tanh form / GELU erf form) and the residual
# prologue h = bf16_rne(x + r) on every path; h is compared bit for bit.

def _check_ex(layer, M, d, act, with_res, seed, **kw):
    x, g = bf16_inputs(M, d, seed)
    res = synth.activations(M, d, seed + 7, "cuda") if with_res else None
    y, h = layer.forward_ex(x, g, EPS, activation=act, residual=res, **kw)
    ref, href = layer.oracle_ex(x, g, EPS, act, res)
    assert_parity(y, ref, f"act={act} res={with_res} M={M} {kw}")
    if with_res:
        assert np.array_equal(synth.bits(h), href), "residual stream differs"
    else:
        assert h is None


@pytest.mark.parametrize("act", [F.FMLP_ACT_SILU, F.FMLP_ACT_GELU_TANH, F.FMLP_ACT_GELU_ERF])
@pytest.mark.parametrize("with_res", [False, True])
@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 3), (F.FMLP_PATH_DECODE, 20),
                                    (SP, 2), (F.FMLP_PATH_PREFILL, 70)])
def test_variants_bf16(tiny, act, with_res, path, M):
    _check_ex(tiny, M, TINY_D, act, with_res, 900 + M, path=path)


@pytest.mark.parametrize("act", [F.FMLP_ACT_GELU_TANH, F.FMLP_ACT_GELU_ERF])
@pytest.mark.parametrize("with_res", [False, True])
@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 1), (F.FMLP_PATH_DECODE, 9),
                                    (F.FMLP_PATH_DECODE, 17), (F.FMLP_PATH_PREFILL, 40)])
def test_variants_int4(act, with_res, path, M):
    layer = Int4Layer(1024, 2048, 61)
    _check_ex(layer, M, 1024, act, with_res, 930 + M, path=path)


@pytest.mark.parametrize("act", [F.FMLP_ACT_SILU, F.FMLP_ACT_GELU_TANH, F.FMLP_ACT_GELU_ERF])
@pytest.mark.parametrize("path,M", [(F.FMLP_PATH_DECODE, 3), (F.FMLP_PATH_DECODE, 20),
                                    (F.FMLP_PATH_PREFILL, 70)])
def test_gate_activations_over_a_wide_range(act, path, M):
    # W_gate ten times larger: the gate pre-activations span about +-10, the
    # range where the kernels' sigmoid and erf approximations (hardware exp
    # and reciprocal; the Abramowitz-Stegun erf) meet both tails, against
    # the oracle's exact functions
    layer = Bf16Layer(TINY_D, TINY_FF, 64)
    layer.wg = (layer.wg.float() * 10.0).to(torch.bfloat16)
    layer.wgu_t = F.fmlp_pack_interleaved(layer.wg, layer.wu)
    layer.host = (synth.bits(layer.wg),) + layer.host[1:]
    x, g = bf16_inputs(M, TINY_D, 990 + M)
    xf, gf = x.float().cpu(), g.float().cpu()
    n = xf * torch.rsqrt(xf.pow(2).mean(1, keepdim=True) + EPS) * gf
    z = n @ layer.wg.float().cpu().T
    assert float(z.abs().max()) > 8.0  # the test reaches the tails
    y, _ = layer.forward_ex(x, g, EPS, activation=act, path=path)
    ref, _ = layer.oracle_ex(x, g, EPS, act, None)
    assert_parity(y, ref, f"wide gate act={act} path={path} M={M}")


@pytest.mark.parametrize("d,ff,M", [(3072, 8192, 1), (4096, 1024, 16), (18432, 64, 2),
                                    (256, 6144, 2)])
def test_residual_stream_bit_exact_at_larger_d(d, ff, M):
    # d = 18432 makes the int4 prep take its second pass over the row
    _check_ex(Bf16Layer(d, ff, 62), M, d, F.FMLP_ACT_GELU_ERF, True, 960 + M)
    _check_ex(Int4Layer(d, ff, 63), M, d, F.FMLP_ACT_SILU, True, 970 + M)


# 2 ff / 256 = 258 bands of gate/up rows at one token tile: one round of
# 256 x 256 tiles and the last two bands as 256 x 128 tail tiles, both in
# the gate/up GEMM's single launch, for every weight kind and gate epilogue
TAIL_D, TAIL_FF, TAIL_M = 64, 33024, 40


@pytest.fixture(scope="module")
def tail_layers():
    from parity_util import F16Layer
    return {"bf16": Bf16Layer(TAIL_D, TAIL_FF, 91), "f16": F16Layer(TAIL_D, TAIL_FF, 91),
            "int4": Int4Layer(TAIL_D, TAIL_FF, 92)}


@pytest.mark.parametrize("wt", ["bf16", "f16", "int4"])
@pytest.mark.parametrize("act", [F.FMLP_ACT_SILU, F.FMLP_ACT_GELU_ERF])
def test_gateup_tail_tiles_in_one_launch(tail_layers, wt, act):
    L = tail_layers[wt]
    x, g = bf16_inputs(TAIL_M, TAIL_D, 930)
    y, _ = L.forward_ex(x, g, EPS, activation=act)
    ref, _ = L.oracle_ex(x, g, EPS, act, None)
    assert_parity(y, ref, f"{wt} act={act} with tail tiles")


def test_gateup_tail_tiles_f16_weights_equal_bf16(tail_layers):
    # on the prefill path the fp16 store is the GEMM's own weight conversion,
    # so both weight kinds give the same bits through the merged launch
    L = tail_layers["f16"]
    x, g = bf16_inputs(TAIL_M, TAIL_D, 931)
    y16 = L.forward(x, g, EPS)
    y = L.forward_bf16(x, g, EPS)
    assert torch.equal(y16.view(torch.int16), y.view(torch.int16))
