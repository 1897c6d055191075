"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties the oracle to a closed form derived by hand, an invariant of
Eq(1), a library routine that computes a special case, or the definition of a
storage format (IEEE binary16 via numpy). The operation is Eq(1) of the
FastTPS review (xllm-io paper-review blog, section 3) with the RMSNorm
prologue of the MLP-block flow / Figure 4 on the same page; the gate/up row
interleave follows the llama.cpp PR digest (blog.cecily.jp).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def bf16_bits(a) -> np.ndarray:
    t = torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def rand_bf16(shape, std, seed, mean=0.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g) * std + mean).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def sigmoid_closed(t):
    return 1.0 / (1.0 + math.exp(-t))


# ------------------------------------------------------------ scalar formats

def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = bf16_values(bits)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_decode_matches_numpy_every_pattern():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f32_to_f16_rne_matches_numpy():
    # numpy's float32 -> float16 cast rounds to nearest even (IEEE default).
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(3.0),
        (rng.random(2000).astype(np.float32) * np.float32(1e-4)),   # subnormal range
        np.float32(2.0) ** rng.integers(-30, 17, 500).astype(np.float32),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, np.inf, -np.inf],
                 dtype=np.float32),
    ])
    # exact ties between two fp16 neighbours: midpoints m + 0.5 ulp
    mids = (np.arange(1024, 2048, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10)
    vals = np.concatenate([vals, mids, -mids]).astype(np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------ SiLU

def test_silu_closed_form_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, abs=1e-15)
    assert oracle.silu(-1.0) == pytest.approx(-0.2689414213699951, abs=1e-15)
    for t in (-7.5, -0.3, 0.25, 2.0, 9.0):
        assert oracle.silu(t) == pytest.approx(t * sigmoid_closed(t), rel=1e-15)
    # limits: SiLU(t) -> t for large t, -> 0 (no NaN) for very negative t
    assert oracle.silu(60.0) == pytest.approx(60.0, rel=1e-15)
    v = oracle.silu(-800.0)
    assert v == 0.0 and not math.isnan(v)


def test_silu_matches_torch():
    t = torch.linspace(-30, 30, 1001, dtype=torch.float64)
    ref = F.silu(t).numpy()
    got = np.array([oracle.silu(float(v)) for v in t])
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------ RMSNorm

def test_rmsnorm_unit_rms_before_gamma():
    # mean(n^2) with gamma = 1 equals ms/(ms+eps) exactly (closed form)
    x = bf16_bits([[3.0, 4.0]])
    g = bf16_bits([1.0, 1.0])
    n = oracle.rmsnorm(x, g, 1e-5)
    assert np.mean(n ** 2) == pytest.approx(12.5 / (12.5 + 1e-5), rel=1e-14)
    assert np.mean(n ** 2) == pytest.approx(0.999999200000640, abs=1e-14)
    xr = rand_bf16((5, 96), 1.7, 11)
    n0 = oracle.rmsnorm(xr, bf16_bits(np.ones(96)), 0.0)
    np.testing.assert_allclose(np.mean(n0 ** 2, axis=1), 1.0, rtol=1e-13)


def test_rmsnorm_matches_torch_library():
    x = rand_bf16((4, 64), 2.0, 3)
    g = rand_bf16((64,), 0.1, 4, mean=1.0)
    for eps in (0.0, 1e-5, 0.3):
        ref = F.rms_norm(torch.from_numpy(bf16_values(x)), (64,),
                         torch.from_numpy(bf16_values(g)), eps).numpy()
        np.testing.assert_allclose(oracle.rmsnorm(x, g, eps), ref, rtol=1e-13)


# ------------------------------------------------------------ hand cases

def _hand(name):
    c = GOLDEN[name]
    return (bf16_bits(c["x"]), bf16_bits(c["gamma"]), bf16_bits(c["w_gate"]),
            bf16_bits(c["w_up"]), bf16_bits(c["w_down"]))


def silu(t):
    return t * sigmoid_closed(t)


@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_h1_closed_form(eps):
    x, g, wg, wu, wd = _hand("H1")
    s = math.sqrt(12.5 + eps)
    a = silu(3.0 / s) * (4.0 / s)
    expect = np.array([[a, 2 * a]])
    y = oracle.forward_unfused(x, g, eps, wg, wu, wd)
    np.testing.assert_allclose(y, expect, rtol=1e-14)
    wgu = oracle.pack_interleaved(wg, wu)
    assert np.array_equal(bf16_values(wgu), [[1.0, 0.0], [0.0, 1.0]])
    np.testing.assert_allclose(oracle.forward_bf16(x, g, eps, wgu, wd), expect, rtol=1e-14)
    # values quoted for this case to 12 digits
    if eps == 0.0:
        assert y[0, 0] == pytest.approx(0.672247962807, abs=1e-12)
    else:
        assert y[0, 0] == pytest.approx(0.672247356617, abs=1e-12)


def test_h2_closed_form_and_interleave():
    x, g, wg, wu, wd = _hand("H2")
    s = math.sqrt(2.5)
    n = np.array([1.0, -1.0, 4.0, -1.0]) / s
    a0 = silu(n[0]) * n[1]
    a1 = silu(n[2]) * (-n[3])
    expect = np.array([[a0, a1, a0 + a1, 0.5 * a0 - 0.5 * a1]])
    y = oracle.forward_unfused(x, g, 0.0, wg, wu, wd)
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=1e-15)
    wgu = oracle.pack_interleaved(wg, wu)
    rows = bf16_values(wgu)
    np.testing.assert_array_equal(rows[0], bf16_values(wg)[0])
    np.testing.assert_array_equal(rows[1], bf16_values(wu)[0])
    np.testing.assert_array_equal(rows[2], bf16_values(wg)[1])
    np.testing.assert_array_equal(rows[3], bf16_values(wu)[1])
    np.testing.assert_allclose(oracle.forward_bf16(x, g, 0.0, wgu, wd), expect, rtol=1e-14,
                               atol=1e-15)
    assert y[0, 3] == pytest.approx(-0.871574165255, abs=1e-12)


# ------------------------------------------------------------ invariants

def _rand_layer(M, d, ff, seed):
    return (rand_bf16((M, d), 1.0, seed), rand_bf16((d,), 0.1, seed + 1, mean=1.0),
            rand_bf16((ff, d), 0.05, seed + 2), rand_bf16((ff, d), 0.05, seed + 3),
            rand_bf16((d, ff), 0.05, seed + 4))


def test_zero_weights_give_zero_output():
    x, g, wg, wu, wd = _rand_layer(3, 32, 24, 100)
    z_ff = np.zeros_like(wg)
    z_d = np.zeros_like(wd)
    for args in ((z_ff, wu, wd), (wg, z_ff, wd), (wg, wu, z_d)):
        y = oracle.forward_unfused(x, g, 1e-5, *args)
        assert np.all(y == 0.0)
    y = oracle.forward_unfused(np.zeros_like(x), g, 1e-5, wg, wu, wd)
    assert np.all(y == 0.0)


def test_interleaved_equals_unfused_bitwise():
    x, g, wg, wu, wd = _rand_layer(4, 64, 40, 200)
    wgu = oracle.pack_interleaved(wg, wu)
    np.testing.assert_array_equal(oracle.forward_bf16(x, g, 1e-5, wgu, wd),
                                  oracle.forward_unfused(x, g, 1e-5, wg, wu, wd))


def test_ff_permutation_invariance():
    x, g, wg, wu, wd = _rand_layer(2, 32, 48, 300)
    perm = np.random.default_rng(1).permutation(48)
    y = oracle.forward_unfused(x, g, 1e-5, wg, wu, wd)
    yp = oracle.forward_unfused(x, g, 1e-5, wg[perm], wu[perm],
                                np.ascontiguousarray(wd[:, perm]))
    np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-14)


def test_rows_independent_and_linear_in_w_down():
    x, g, wg, wu, wd = _rand_layer(5, 32, 16, 400)
    y = oracle.forward_unfused(x, g, 1e-5, wg, wu, wd)
    for m in range(5):
        np.testing.assert_array_equal(oracle.forward_unfused(x[m:m + 1], g, 1e-5, wg, wu, wd),
                                      y[m:m + 1])
    # 2*W_down is exact in bf16, so y doubles exactly
    wd2 = bf16_bits(2.0 * bf16_values(wd))
    np.testing.assert_array_equal(oracle.forward_unfused(x, g, 1e-5, wg, wu, wd2), 2.0 * y)


def test_scale_invariance_with_zero_eps():
    x, g, wg, wu, wd = _rand_layer(3, 32, 16, 500)
    x4 = bf16_bits(4.0 * bf16_values(x))   # exact in bf16
    np.testing.assert_allclose(oracle.forward_unfused(x4, g, 0.0, wg, wu, wd),
                               oracle.forward_unfused(x, g, 0.0, wg, wu, wd), rtol=1e-13,
                               atol=1e-15)


# (37 rows: the oracle takes tokens 16 at a time, so this crosses two chunk
# boundaries and ends in a partial chunk)
@pytest.mark.parametrize("M,d,ff,seed", [(1, 32, 32, 1), (3, 64, 96, 2), (2, 256, 704, 3),
                                         (37, 64, 96, 4)])
def test_matches_torch_fp64_composition(M, d, ff, seed):
    # An independent implementation from library routines: rms_norm, matmul, silu.
    x, g, wg, wu, wd = _rand_layer(M, d, ff, 600 + seed)
    X, G, WG, WU, WD = (torch.from_numpy(bf16_values(a)) for a in (x, g, wg, wu, wd))
    n = F.rms_norm(X, (d,), G, 1e-5)
    ref = (F.silu(n @ WG.T) * (n @ WU.T)) @ WD.T
    y = oracle.forward_unfused(x, g, 1e-5, wg, wu, wd)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-13 * np.abs(ref.numpy()).max())


# ------------------------------------------------------------ packing

def test_pack_matches_numpy_slicing():
    wg = rand_bf16((40, 64), 1.0, 7)
    wu = rand_bf16((40, 64), 1.0, 8)
    p = oracle.pack_interleaved(wg, wu)
    assert np.array_equal(p[0::2], wg) and np.array_equal(p[1::2], wu)


# ------------------------------------------------------------ int4

def test_q1_ties_to_even():
    c = GOLDEN["Q1"]
    st, q, s = oracle.quantize_int4(bf16_bits([c["w"]]))
    assert st == 0
    assert s.view(np.float16)[0, 0] == np.float16(c["scale"])
    deq = oracle.dequant_int4(q, s)
    np.testing.assert_array_equal(deq[0], np.array(c["q"], np.float32) * np.float32(0.125))
    # nibble layout: even k low nibble, two's complement
    assert q[0, 0] == (7 | ((2 & 0xF) << 4))
    assert q[0, 1] == ((-2 & 0xF) | (2 << 4))


def _nibbles(q):
    lo = (q & 0xF).astype(np.int32)
    hi = (q >> 4).astype(np.int32)
    v = np.empty((q.shape[0], q.shape[1] * 2), np.int32)
    v[:, 0::2], v[:, 1::2] = lo, hi
    return np.where(v >= 8, v - 16, v)


def test_quantize_is_nearest_with_ties_even():
    w = rand_bf16((16, 256), 0.02, 9)
    st, q, s = oracle.quantize_int4(w)
    assert st == 0
    wv = bf16_values(w).astype(np.float32).reshape(16, 8, 32)
    # the scale: fp16(fp32(max|w|) / fp32(7)) computed with numpy
    mx = np.abs(wv).max(axis=2)
    np.testing.assert_array_equal(s, (mx / np.float32(7)).astype(np.float16).view(np.uint16))
    sv = s.view(np.float16).astype(np.float32)[:, :, None]
    qv = _nibbles(q).reshape(16, 8, 32)
    ratio = wv / sv                      # fp32 division, as the definition says
    # brute force: q is the integer in [-8,7] nearest to w/s, ties to even
    cand = np.arange(-8, 8)
    dist = np.abs(ratio[..., None] - cand)
    best = dist.min(axis=-1, keepdims=True)
    ok = dist == best
    choice = np.where(ok.sum(-1) == 1, cand[ok.argmax(-1)],
                      np.where(ok & (cand % 2 == 0), cand, 99).min(-1))
    np.testing.assert_array_equal(qv, choice)
    # round-trip error at most half a step
    assert np.all(np.abs(wv - sv * qv) <= sv / 2 + 1e-12)


def test_quantize_zero_group_and_range_error():
    st, q, s = oracle.quantize_int4(np.zeros((2, 64), np.uint16))
    assert st == 0 and np.all(q == 0) and np.all(s == 0)
    big = bf16_bits(np.full((1, 32), 1e6))
    assert oracle.quantize_int4(big)[0] == oracle.RANGE_ERROR
    inf = bf16_bits(np.array([[np.inf] + [0.0] * 31]))
    assert oracle.quantize_int4(inf)[0] == oracle.RANGE_ERROR


def test_quantize_commutes_with_interleave():
    wg = rand_bf16((24, 128), 0.02, 12)
    wu = rand_bf16((24, 128), 0.02, 13)
    st1, q1, s1 = oracle.quantize_int4(oracle.pack_interleaved(wg, wu))
    _, qg, sg = oracle.quantize_int4(wg)
    _, qu, su = oracle.quantize_int4(wu)
    assert st1 == 0
    assert np.array_equal(q1[0::2], qg) and np.array_equal(q1[1::2], qu)
    assert np.array_equal(s1[0::2], sg) and np.array_equal(s1[1::2], su)


def test_dequant_is_exact_product():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (8, 64), dtype=np.uint8)
    s = (rng.random((8, 4)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    deq = oracle.dequant_int4(q, s)
    ref = (np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)
           * _nibbles(q).astype(np.float64))
    np.testing.assert_array_equal(deq.astype(np.float64), ref)


def test_int4_forward_matches_torch_composition():
    rng = np.random.default_rng(6)
    M, d, ff = 2, 64, 96
    x = rand_bf16((M, d), 1.0, 20)
    g = rand_bf16((d,), 0.1, 21, mean=1.0)
    q_gu = rng.integers(0, 256, (2 * ff, d // 2), dtype=np.uint8)
    s_gu = (rng.random((2 * ff, d // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    q_d = rng.integers(0, 256, (d, ff // 2), dtype=np.uint8)
    s_d = (rng.random((d, ff // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    wgu = np.repeat(s_gu.view(np.float16).astype(np.float64), 32, 1) * _nibbles(q_gu)
    wdn = np.repeat(s_d.view(np.float16).astype(np.float64), 32, 1) * _nibbles(q_d)
    n = F.rms_norm(torch.from_numpy(bf16_values(x)), (d,), torch.from_numpy(bf16_values(g)), 1e-5)
    WGU = torch.from_numpy(wgu)
    ref = (F.silu(n @ WGU[0::2].T) * (n @ WGU[1::2].T)) @ torch.from_numpy(wdn).T
    y = oracle.forward_int4(x, g, 1e-5, q_gu, s_gu, q_d, s_d)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-11, atol=1e-13 * np.abs(ref.numpy()).max())


# ------------------------------------------------------------ tiled layouts
# Positions worked out by hand from the layout definition (16-row x 32-column
# tiles; slot L = 16*((k%32)/8) + r%16 of 8 consecutive columns).

def test_tile_bf16_positions_by_hand():
    R, K = 32, 96
    w = np.arange(R * K, dtype=np.uint16).reshape(R, K)
    t = oracle.tile_bf16(w)
    # (r=17, k=45): tile (1, 1) -> index 1*3+1 = 4; slot 16*1 + 1 = 17; offset 5
    assert t[4 * 512 + 17 * 8 + 5] == w[17, 45]
    # (r=0, k=8): tile 0, slot 16, offset 0
    assert t[16 * 8] == w[0, 8]
    # (r=15, k=95): tile (0, 2) -> 2; slot 16*3 + 15 = 63; offset 7
    assert t[2 * 512 + 63 * 8 + 7] == w[15, 95]
    assert np.array_equal(oracle.untile_bf16(t, R, K), w)
    assert sorted(t.tolist()) == list(range(R * K))  # a permutation


def test_tile_int4_positions_by_hand():
    R, K = 32, 256          # nq = 2 super-tiles per 16-row block
    q = np.zeros((R, K // 2), np.uint8)
    s = np.zeros((R, K // 32), np.uint16)
    q[5, 70 // 2] = 0x0B    # code (5, 70) = 0xB (-5), even k -> low nibble
    s[21, 6] = 0x1234       # scale (21, group 6)
    qt, st = oracle.tile_int4(q, s)
    # (5, 70): g = 2 -> super-tile 0; slot 16*((70%32)//8) + 5 = 5; word 5*4 + 2 = 22;
    # nibble 70%8 = 6 -> byte 22*4 + 3 = 91, low nibble
    assert qt[91] == 0x0B and np.count_nonzero(qt) == 1
    # scale (21, 6): super-tile (1, 1) -> 1*2 + 1 = 3; element 3*64 + 5*4 + 2 = 214
    assert st[214] == 0x1234 and np.count_nonzero(st) == 1
    q2, s2 = oracle.untile_int4(qt, st, R, K)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_tile_int4_padding_is_zero():
    R, K = 16, 96           # 3 groups -> one super-tile with one padding group
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    s = rng.integers(1, 30000, (R, K // 32), dtype=np.uint16)
    qt, st = oracle.tile_int4(q, s)
    words = qt.view(np.uint32).reshape(64, 4)
    assert np.all(words[:, 3] == 0)
    assert np.all(st.reshape(16, 4)[:, 3] == 0)


# ------------------------------------------------------------ variants: GELU gate, residual prologue
# The Together AI fusion post (blog.hotdry.top) fuses an MLP whose activation
# is GELU, and fuses the residual add / all-reduce into the next
# normalisation; the pages give neither formula, so the oracle's readings are
# pinned here against the standard normal table, odd-part identities and
# torch's own implementations.

PHI_1 = 0.8413447460685429  # standard normal distribution function at 1 (tables)


def test_gelu_closed_form_values():
    assert oracle.gelu_erf(0.0) == 0.0 and oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_erf(1.0) == pytest.approx(PHI_1, abs=1e-15)
    assert oracle.gelu_erf(-1.0) == pytest.approx(-(1.0 - PHI_1), abs=1e-15)
    # GELU(t) - GELU(-t) = t for both forms (Phi(t) + Phi(-t) = 1; tanh is odd)
    for t in (-6.0, -1.3, -0.2, 0.07, 0.9, 2.5, 7.0):
        for f in (oracle.gelu_erf, oracle.gelu_tanh):
            assert f(t) - f(-t) == pytest.approx(t, rel=1e-14, abs=1e-15)
    # the tanh form approximates the erf form to ~1e-3 absolute
    for t in np.linspace(-5, 5, 41):
        assert abs(oracle.gelu_tanh(float(t)) - oracle.gelu_erf(float(t))) < 1e-3
    # limits: -> t for large t, -> 0 for very negative t
    for f in (oracle.gelu_erf, oracle.gelu_tanh):
        assert f(40.0) == pytest.approx(40.0, rel=1e-15)
        assert abs(f(-40.0)) < 1e-300 or f(-40.0) == 0.0


@pytest.mark.parametrize("approximate,fn", [("none", "gelu_erf"), ("tanh", "gelu_tanh")])
def test_gelu_matches_torch(approximate, fn):
    t = torch.linspace(-12, 12, 1201, dtype=torch.float64)
    ref = F.gelu(t, approximate=approximate).numpy()
    got = np.array([getattr(oracle, fn)(float(v)) for v in t])
    # 1 + tanh(.) cancels for very negative t: compare there on an absolute scale
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_bf16_rne_ties_subnormals_and_overflow():
    r = oracle.bf16_rne
    assert r(1.0 + 2 ** -8) == 0x3F80           # tie between 1 and 1+2^-7: even
    assert r(1.0 + 3 * 2 ** -8) == 0x3F82       # tie between 1+2^-7 and 1+2^-6: even
    assert r(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81  # just above the tie
    assert r(-(2.0 + 2 ** -7)) == 0xC000        # tie at the next binade: even
    assert r(-0.0) == 0x8000 and r(0.0) == 0
    assert r(2 ** -133) == 0x0001 and r(2 ** -134) == 0 and r(3 * 2 ** -135) == 0x0001
    assert r(3.3895313892515355e38) == 0x7F7F   # largest finite bf16
    assert r(3.5e38) == 0x7F80 and r(-math.inf) == 0xFF80
    assert (r(math.nan) & 0x7FFF) > 0x7F80


def test_bf16_rne_matches_torch_on_float32_values():
    # every binary32 value is exact in double, and torch rounds binary32 to
    # bf16 to nearest even: the two must agree bit for bit
    g = torch.Generator().manual_seed(7)
    v = torch.cat([torch.randn(4000, generator=g) * 10.0 ** float(e) for e in range(-30, 31, 6)])
    want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, want)


def test_residual_add_matches_torch():
    # bf16 + bf16 in binary32 then rounded to bf16 is the correctly rounded
    # sum (24 >= 2*8 + 2 bits: the double rounding is innocuous)
    x = rand_bf16((8, 512), 1.0, 71)
    r = rand_bf16((8, 512), 3.0, 72)
    r[0, :8] = bf16_bits([1e-30, -1e-30, 2.0 ** -8, 2.0 ** 100, -1.0, 0.0, 1.0 + 2 ** -7, 7.0])
    want = (torch.from_numpy(bf16_values(x)).float() + torch.from_numpy(bf16_values(r)).float())
    want = want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.residual_add(x, r), want)


def test_forward_ex_defaults_are_eq1():
    x, g, wg, wu, wd = _rand_layer(3, 64, 96, 800)
    y, h = oracle.forward_unfused_ex(x, g, 1e-5, wg, wu, wd)
    assert h is None
    assert np.array_equal(y, oracle.forward_unfused(x, g, 1e-5, wg, wu, wd))


@pytest.mark.parametrize("act,approx", [(oracle.ACT_SILU, None), (oracle.ACT_GELU_TANH, "tanh"),
                                        (oracle.ACT_GELU_ERF, "none")])
@pytest.mark.parametrize("with_res", [False, True])
@pytest.mark.parametrize("M", [3, 37])
def test_forward_ex_matches_torch_composition(act, approx, with_res, M):
    d, ff = 128, 160
    x, g, wg, wu, wd = _rand_layer(M, d, ff, 810 + act)
    res = rand_bf16((M, d), 2.0, 820 + act) if with_res else None
    X = torch.from_numpy(bf16_values(x))
    if with_res:
        hb = (X.float() + torch.from_numpy(bf16_values(res)).float()).to(torch.bfloat16)
        X = hb.double()
    G, WG, WU, WD = (torch.from_numpy(bf16_values(a)) for a in (g, wg, wu, wd))
    n = F.rms_norm(X, (d,), G, 1e-5)
    z = n @ WG.T
    gate = F.silu(z) if approx is None else F.gelu(z, approximate=approx)
    ref = ((gate * (n @ WU.T)) @ WD.T).numpy()
    y, h = oracle.forward_unfused_ex(x, g, 1e-5, wg, wu, wd, act=act, residual=res)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())
    if with_res:
        assert np.array_equal(h, hb.view(torch.int16).numpy().view(np.uint16))


def test_int4_forward_ex_matches_torch_composition():
    # int4 variant: the same composition with w = s*q built here from the nibbles
    rng = np.random.default_rng(9)
    M, d, ff = 2, 128, 96
    x = rand_bf16((M, d), 1.0, 832)
    g = rand_bf16((d,), 0.1, 833, mean=1.0)
    res = rand_bf16((M, d), 1.0, 834)
    q_gu = rng.integers(0, 256, (2 * ff, d // 2), dtype=np.uint8)
    s_gu = (rng.random((2 * ff, d // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    q_d = rng.integers(0, 256, (d, ff // 2), dtype=np.uint8)
    s_d = (rng.random((d, ff // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    wgu = np.repeat(s_gu.view(np.float16).astype(np.float64), 32, 1) * _nibbles(q_gu)
    wdn = np.repeat(s_d.view(np.float16).astype(np.float64), 32, 1) * _nibbles(q_d)
    hb = (torch.from_numpy(bf16_values(x)).float() + torch.from_numpy(bf16_values(res)).float())
    hb = hb.to(torch.bfloat16)
    n = F.rms_norm(hb.double(), (d,), torch.from_numpy(bf16_values(g)), 1e-5)
    WGU = torch.from_numpy(wgu)
    ref = ((F.gelu(n @ WGU[0::2].T) * (n @ WGU[1::2].T)) @ torch.from_numpy(wdn).T).numpy()
    y, h = oracle.forward_int4_ex(x, g, 1e-5, q_gu, s_gu, q_d, s_d, act=oracle.ACT_GELU_ERF,
                                  residual=res)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())
    assert np.array_equal(h, hb.view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------ fp16 weight storage
# bf16 -> fp16 by truncation toward zero. Expected patterns worked out by hand
# from the two formats: bf16 = sign | 8-bit exponent (bias 127) | 7 bits;
# fp16 = sign | 5-bit exponent (bias 15) | 10 bits, subnormal unit 2^-24.
F16_TRUNC_HAND = [
    (0x3F80, 0x3C00),  # 1.0
    (0xC000, 0xC000),  # -2.0
    (0x477F, 0x7BF8),  # 65280 = 2^15 * (1 + 1016/1024), largest bf16 below 65504
    (0x3880, 0x0400),  # 2^-14, smallest fp16 normal
    (0x3800, 0x0200),  # 2^-15 = 512 * 2^-24, exact subnormal
    (0x3380, 0x0001),  # 2^-24, smallest fp16 subnormal
    (0x33C0, 0x0001),  # 1.5 * 2^-24 truncates to 2^-24 (nearest-even would give 2 units)
    (0x3300, 0x0000),  # 2^-25 truncates to +0
    (0xB300, 0x8000),  # -2^-25 truncates to -0
    (0x35E0, 0x001C),  # 1.75 * 2^-20 = 28 units of 2^-24
    (0x8000, 0x8000),  # -0
]
F16_TRUNC_RANGE = [0x4780, 0xC780, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F]  # 65536, -65536, +-inf, NaN, max bf16


def test_f16_trunc_hand_values():
    w = np.array([b for b, _ in F16_TRUNC_HAND], np.uint16)
    out, bad = oracle.bf16_to_f16_trunc(w)
    assert bad == 0
    assert [int(v) for v in out] == [h for _, h in F16_TRUNC_HAND]
    for b in F16_TRUNC_RANGE:
        _, bad = oracle.bf16_to_f16_trunc(np.array([0x3F80, b], np.uint16))
        assert bad == 1, hex(b)


def test_f16_trunc_every_pattern():
    # every bf16 pattern: exact in the fp16 normal range, the largest fp16
    # magnitude not above |v| below it (sign kept), range errors exactly for
    # non-finite values and magnitudes above 65504; fp16 decoded by numpy
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_values(bits)
    out, bad = oracle.bf16_to_f16_trunc(bits)
    err = ~np.isfinite(v) | (np.abs(v) > 65504.0)
    assert bad == int(err.sum())
    assert not out[err].any()
    ok = ~err
    h = out[ok].view(np.float16)
    hv, a = h.astype(np.float64), np.abs(v[ok])
    assert np.array_equal(out[ok] >> 15, bits[ok] >> 15)
    normal = a >= 2.0 ** -14
    assert np.array_equal(np.abs(hv[normal]), a[normal])
    up = np.nextafter(np.abs(h), np.float16(np.inf)).astype(np.float64)
    assert np.all(np.abs(hv) <= a) and np.all(a < up)


def _f16_layer(M, d, ff, seed):
    x, g, wg, wu, wd = _rand_layer(M, d, ff, seed)
    wgu = oracle.pack_interleaved(wg, wu)
    # a few weights in the fp16 subnormal range, where the conversion rounds
    tiny = bf16_bits(np.array([3.1e-7, -4.7e-6, 2.9e-5, -6.0e-5], np.float32))
    wgu.reshape(-1)[[3, 70, 1000, 5001]] = tiny
    wd.reshape(-1)[[5, 77, 900]] = tiny[:3]
    return x, g, wgu, wd


@pytest.mark.parametrize("act,approx,with_res", [(oracle.ACT_SILU, None, False),
                                                 (oracle.ACT_GELU_TANH, "tanh", True)])
def test_f16_forward_matches_torch_composition(act, approx, with_res):
    M, d, ff = 3, 128, 160
    x, g, wgu, wd = _f16_layer(M, d, ff, 850)
    hgu, bad1 = oracle.bf16_to_f16_trunc(wgu)
    hd, bad2 = oracle.bf16_to_f16_trunc(wd)
    assert bad1 == 0 and bad2 == 0
    res = rand_bf16((M, d), 2.0, 851) if with_res else None
    X = torch.from_numpy(bf16_values(x))
    if with_res:
        hb = (X.float() + torch.from_numpy(bf16_values(res)).float()).to(torch.bfloat16)
        X = hb.double()
    WGU = torch.from_numpy(hgu.view(np.float16).astype(np.float64))
    WD = torch.from_numpy(hd.view(np.float16).astype(np.float64))
    n = F.rms_norm(X, (d,), torch.from_numpy(bf16_values(g)), 1e-5)
    z = n @ WGU[0::2].T
    gate = F.silu(z) if approx is None else F.gelu(z, approximate=approx)
    ref = ((gate * (n @ WGU[1::2].T)) @ WD.T).numpy()
    y, h = oracle.forward_f16_ex(x, g, 1e-5, hgu, hd, act=act, residual=res)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13 * np.abs(ref).max())
    if with_res:
        assert np.array_equal(h, hb.view(torch.int16).numpy().view(np.uint16))


def test_f16_forward_equals_bf16_forward_when_exact():
    # weights inside the fp16 normal range convert exactly, so the fp16 forward
    # reads the same values as the bf16 one and gives the same doubles
    x, g, wg, wu, wd = _rand_layer(2, 64, 96, 860)
    wgu = oracle.pack_interleaved(wg, wu)
    tiny = lambda w: np.abs(bf16_values(w)) < 2.0 ** -14
    wgu[tiny(wgu)] = wgu[tiny(wgu)] & 0x8000  # signed zeros
    wd[tiny(wd)] = wd[tiny(wd)] & 0x8000
    hgu, _ = oracle.bf16_to_f16_trunc(wgu)
    hd, _ = oracle.bf16_to_f16_trunc(wd)
    y16, _ = oracle.forward_f16_ex(x, g, 1e-5, hgu, hd)
    assert np.array_equal(y16, oracle.forward_bf16(x, g, 1e-5, wgu, wd))


# ------------------------------------------------------------ brute force in decimal
# The whole forward re-evaluated in Python's decimal arithmetic at 40
# significant digits: every bf16 / fp16 input converts to Decimal exactly,
# sqrt and exp are decimal's own, and nothing is shared with the C++ oracle
# or with IEEE double arithmetic. The fp64 oracle must agree to within its
# own rounding: 1e-12 of the sum of |terms| of each output.

def _dec_forward(x, g, eps, wg, wu, wd, act_is_int4_scaled=False):
    from decimal import Decimal, localcontext
    with localcontext() as c:
        c.prec = 40
        M, d = x.shape
        ff = wg.shape[0]
        D = lambda v: Decimal(float(v))
        eps_d = D(eps)
        y = np.zeros((M, d))
        mag = np.zeros((M, d))
        for m in range(M):
            xm = [D(v) for v in x[m]]
            ss = sum(v * v for v in xm)
            r = 1 / (ss / d + eps_d).sqrt()
            n = [xm[k] * r * D(g[k]) for k in range(d)]
            a = []
            for i in range(ff):
                gi = sum(D(wg[i, k]) * n[k] for k in range(d))
                ui = sum(D(wu[i, k]) * n[k] for k in range(d))
                a.append(gi / (1 + (-gi).exp()) * ui)
            for j in range(d):
                terms = [D(wd[j, i]) * a[i] for i in range(ff)]
                y[m, j] = float(sum(terms))
                mag[m, j] = float(sum(abs(t) for t in terms))
        return y, mag


@pytest.mark.parametrize("M,d,ff,seed", [(1, 2, 1, 11), (4, 64, 64, 12), (3, 32, 48, 13),
                                         (2, 64, 16, 14)])
def test_brute_force_decimal_bf16(M, d, ff, seed):
    x = rand_bf16((M, d), 1.0, seed)
    g = rand_bf16((d,), 0.1, seed + 1, mean=1.0)
    wg = rand_bf16((ff, d), 0.3, seed + 2)
    wu = rand_bf16((ff, d), 0.3, seed + 3)
    wd = rand_bf16((d, ff), 0.3, seed + 4)
    vals = [bf16_values(a) for a in (x, g, wg, wu, wd)]
    for eps in (1e-5, 0.0):
        ref, mag = _dec_forward(*vals[:2], eps, *vals[2:])
        got = oracle.forward_unfused(x, g, eps, wg, wu, wd)
        assert np.all(np.abs(got - ref) <= 1e-12 * mag + 1e-300), (eps, np.abs(got - ref).max())
        got2 = oracle.forward_bf16(x, g, eps, oracle.pack_interleaved(wg, wu), wd)
        assert np.array_equal(got, got2)


def test_brute_force_decimal_large_and_tiny_magnitudes():
    # rows of very different scales and a weight set with a large range of
    # gate pre-activations (SiLU far into both tails)
    x = np.concatenate([rand_bf16((1, 32), 1e4, 21), rand_bf16((1, 32), 1e-4, 22),
                        rand_bf16((1, 32), 1.0, 23)])
    g = rand_bf16((32,), 0.5, 24, mean=1.0)
    wg = rand_bf16((24, 32), 3.0, 25)
    wu = rand_bf16((24, 32), 0.02, 26)
    wd = rand_bf16((32, 24), 0.02, 27)
    vals = [bf16_values(a) for a in (x, g, wg, wu, wd)]
    ref, mag = _dec_forward(*vals[:2], 1e-5, *vals[2:])
    got = oracle.forward_unfused(x, g, 1e-5, wg, wu, wd)
    assert np.all(np.abs(got - ref) <= 1e-12 * mag + 1e-300)


def test_brute_force_decimal_int4():
    # int4 weights: w = s * q exactly, in decimal as in the oracle
    rng = np.random.default_rng(31)
    M, d, ff = 2, 64, 32
    x = rand_bf16((M, d), 1.0, 32)
    g = rand_bf16((d,), 0.1, 33, mean=1.0)
    q_gu = rng.integers(0, 256, (2 * ff, d // 2), dtype=np.uint8)
    q_d = rng.integers(0, 256, (d, ff // 2), dtype=np.uint8)
    s_gu = (rng.random((2 * ff, d // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)
    s_d = (rng.random((d, ff // 32)) * 0.015 + 0.005).astype(np.float16).view(np.uint16)

    def dense(q, s):
        lo = (q & 0xF).astype(np.int64)
        hi = (q >> 4).astype(np.int64)
        codes = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
        codes[:, 0::2], codes[:, 1::2] = lo, hi
        codes = np.where(codes >= 8, codes - 16, codes)
        sc = np.repeat(s.view(np.float16).astype(np.float64), 32, axis=1)
        return sc * codes  # exact: an 11-bit scale times a 4-bit integer

    wgu = dense(q_gu, s_gu)
    ref, mag = _dec_forward(bf16_values(x), bf16_values(g), 1e-5, wgu[0::2], wgu[1::2],
                            dense(q_d, s_d))
    got = oracle.forward_int4(x, g, 1e-5, q_gu, s_gu, q_d, s_d)
    assert np.all(np.abs(got - ref) <= 1e-12 * mag + 1e-300)
