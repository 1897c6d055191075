"""Shared helpers for the GPU parity tests: run the HIP path and the CPU
oracle on the same seeded inputs and compare with the accuracy bar

    max |y - y_ref| <= 2e-2 * rms(y_ref)   and   sum|y - y_ref| / sum|y_ref| <= 3e-3

(y_ref is the oracle's fp64 result, y the library's bf16 output). The oracle
always receives the seeded inputs themselves (host copies), never a buffer
the HIP library produced."""
import numpy as np
import torch

from oracle import oracle
from swiglu_mlp_rmsnorm_amd import fmlp as F
from swiglu_mlp_rmsnorm_amd import synth

MAX_REL_TOL = 2e-2
L1_REL_TOL = 3e-3


def errors(y_gpu: torch.Tensor, y_ref: np.ndarray):
    y = y_gpu.detach().float().cpu().double().numpy()
    assert y.shape == y_ref.shape
    err = np.abs(y - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    return float(err.max() / rms), float(err.sum() / np.abs(y_ref).sum())


def assert_parity(y_gpu, y_ref, what=""):
    y = y_gpu.detach().float().cpu().numpy()
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    mx, l1 = errors(y_gpu, y_ref)
    assert mx <= MAX_REL_TOL and l1 <= L1_REL_TOL, f"{what}: max/rms {mx:.3e}, L1 rel {l1:.3e}"
    return mx, l1


class Bf16Layer:
    """Row-major synthetic weights (oracle side) and their packed, tiled
    device copies (HIP side)."""

    def __init__(self, d, ff, seed, device="cuda"):
        self.d, self.ff = d, ff
        self.wg = synth.bf16_weight(ff, d, seed + 2, device)
        self.wu = synth.bf16_weight(ff, d, seed + 3, device)
        self.wd = synth.bf16_weight(d, ff, seed + 4, device)
        self.wgu_t = F.fmlp_pack_interleaved(self.wg, self.wu)
        self.wd_t = F.fmlp_pack_matrix(self.wd)
        self.host = tuple(synth.bits(t) for t in (self.wg, self.wu, self.wd))

    def oracle(self, x, g, eps):
        wg, wu, wd = self.host
        return oracle.forward_unfused(synth.bits(x), synth.bits(g), eps, wg, wu, wd)

    def forward(self, x, g, eps, **kw):
        return F.fmlp_forward_path(x, g, eps, self.wgu_t, self.wd_t, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        wg, wu, wd = self.host
        return oracle.forward_unfused_ex(synth.bits(x), synth.bits(g), eps, wg, wu, wd, act=act,
                                         residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return F.fmlp_forward_ex(x, g, eps, self.wgu_t, self.wd_t, **kw)


class Int4Layer:
    """Synthetic tiled int4 weights; the oracle untiles the same seeded bytes."""

    def __init__(self, d, ff, seed, device="cuda"):
        self.d, self.ff = d, ff
        self.q_gu, self.s_gu = synth.int4_weight(2 * ff, d, seed, seed + 1, device)
        self.q_d, self.s_d = synth.int4_weight(d, ff, seed + 2, seed + 3, device)
        b = synth.bits
        q_gu, s_gu = oracle.untile_int4(b(self.q_gu), b(self.s_gu), 2 * ff, d)
        q_d, s_d = oracle.untile_int4(b(self.q_d), b(self.s_d), d, ff)
        self.host = (q_gu, s_gu, q_d, s_d)

    def oracle(self, x, g, eps):
        return oracle.forward_int4(synth.bits(x), synth.bits(g), eps, *self.host)

    def forward(self, x, g, eps, **kw):
        return F.fmlp_forward_path(x, g, eps, self.q_gu, self.q_d, self.s_gu, self.s_d,
                                   ff=self.ff, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        return oracle.forward_int4_ex(synth.bits(x), synth.bits(g), eps, *self.host, act=act,
                                      residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return F.fmlp_forward_ex(x, g, eps, self.q_gu, self.q_d, self.s_gu, self.s_d, ff=self.ff,
                                 **kw)


def bf16_inputs(M, d, seed, device="cuda"):
    return synth.activations(M, d, seed, device), synth.gamma(d, seed + 1, device)


class F16Layer(Bf16Layer):
    """The seeded bf16 weights converted to fp16 (FMLP_W_F16): the library
    converts its packed tiles, the oracle converts the same host bits itself."""

    def __init__(self, d, ff, seed, device="cuda"):
        super().__init__(d, ff, seed, device)
        self.hgu_t = F.fmlp_convert_f16(self.wgu_t)
        self.hd_t = F.fmlp_convert_f16(self.wd_t)
        wg, wu, wd = self.host
        hgu, bad1 = oracle.bf16_to_f16_trunc(oracle.pack_interleaved(wg, wu))
        hd, bad2 = oracle.bf16_to_f16_trunc(wd)
        assert bad1 == 0 and bad2 == 0
        self.host16 = (hgu, hd)

    def oracle(self, x, g, eps):
        return oracle.forward_f16_ex(synth.bits(x), synth.bits(g), eps, *self.host16)[0]

    def forward(self, x, g, eps, **kw):
        return F.fmlp_forward_path(x, g, eps, self.hgu_t, self.hd_t, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        return oracle.forward_f16_ex(synth.bits(x), synth.bits(g), eps, *self.host16, act=act,
                                     residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return F.fmlp_forward_ex(x, g, eps, self.hgu_t, self.hd_t, **kw)

    def forward_bf16(self, x, g, eps, **kw):
        return F.fmlp_forward_path(x, g, eps, self.wgu_t, self.wd_t, **kw)
