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

# Guard regions: every output and scratch buffer the helpers below hand to
# the library sits inside a larger allocation whose GUARD bytes before and
# after it hold a sentinel; a write outside the buffer changes them.
GUARD = 256
SENTINEL = 0x5A


class Guarded:
    """A device buffer of `nbytes` with sentinel guards on both sides; its
    interior starts as 0xFF bytes (NaN for bf16 and fp32)."""

    def __init__(self, nbytes, device="cuda"):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=device)
        self.buf[GUARD:GUARD + self.n] = 0xFF

    def bytes(self):
        return self.buf[GUARD:GUARD + self.n]

    def bf16(self, *shape):
        return self.bytes().view(torch.bfloat16).view(*shape)

    def check(self, what):
        lo, hi = self.buf[:GUARD], self.buf[GUARD + self.n:]
        assert torch.all(lo == SENTINEL) and torch.all(hi == SENTINEL), \
            f"{what}: a write landed outside the buffer"


def guarded_call(fn, M, d, ff, wtype, with_h=False, **kw):
    """Run fn(..., y=, workspace=[, h_out=]) on guarded buffers (unless the
    caller passed its own), then check every guard."""
    guards = []
    if kw.get("y") is None:
        g = Guarded(M * d * 2)
        kw["y"] = g.bf16(M, d)
        guards.append(("y", g))
    if kw.get("workspace") is None:
        g = Guarded(max(F.fmlp_workspace_size(M, d, ff, wtype), 1))
        kw["workspace"] = g.bytes()
        guards.append(("workspace", g))
    if with_h and kw.get("h_out") is None:
        g = Guarded(M * d * 2)
        kw["h_out"] = g.bf16(M, d)
        guards.append(("h_out", g))
    out = fn(**kw)
    if guards:  # (none when the caller brought every buffer, e.g. under graph capture)
        torch.cuda.synchronize()
        for what, g in guards:
            g.check(what)
    return out


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

    wtype = F.FMLP_W_BF16

    def forward(self, x, g, eps, **kw):
        return guarded_call(lambda **k: F.fmlp_forward_path(x, g, eps, self.wgu_t, self.wd_t, **k),
                            x.shape[0], self.d, self.ff, self.wtype, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        wg, wu, wd = self.host
        return oracle.forward_unfused_ex(synth.bits(x), synth.bits(g), eps, wg, wu, wd, act=act,
                                         residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return guarded_call(lambda **k: F.fmlp_forward_ex(x, g, eps, self.wgu_t, self.wd_t, **k),
                            x.shape[0], self.d, self.ff, self.wtype,
                            with_h=kw.get("residual") is not None, **kw)


class Int4Layer:
    """Synthetic int4 weights in the row-major exchange format (gate, up and
    down drawn separately), packed to the tiled layout by the library; the
    oracle interleaves the same seeded rows itself."""

    def __init__(self, d, ff, seed, device="cuda"):
        self.d, self.ff = d, ff
        self.q_g, self.s_g = synth.int4_weight(ff, d, seed, seed + 1, device)
        self.q_u, self.s_u = synth.int4_weight(ff, d, seed + 4, seed + 5, device)
        self.q_dn, self.s_dn = synth.int4_weight(d, ff, seed + 2, seed + 3, device)
        self.q_gu, self.s_gu = F.fmlp_pack_int4_interleaved(self.q_g, self.s_g, self.q_u, self.s_u)
        self.q_d, self.s_d = F.fmlp_pack_int4_matrix(self.q_dn, self.s_dn)
        b = synth.bits
        q_gu, s_gu = oracle.pack_interleaved_int4(b(self.q_g), b(self.s_g), b(self.q_u),
                                                  b(self.s_u))
        self.host = (q_gu, s_gu, b(self.q_dn), b(self.s_dn))

    def oracle(self, x, g, eps):
        return oracle.forward_int4(synth.bits(x), synth.bits(g), eps, *self.host)

    wtype = F.FMLP_W_INT4_G32

    def forward(self, x, g, eps, **kw):
        return guarded_call(lambda **k: F.fmlp_forward_path(
            x, g, eps, self.q_gu, self.q_d, self.s_gu, self.s_d, ff=self.ff, **k),
            x.shape[0], self.d, self.ff, self.wtype, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        return oracle.forward_int4_ex(synth.bits(x), synth.bits(g), eps, *self.host, act=act,
                                      residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return guarded_call(lambda **k: F.fmlp_forward_ex(
            x, g, eps, self.q_gu, self.q_d, self.s_gu, self.s_d, ff=self.ff, **k),
            x.shape[0], self.d, self.ff, self.wtype, with_h=kw.get("residual") is not None,
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
        return guarded_call(lambda **k: F.fmlp_forward_path(x, g, eps, self.hgu_t, self.hd_t, **k),
                            x.shape[0], self.d, self.ff, F.FMLP_W_F16, **kw)

    def oracle_ex(self, x, g, eps, act, res):
        return oracle.forward_f16_ex(synth.bits(x), synth.bits(g), eps, *self.host16, act=act,
                                     residual=None if res is None else synth.bits(res))

    def forward_ex(self, x, g, eps, **kw):
        return guarded_call(lambda **k: F.fmlp_forward_ex(x, g, eps, self.hgu_t, self.hd_t, **k),
                            x.shape[0], self.d, self.ff, F.FMLP_W_F16,
                            with_h=kw.get("residual") is not None, **kw)

    def forward_bf16(self, x, g, eps, **kw):
        return Bf16Layer.forward(self, x, g, eps, **kw)
