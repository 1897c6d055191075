"""Shared helpers for the GPU parity tests: run the HIP path and the CPU
oracle on the same seeded inputs and compare with the accuracy bar

    max |y - y_ref| <= 2e-2 * rms(y_ref)   and   sum|y - y_ref| / sum|y_ref| <= 3e-3

(y_ref is the oracle's fp64 result, y the library's bf16 output)."""
import numpy as np
import torch

from oracle import oracle
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


def bf16_layer(d, ff, seed, device="cuda"):
    """(w_gate, w_up, w_down) bf16 on the device, N(0, 0.02)."""
    return (synth.bf16_weight(ff, d, seed + 2, device), synth.bf16_weight(ff, d, seed + 3, device),
            synth.bf16_weight(d, ff, seed + 4, device))


def bf16_inputs(M, d, seed, device="cuda"):
    return synth.activations(M, d, seed, device), synth.gamma(d, seed + 1, device)


def oracle_bf16(x, g, eps, w_gu, w_down):
    b = synth.bits
    return oracle.forward_bf16(b(x), b(g), eps, b(w_gu), b(w_down))


def oracle_int4(x, g, eps, q_gu, s_gu, q_d, s_d):
    b = synth.bits
    return oracle.forward_int4(b(x), b(g), eps, b(q_gu), b(s_gu), b(q_d), b(s_d))
