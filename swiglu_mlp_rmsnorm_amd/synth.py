"""Seeded synthetic inputs for the fused gated MLP.

This module holds no arithmetic of the method: it only draws random numbers
with the shapes and distributions of the workloads below and rounds them to
the storage types (bf16 / fp16 / raw int4 bytes). Both the HIP path and the
CPU oracle consume what it returns (the oracle through host copies), so the
two sides see bit-identical inputs.

Workloads (synthetic stand-ins for the models the pages measure: Phi-3-mini,
Llama-3.1-8B and Llama-70B shaped layers, and one GPU's tensor-parallel share
of the last two; no checkpoint or dataset is used):
  x ~ N(0,1), gamma = 1 + N(0,0.1), W_gate / W_up / W_down ~ N(0,0.02), all
  rounded to bf16 (RNE); eps = 1e-5. int4 layers, in the row-major exchange
  format (codes [rows, K/2], scales [rows, K/32]): every packed byte uniform
  in [0,255], i.e. both nibbles uniform over the 16 two's-complement values
  [-8,7]; scales ~ U(0.005,0.02) rounded to fp16. Gate, up and down are
  drawn separately, as bf16 layers are.
"""
from __future__ import annotations

import dataclasses

import torch

EPS = 1e-5

# tensor ids inside one layer's seed space
T_X, T_GAMMA, T_WGATE, T_WUP, T_WDOWN, T_QGATE, T_SGATE, T_QD, T_SD, T_QUP, T_SUP = range(11)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed namespace
    d: int
    ff: int
    Ms: tuple
    sets: int           # distinct layer weight sets rotated per step
    wtype: str          # "bf16" or "int4"
    prefill_Ms: tuple = ()  # token counts also measured on the prefill path


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_d256_ff704", 0, 256, 704, (1,), 1, "bf16"),
        Workload("phi3mini_decode_d3072_ff8192", 1, 3072, 8192, (1, 8), 32, "bf16"),
        Workload("llama8b_decode_d4096_ff14336", 2, 4096, 14336, (1, 4, 16, 32), 32, "bf16"),
        Workload("llama8b_prefill_d4096_ff14336", 3, 4096, 14336, (512, 2048), 1, "bf16"),
        # (and its int4 weights through the prefill GEMMs, at the Llama-8B
        # prefill token counts)
        Workload("llama70b_int4_decode_d8192_ff28672", 4, 8192, 28672, (1, 16), 20, "int4",
                 (512, 2048)),
        # one GPU's share of the two decode layers under 8-way tensor
        # parallelism over ff (each GPU holds ff/8 gate/up pairs and the
        # matching W_down columns; the partial y of the eight would then be
        # summed across GPUs): 44 MB and 50 MB of weights per set, 16 sets
        Workload("llama8b_tp8_shard_decode_d4096_ff1792", 5, 4096, 1792, (1, 16), 16, "bf16"),
        Workload("llama70b_int4_tp8_shard_decode_d8192_ff3584", 6, 8192, 3584, (1, 16), 16,
                 "int4"),
    )
}


def seed_of(workload_index: int, layer: int, tensor_id: int) -> int:
    return 1_000_003 * workload_index + 1_009 * layer + tensor_id


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, mean: float, std: float, seed: int, device="cpu") -> torch.Tensor:
    """N(mean, std^2) drawn in fp32, rounded to bf16 (round-to-nearest-even)."""
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return (t * std + mean).to(torch.bfloat16)


def uniform_bytes(shape, seed: int, device="cpu") -> torch.Tensor:
    """Uniform bytes in [0, 255] (two uniform 4-bit fields per byte)."""
    return torch.randint(0, 256, shape, generator=_gen(seed, device), device=device,
                         dtype=torch.int32).to(torch.uint8)


def uniform_f16(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    """U(lo, hi) drawn in fp32, rounded to fp16."""
    t = torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return (lo + (hi - lo) * t).to(torch.float16)


def activations(M: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    return normal_bf16((M, d), 0.0, 1.0, seed, device)


def gamma(d: int, seed: int, device="cpu") -> torch.Tensor:
    return normal_bf16((d,), 1.0, 0.1, seed, device)


def bf16_weight(rows: int, cols: int, seed: int, device="cpu", std: float = 0.02) -> torch.Tensor:
    return normal_bf16((rows, cols), 0.0, std, seed, device)


def int4_weight(rows: int, K: int, seed_q: int, seed_s: int, device="cpu"):
    """Row-major int4 in the exchange format: codes uint8 [rows, K/2] (uniform
    bytes, so every code is uniform over [-8, 7]) and fp16 scales
    [rows, K/32] ~ U(0.005, 0.02)."""
    return (uniform_bytes((rows, K // 2), seed_q, device),
            uniform_f16((rows, K // 32), 0.005, 0.02, seed_s, device))


def layer_bf16(w: Workload, layer: int, device="cpu"):
    """(w_gate [ff,d], w_up [ff,d], w_down [d,ff]) for one layer, bf16."""
    s = lambda t: seed_of(w.index, layer, t)
    return (bf16_weight(w.ff, w.d, s(T_WGATE), device),
            bf16_weight(w.ff, w.d, s(T_WUP), device),
            bf16_weight(w.d, w.ff, s(T_WDOWN), device))


def layer_int4(w: Workload, layer: int, device="cpu"):
    """Row-major int4 (codes, scales) of W_gate [ff, d], W_up [ff, d] and
    W_down [d, ff]: (q_gate, s_gate, q_up, s_up, q_down, s_down)."""
    s = lambda t: seed_of(w.index, layer, t)
    q_g, s_g = int4_weight(w.ff, w.d, s(T_QGATE), s(T_SGATE), device)
    q_u, s_u = int4_weight(w.ff, w.d, s(T_QUP), s(T_SUP), device)
    q_d, s_d = int4_weight(w.d, w.ff, s(T_QD), s(T_SD), device)
    return q_g, s_g, q_u, s_u, q_d, s_d


def inputs(w: Workload, M: int, device="cpu", layer: int = 0):
    """(x [M,d] bf16, gamma [d] bf16) for one step."""
    return (activations(M, w.d, seed_of(w.index, layer, T_X), device),
            gamma(w.d, seed_of(w.index, layer, T_GAMMA), device))


def bits(t: torch.Tensor):
    """Host numpy view of a tensor's raw bits (uint16 for 2-byte types)."""
    import numpy as np
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)
