"""Fused gated (SwiGLU) MLP with an RMSNorm prologue for MI355X (gfx950).

The computation lives in libfmlp.so (hand-written HIP kernels behind the C
ABI of include/fmlp.h); this package is the thin binding over it plus the
seeded synthetic-input generator used by tests and benchmarks.
"""
from .fmlp import (  # noqa: F401
    FMLP_PATH_AUTO, FMLP_PATH_DECODE, FMLP_PATH_PREFILL, FMLP_W_BF16, FMLP_W_INT4_G32,
    FmlpError, fmlp_dequant_int4, fmlp_forward, fmlp_forward_path, fmlp_pack_int4_interleaved,
    fmlp_pack_int4_matrix, fmlp_pack_interleaved, fmlp_quantize_int4, fmlp_status_string,
    fmlp_workspace_size, lib,
)
