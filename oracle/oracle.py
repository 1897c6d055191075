"""ctypes wrapper around the fp64 CPU oracle (oracle/fmlp_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package. It shares no code
with the HIP library. Inputs are numpy arrays holding raw bit patterns
(uint16 for bf16/fp16, uint8 for packed int4); outputs are float64 (forward)
or exact float32 (dequant) or bit patterns (pack, quantise).

What each function computes, and the pages it follows, is stated in the C++
source; each wrapper below repeats the one-line definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FMLP_ORACLE_SRC / FMLP_ORACLE_LIB let the mutation test build a deliberately
# broken copy of the oracle elsewhere and check that the pins reject it.
_SRC = os.environ.get("FMLP_ORACLE_SRC", os.path.join(_HERE, "fmlp_oracle.cpp"))
_LIB = os.environ.get("FMLP_ORACLE_LIB", os.path.join(_HERE, "liboracle.so"))
_lock = threading.Lock()
_lib = None

RANGE_ERROR = -5


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (host only, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "g++", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", tmp, _SRC,
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I64, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        sig = {
            "oracle_bf16_to_double": (D, [ctypes.c_uint16]),
            "oracle_f16_to_double": (D, [ctypes.c_uint16]),
            "oracle_f32_to_f16_rne": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_silu": (D, [D]),
            "oracle_gelu_erf": (D, [D]),
            "oracle_gelu_tanh": (D, [D]),
            "oracle_bf16_rne": (ctypes.c_uint16, [D]),
            "oracle_residual_add": (None, [P, P, I64, P]),
            "oracle_forward_unfused_ex": (None, [P, P, P, P, D, ctypes.c_int, P, P, P, I64, I64,
                                                 I64, P]),
            "oracle_forward_int4_ex": (None, [P, P, P, P, D, ctypes.c_int, P, P, P, P, I64, I64,
                                              I64, P]),
            "oracle_rms_scale": (None, [P, I64, I64, D, P]),
            "oracle_rmsnorm": (None, [P, P, D, I64, I64, P]),
            "oracle_pack_interleaved": (None, [P, P, P, I64, I64]),
            "oracle_quantize_int4": (ctypes.c_int, [P, I64, I64, P, P]),
            "oracle_dequant_int4": (None, [P, P, I64, I64, P]),
            "oracle_forward_unfused": (None, [P, P, D, P, P, P, I64, I64, I64, P]),
            "oracle_forward_bf16": (None, [P, P, D, P, P, I64, I64, I64, P]),
            "oracle_forward_int4": (None, [P, P, D, P, P, P, P, I64, I64, I64, P]),
            "oracle_omp_threads": (ctypes.c_int, []),
            "oracle_set_threads": (None, [ctypes.c_int]),
            "oracle_bf16_to_f16_trunc": (I64, [P, I64, P]),
            "oracle_forward_f16_ex": (None, [P, P, P, P, D, ctypes.c_int, P, P, I64, I64, I64,
                                             P]),
            "oracle_tile_bf16": (None, [P, I64, I64, P]),
            "oracle_untile_bf16": (None, [P, I64, I64, P]),
            "oracle_int4_tiled_code_bytes": (I64, [I64, I64]),
            "oracle_int4_tiled_scale_count": (I64, [I64, I64]),
            "oracle_tile_int4": (None, [P, P, I64, I64, P, P]),
            "oracle_untile_int4": (None, [P, P, I64, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return _load().oracle_omp_threads()


def set_threads(n: int) -> None:
    """Threads of the OpenMP loops from now on (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def bf16_to_double(b: int) -> float:
    return _load().oracle_bf16_to_double(b)


def f16_to_double(h: int) -> float:
    return _load().oracle_f16_to_double(h)


def f32_to_f16_rne(f: float) -> int:
    return _load().oracle_f32_to_f16_rne(f)


def silu(t: float) -> float:
    """SiLU(t) = t / (1 + exp(-t))."""
    return _load().oracle_silu(t)


ACT_SILU, ACT_GELU_TANH, ACT_GELU_ERF = 0, 1, 2


def gelu_erf(t: float) -> float:
    """GELU(t) = t * Phi(t) = 0.5 t (1 + erf(t / sqrt 2))."""
    return _load().oracle_gelu_erf(t)


def gelu_tanh(t: float) -> float:
    """GELU(t) ~ 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3)))."""
    return _load().oracle_gelu_tanh(t)


def bf16_rne(v: float) -> int:
    """double -> bf16 bit pattern, round to nearest even."""
    return _load().oracle_bf16_rne(v)


def residual_add(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """h = bf16_rne(x + r), element-wise on bf16 bit patterns."""
    x, r = _c(x, np.uint16), _c(r, np.uint16)
    assert x.shape == r.shape
    h = np.empty(x.shape, np.uint16)
    _load().oracle_residual_add(_p(x), _p(r), x.size, _p(h))
    return h


def rms_scale(x: np.ndarray, eps: float) -> np.ndarray:
    """r[m] = 1/sqrt(mean_k x[m,k]^2 + eps); x bf16 bits [M, d]."""
    x = _c(x, np.uint16)
    M, d = x.shape
    r = np.empty(M, np.float64)
    _load().oracle_rms_scale(_p(x), M, d, eps, _p(r))
    return r


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """n[m,k] = x[m,k] * r[m] * gamma[k]."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    M, d = x.shape
    n = np.empty((M, d), np.float64)
    _load().oracle_rmsnorm(_p(x), _p(gamma), eps, M, d, _p(n))
    return n


def pack_interleaved(w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """w_gu[2i] = w_gate[i], w_gu[2i+1] = w_up[i] (bit copies)."""
    w_gate, w_up = _c(w_gate, np.uint16), _c(w_up, np.uint16)
    ff, d = w_gate.shape
    out = np.empty((2 * ff, d), np.uint16)
    _load().oracle_pack_interleaved(_p(w_gate), _p(w_up), _p(out), ff, d)
    return out


def pack_interleaved_int4(q_gate, s_gate, q_up, s_up):
    """Row interleave of int4 matrices in the exchange format (codes uint8
    [ff, d/2], scales fp16 bits [ff, d/32]): gate row i -> row 2i, up row i
    -> row 2i+1. The packer above moves each row's raw bytes (codes viewed
    as 16-bit pairs; d/2 is even)."""
    qg, qu = _c(q_gate, np.uint8), _c(q_up, np.uint8)
    q = pack_interleaved(qg.view(np.uint16), qu.view(np.uint16)).view(np.uint8)
    return q, pack_interleaved(_c(s_gate, np.uint16), _c(s_up, np.uint16))


def quantize_int4(w: np.ndarray):
    """Symmetric group-32 int4 with fp16 scales; returns (status, q, s)."""
    w = _c(w, np.uint16)
    rows, K = w.shape
    q = np.zeros((rows, K // 2), np.uint8)
    s = np.zeros((rows, K // 32), np.uint16)
    st = _load().oracle_quantize_int4(_p(w), rows, K, _p(q), _p(s))
    return st, q, s


def dequant_int4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """out[r,k] = float32(s[r,k//32]) * q[r,k] (exact)."""
    q, s = _c(q, np.uint8), _c(s, np.uint16)
    rows, half = q.shape
    K = half * 2
    out = np.empty((rows, K), np.float32)
    _load().oracle_dequant_int4(_p(q), _p(s), rows, K, _p(out))
    return out


def forward_unfused(x, gamma, eps, w_gate, w_up, w_down) -> np.ndarray:
    """Eq(1) with RMSNorm prologue, from separate gate/up matrices; fp64."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    w_gate, w_up, w_down = (_c(a, np.uint16) for a in (w_gate, w_up, w_down))
    M, d = x.shape
    ff = w_gate.shape[0]
    y = np.empty((M, d), np.float64)
    _load().oracle_forward_unfused(_p(x), _p(gamma), eps, _p(w_gate), _p(w_up),
                                   _p(w_down), M, d, ff, _p(y))
    return y


def forward_unfused_ex(x, gamma, eps, w_gate, w_up, w_down, act=ACT_SILU, residual=None):
    """Eq(1) with gate activation `act` and, when `residual` is given, the
    residual prologue h = bf16_rne(x + residual) normalised in place of x.
    Returns (y fp64 [M, d], h bf16 bits [M, d] or None)."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    w_gate, w_up, w_down = (_c(a, np.uint16) for a in (w_gate, w_up, w_down))
    M, d = x.shape
    ff = w_gate.shape[0]
    y = np.empty((M, d), np.float64)
    res = None if residual is None else _c(residual, np.uint16)
    h = None if residual is None else np.empty((M, d), np.uint16)
    _load().oracle_forward_unfused_ex(_p(x), None if res is None else _p(res),
                                      None if h is None else _p(h), _p(gamma), eps, act,
                                      _p(w_gate), _p(w_up), _p(w_down), M, d, ff, _p(y))
    return y, h


def forward_bf16(x, gamma, eps, w_gu, w_down) -> np.ndarray:
    """Eq(1) with RMSNorm prologue, from the interleaved w_gu [2ff, d]; fp64."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    w_gu, w_down = _c(w_gu, np.uint16), _c(w_down, np.uint16)
    M, d = x.shape
    ff = w_gu.shape[0] // 2
    y = np.empty((M, d), np.float64)
    _load().oracle_forward_bf16(_p(x), _p(gamma), eps, _p(w_gu), _p(w_down),
                                M, d, ff, _p(y))
    return y


def forward_int4(x, gamma, eps, q_gu, s_gu, q_down, s_down) -> np.ndarray:
    """Eq(1) with RMSNorm prologue, int4 weights w = s*q; fp64."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    q_gu, q_down = _c(q_gu, np.uint8), _c(q_down, np.uint8)
    s_gu, s_down = _c(s_gu, np.uint16), _c(s_down, np.uint16)
    M, d = x.shape
    ff = q_gu.shape[0] // 2
    y = np.empty((M, d), np.float64)
    _load().oracle_forward_int4(_p(x), _p(gamma), eps, _p(q_gu), _p(s_gu),
                                _p(q_down), _p(s_down), M, d, ff, _p(y))
    return y


def forward_int4_ex(x, gamma, eps, q_gu, s_gu, q_down, s_down, act=ACT_SILU, residual=None):
    """forward_int4 with gate activation `act` and the optional residual
    prologue; returns (y, h) as forward_unfused_ex."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    q_gu, q_down = _c(q_gu, np.uint8), _c(q_down, np.uint8)
    s_gu, s_down = _c(s_gu, np.uint16), _c(s_down, np.uint16)
    M, d = x.shape
    ff = q_gu.shape[0] // 2
    y = np.empty((M, d), np.float64)
    res = None if residual is None else _c(residual, np.uint16)
    h = None if residual is None else np.empty((M, d), np.uint16)
    _load().oracle_forward_int4_ex(_p(x), None if res is None else _p(res),
                                   None if h is None else _p(h), _p(gamma), eps, act,
                                   _p(q_gu), _p(s_gu), _p(q_down), _p(s_down), M, d, ff, _p(y))
    return y, h


def bf16_to_f16_trunc(w: np.ndarray):
    """bf16 -> fp16 bits, truncation toward zero (exact in the fp16 normal
    range); returns (out, number of non-finite or > 65504 elements)."""
    w = _c(w, np.uint16)
    out = np.empty(w.shape, np.uint16)
    bad = _load().oracle_bf16_to_f16_trunc(_p(w), w.size, _p(out))
    return out, int(bad)


def forward_f16_ex(x, gamma, eps, w_gu, w_down, act=ACT_SILU, residual=None):
    """Eq(1) with fp16 weights (interleaved w_gu [2ff, d], w_down [d, ff],
    fp16 bits), gate activation `act` and the optional residual prologue;
    returns (y fp64 [M, d], h bf16 bits [M, d] or None)."""
    x, gamma = _c(x, np.uint16), _c(gamma, np.uint16)
    w_gu, w_down = _c(w_gu, np.uint16), _c(w_down, np.uint16)
    M, d = x.shape
    ff = w_gu.shape[0] // 2
    y = np.empty((M, d), np.float64)
    res = None if residual is None else _c(residual, np.uint16)
    h = None if residual is None else np.empty((M, d), np.uint16)
    _load().oracle_forward_f16_ex(_p(x), None if res is None else _p(res),
                                  None if h is None else _p(h), _p(gamma), eps, act,
                                  _p(w_gu), _p(w_down), M, d, ff, _p(y))
    return y, h


# ---------------------------------------------------------------- tiled layouts
# The library's physical weight layout (see the C++ source for the index maps).

def tile_bf16(w: np.ndarray) -> np.ndarray:
    """Row-major bf16 [R, K] -> fragment-tiled (flat, same element count)."""
    w = _c(w, np.uint16)
    R, K = w.shape
    out = np.empty(R * K, np.uint16)
    _load().oracle_tile_bf16(_p(w), R, K, _p(out))
    return out


def untile_bf16(t: np.ndarray, R: int, K: int) -> np.ndarray:
    """Fragment-tiled bf16 (any shape, R*K elements) -> row-major [R, K]."""
    t = _c(t, np.uint16).reshape(-1)
    assert t.size == R * K
    out = np.empty((R, K), np.uint16)
    _load().oracle_untile_bf16(_p(t), R, K, _p(out))
    return out


def int4_tiled_sizes(R: int, K: int):
    """(code bytes, scale count) of the tiled int4 format."""
    L = _load()
    return int(L.oracle_int4_tiled_code_bytes(R, K)), int(L.oracle_int4_tiled_scale_count(R, K))


def tile_int4(q: np.ndarray, s: np.ndarray):
    """Row-major (q [R, K/2], s [R, K/32]) -> tiled (codes, scales), flat."""
    q, s = _c(q, np.uint8), _c(s, np.uint16)
    R, K = q.shape[0], q.shape[1] * 2
    nb, ns = int4_tiled_sizes(R, K)
    qt, st = np.empty(nb, np.uint8), np.empty(ns, np.uint16)
    _load().oracle_tile_int4(_p(q), _p(s), R, K, _p(qt), _p(st))
    return qt, st


def untile_int4(qt: np.ndarray, st: np.ndarray, R: int, K: int):
    """Tiled int4 (flat codes, flat scales) -> row-major (q [R, K/2], s [R, K/32])."""
    qt, st = _c(qt, np.uint8).reshape(-1), _c(st, np.uint16).reshape(-1)
    q = np.empty((R, K // 2), np.uint8)
    s = np.empty((R, K // 32), np.uint16)
    _load().oracle_untile_int4(_p(qt), _p(st), R, K, _p(q), _p(s))
    return q, s
