"""Thin Python binding over libfmlp.so (C ABI in include/fmlp.h).

Argument marshalling only: torch tensors in, raw device pointers and the
current HIP stream handle out, status codes turned into exceptions. Every
step of the computation runs in the library's HIP kernels; there is no
fallback of any kind, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmlp.so")
_lock = threading.Lock()
_lib = None

FMLP_OK = 0
FMLP_ERR_INVALID_ARG = -1
FMLP_ERR_UNSUPPORTED_SHAPE = -2
FMLP_ERR_ALIGNMENT = -3
FMLP_ERR_WORKSPACE = -4
FMLP_ERR_RANGE = -5
FMLP_ERR_HIP = -6
FMLP_ERR_DEVICE = -7

FMLP_W_BF16 = 0
FMLP_W_INT4_G32 = 1
FMLP_W_F16 = 2

FMLP_PATH_AUTO = 0
FMLP_PATH_DECODE = 1
FMLP_PATH_PREFILL = 2
FMLP_PATH_SINGLE_PASS = 3

FMLP_NOALLOC_SCRATCH_BYTES = 32 << 20

FMLP_ACT_SILU = 0
FMLP_ACT_GELU_TANH = 1
FMLP_ACT_GELU_ERF = 2

EXPORTS = (
    "fmlp_pack_interleaved", "fmlp_pack_matrix", "fmlp_int4_sizes", "fmlp_quantize_int4",
    "fmlp_pack_int4_interleaved", "fmlp_pack_int4_matrix", "fmlp_dequant_int4",
    "fmlp_convert_f16", "fmlp_workspace_size", "fmlp_forward", "fmlp_forward_path", "fmlp_forward_ex",
    "fmlp_forward_noalloc",
    "fmlp_status_string", "fmlp_last_hip_error", "fmlp_profile_enable",
    "fmlp_profile_read", "fmlp_kernel_name", "fmlp_read_probe",
)


class FmlpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().fmlp_status_string(status).decode()
        if status == FMLP_ERR_HIP:
            msg += f" (hipError_t {lib().fmlp_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m swiglu_mlp_rmsnorm_amd.build_lib` (hipcc, gfx950)")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.fmlp_pack_interleaved.argtypes = [P, P, P, I64, I64, P]
        L.fmlp_pack_matrix.argtypes = [P, P, I64, I64, P]
        L.fmlp_int4_sizes.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
        L.fmlp_quantize_int4.argtypes = [P, I64, I64, P, P, P]
        L.fmlp_pack_int4_interleaved.argtypes = [P, P, P, P, I64, I64, P, P, P]
        L.fmlp_pack_int4_matrix.argtypes = [P, P, I64, I64, P, P, P]
        L.fmlp_dequant_int4.argtypes = [P, P, I64, I64, P, P]
        L.fmlp_convert_f16.argtypes = [P, P, I64, P]
        L.fmlp_workspace_size.argtypes = [I64, I64, I64, I32]
        L.fmlp_workspace_size.restype = SZ
        fwd = [P, P, ctypes.c_float, I32, P, P, P, P, P, I64, I64, I64, P, SZ, P]
        L.fmlp_forward.argtypes = fwd
        L.fmlp_forward_path.argtypes = fwd + [I32]
        L.fmlp_forward_noalloc.argtypes = [P, P, ctypes.c_float, I32, P, P, P, P, P, I64, I64, I64,
                                           P]
        L.fmlp_forward_ex.argtypes = [P, P, P, P, ctypes.c_float, I32, I32, P, P, P, P, P, I64, I64,
                                      I64, P, SZ, P, I32]
        L.fmlp_status_string.argtypes = [ctypes.c_int]
        L.fmlp_status_string.restype = ctypes.c_char_p
        L.fmlp_last_hip_error.argtypes = []
        L.fmlp_profile_enable.argtypes = [I32]
        L.fmlp_profile_read.argtypes = [I32, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_double)]
        L.fmlp_read_probe.argtypes = [P, I64, P, I32, P]
        L.fmlp_read_probe.restype = ctypes.c_int
        L.fmlp_kernel_name.argtypes = [I32]
        L.fmlp_kernel_name.restype = ctypes.c_char_p
        for name in ("fmlp_pack_interleaved", "fmlp_pack_matrix", "fmlp_int4_sizes",
                     "fmlp_quantize_int4", "fmlp_pack_int4_interleaved",
                     "fmlp_pack_int4_matrix", "fmlp_dequant_int4", "fmlp_convert_f16",
                     "fmlp_forward", "fmlp_forward_path", "fmlp_forward_ex",
                     "fmlp_forward_noalloc", "fmlp_last_hip_error",
                     "fmlp_profile_enable", "fmlp_profile_read"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
        return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st: int, where: str):
    if st != FMLP_OK:
        raise FmlpError(st, where)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def fmlp_status_string(status: int) -> str:
    return lib().fmlp_status_string(status).decode()


def fmlp_pack_interleaved(w_gate, w_up, w_gu=None, stream=None):
    """W_gu[2i] = W_gate[i], W_gu[2i+1] = W_up[i]; bf16 [ff,d] x2 -> [2ff,d]."""
    _need(w_gate, torch.bfloat16, "w_gate")
    _need(w_up, torch.bfloat16, "w_up")
    ff, d = w_gate.shape
    if w_up.shape != (ff, d):
        raise ValueError("w_up shape differs from w_gate")
    if w_gu is None:
        w_gu = torch.empty((2 * ff, d), dtype=torch.bfloat16, device=w_gate.device)
    _need(w_gu, torch.bfloat16, "w_gu")
    if w_gu.shape != (2 * ff, d):
        raise ValueError("w_gu must be [2ff, d]")
    _check(lib().fmlp_pack_interleaved(_ptr(w_gate), _ptr(w_up), _ptr(w_gu), ff, d,
                                       _stream(stream)), "fmlp_pack_interleaved")
    return w_gu


def fmlp_pack_matrix(w, w_tiled=None, stream=None):
    """Row-major bf16 [rows, K] -> the same matrix in the tiled layout (shape kept)."""
    _need(w, torch.bfloat16, "w")
    rows, K = w.shape
    if w_tiled is None:
        w_tiled = torch.empty((rows, K), dtype=torch.bfloat16, device=w.device)
    _need(w_tiled, torch.bfloat16, "w_tiled")
    if w_tiled.numel() != rows * K:
        raise ValueError("w_tiled must hold rows*K elements")
    _check(lib().fmlp_pack_matrix(_ptr(w), _ptr(w_tiled), rows, K, _stream(stream)),
           "fmlp_pack_matrix")
    return w_tiled


def fmlp_int4_sizes(rows: int, K: int):
    """(code bytes, scale bytes) of a tiled int4 [rows, K] matrix."""
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().fmlp_int4_sizes(rows, K, ctypes.byref(cb), ctypes.byref(sb)), "fmlp_int4_sizes")
    return int(cb.value), int(sb.value)


def fmlp_quantize_int4(w, q=None, scales=None, stream=None):
    """Row-major bf16 [rows, K] -> int4 exchange format: codes uint8
    [rows, K/2] (even column in the low nibble) and fp16 scales [rows, K/32]."""
    _need(w, torch.bfloat16, "w")
    rows, K = w.shape
    if q is None:
        q = torch.empty((rows, K // 2), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((rows, K // 32), dtype=torch.float16, device=w.device)
    _need(q, torch.uint8, "q")
    _need(scales, torch.float16, "scales")
    if q.shape != (rows, K // 2) or scales.shape != (rows, K // 32):
        raise ValueError("q must be [rows, K/2] and scales [rows, K/32]")
    _check(lib().fmlp_quantize_int4(_ptr(w), rows, K, _ptr(q), _ptr(scales), _stream(stream)),
           "fmlp_quantize_int4")
    return q, scales


def _need_int4(q, s, name):
    _need(q, torch.uint8, name + " codes")
    _need(s, torch.float16, name + " scales")
    if q.dim() != 2 or s.dim() != 2 or q.shape[0] != s.shape[0] or q.shape[1] != 16 * s.shape[1]:
        raise ValueError(f"{name}: codes must be [rows, K/2] and scales [rows, K/32]")
    return q.shape[0], q.shape[1] * 2


def _tiled_int4_buffers(rows, K, device, q_tiled, s_tiled):
    cb, sb = fmlp_int4_sizes(rows, K)
    if q_tiled is None:
        q_tiled = torch.empty(cb, dtype=torch.uint8, device=device)
    if s_tiled is None:
        s_tiled = torch.empty(sb // 2, dtype=torch.float16, device=device)
    _need(q_tiled, torch.uint8, "q_tiled")
    _need(s_tiled, torch.float16, "s_tiled")
    if q_tiled.numel() < cb or s_tiled.numel() * 2 < sb:
        raise ValueError("tiled int4 buffers too small")
    return q_tiled, s_tiled


def fmlp_pack_int4_interleaved(q_gate, s_gate, q_up, s_up, q_gu=None, s_gu=None, stream=None):
    """Exchange-format int4 gate and up [ff, d] -> tiled int4 (flat codes,
    flat scales) of the interleaved [2ff, d] matrix (gate row i at 2i)."""
    ff, d = _need_int4(q_gate, s_gate, "gate")
    if _need_int4(q_up, s_up, "up") != (ff, d):
        raise ValueError("up shape differs from gate")
    q_gu, s_gu = _tiled_int4_buffers(2 * ff, d, q_gate.device, q_gu, s_gu)
    _check(lib().fmlp_pack_int4_interleaved(_ptr(q_gate), _ptr(s_gate), _ptr(q_up), _ptr(s_up),
                                            ff, d, _ptr(q_gu), _ptr(s_gu), _stream(stream)),
           "fmlp_pack_int4_interleaved")
    return q_gu, s_gu


def fmlp_pack_int4_matrix(q, scales, q_tiled=None, s_tiled=None, stream=None):
    """Exchange-format int4 [rows, K] -> tiled int4 (flat codes, flat scales)."""
    rows, K = _need_int4(q, scales, "matrix")
    q_tiled, s_tiled = _tiled_int4_buffers(rows, K, q.device, q_tiled, s_tiled)
    _check(lib().fmlp_pack_int4_matrix(_ptr(q), _ptr(scales), rows, K, _ptr(q_tiled),
                                       _ptr(s_tiled), _stream(stream)), "fmlp_pack_int4_matrix")
    return q_tiled, s_tiled


def fmlp_dequant_int4(q, scales, out=None, stream=None):
    """Exchange-format int4 (codes [rows, K/2], scales [rows, K/32]) ->
    exact row-major fp32 [rows, K]."""
    rows, K = _need_int4(q, scales, "int4")
    if out is None:
        out = torch.empty((rows, K), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out")
    if out.shape != (rows, K):
        raise ValueError("out must be [rows, K]")
    _check(lib().fmlp_dequant_int4(_ptr(q), _ptr(scales), rows, K, _ptr(out), _stream(stream)),
           "fmlp_dequant_int4")
    return out


def fmlp_convert_f16(w, out=None, stream=None):
    """bf16 weights (any shape, e.g. the tiled matrices) -> fp16 of the same
    shape, truncating toward zero; the FMLP_W_F16 weight type."""
    _need(w, torch.bfloat16, "w")
    if out is None:
        out = torch.empty(w.shape, dtype=torch.float16, device=w.device)
    _need(out, torch.float16, "out")
    if out.numel() != w.numel():
        raise ValueError("out must hold as many elements as w")
    _check(lib().fmlp_convert_f16(_ptr(w), _ptr(out), w.numel(), _stream(stream)),
           "fmlp_convert_f16")
    return out


def fmlp_workspace_size(M: int, d: int, ff: int, wtype: int = FMLP_W_BF16) -> int:
    return int(lib().fmlp_workspace_size(M, d, ff, wtype))


def _forward(x, gamma, eps, w_gu, w_down, gu_scales, down_scales, y, workspace, stream, path,
             ff=None, activation=None, residual=None, h_out=None):
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    M, d = x.shape
    int4 = w_gu.dtype == torch.uint8
    if int4:
        _need(w_gu, torch.uint8, "w_gu")
        _need(w_down, torch.uint8, "w_down")
        _need(gu_scales, torch.float16, "gu_scales")
        _need(down_scales, torch.float16, "down_scales")
        if ff is None:
            raise ValueError("int4 weights are flat buffers: pass ff")
        wtype = FMLP_W_INT4_G32
        for (t, s_, R, K) in ((w_gu, gu_scales, 2 * ff, d), (w_down, down_scales, d, ff)):
            cb, sb = fmlp_int4_sizes(R, K)
            if t.numel() < cb or s_.numel() * 2 < sb:
                raise ValueError("int4 weight buffers too small for the shapes")
    else:
        wdt = torch.float16 if w_gu.dtype == torch.float16 else torch.bfloat16
        _need(w_gu, wdt, "w_gu")
        _need(w_down, wdt, "w_down")
        ff = w_down.shape[1]
        wtype = FMLP_W_F16 if wdt == torch.float16 else FMLP_W_BF16
        if w_gu.shape != (2 * ff, d) or w_down.shape != (d, ff):
            raise ValueError("weight shapes do not match x")
    if gamma.shape != (d,):
        raise ValueError("gamma must be [d]")
    if y is None:
        y = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if y.shape != (M, d):
        raise ValueError("y must be [M, d]")
    need = fmlp_workspace_size(M, d, ff, wtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _need(workspace, torch.uint8, "workspace")
    args = (_ptr(x), _ptr(gamma), float(eps), wtype, _ptr(w_gu), _ptr(gu_scales), _ptr(w_down),
            _ptr(down_scales), _ptr(y), M, d, ff, _ptr(workspace), workspace.numel(),
            _stream(stream))
    if activation is not None:  # fmlp_forward_ex
        if residual is not None:
            _need(residual, torch.bfloat16, "residual")
            if residual.shape != (M, d):
                raise ValueError("residual must be [M, d]")
            if h_out is None:
                h_out = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
            _need(h_out, torch.bfloat16, "h_out")
            if h_out.shape != (M, d):
                raise ValueError("h_out must be [M, d]")
        elif h_out is not None:
            raise ValueError("h_out is written only together with a residual")
        _check(lib().fmlp_forward_ex(_ptr(x), _ptr(residual), _ptr(h_out), _ptr(gamma),
                                     float(eps), int(activation), wtype, _ptr(w_gu),
                                     _ptr(gu_scales), _ptr(w_down), _ptr(down_scales), _ptr(y),
                                     M, d, ff, _ptr(workspace), workspace.numel(),
                                     _stream(stream), FMLP_PATH_AUTO if path is None else path),
               "fmlp_forward_ex")
        return y, h_out
    if path is None:
        _check(lib().fmlp_forward(*args), "fmlp_forward")
    else:
        _check(lib().fmlp_forward_path(*args, path), "fmlp_forward_path")
    return y


def fmlp_forward(x, gamma, eps, w_gu, w_down, gu_scales=None, down_scales=None, y=None,
                 workspace=None, stream=None, ff=None):
    """y = W_down(SiLU(W_gate n) * (W_up n)), n = RMSNorm(x); bf16 x [M,d] -> y [M,d].

    bf16 weights: tiled w_gu [2ff,d] (fmlp_pack_interleaved) and tiled w_down
    [d,ff] (fmlp_pack_matrix); fp16 weights: those after fmlp_convert_f16.
    int4 weights: the flat tiled code/scale buffers of fmlp_pack_int4_interleaved
    (W_gu) and fmlp_pack_int4_matrix (W_down), with ff given explicitly.
    Output and workspace are allocated with torch when not given.
    """
    return _forward(x, gamma, eps, w_gu, w_down, gu_scales, down_scales, y, workspace, stream,
                    None, ff)


def fmlp_forward_path(x, gamma, eps, w_gu, w_down, gu_scales=None, down_scales=None, y=None,
                      workspace=None, stream=None, path=FMLP_PATH_AUTO, ff=None):
    """fmlp_forward with the kernel path chosen by the caller (FMLP_PATH_*)."""
    return _forward(x, gamma, eps, w_gu, w_down, gu_scales, down_scales, y, workspace, stream,
                    path, ff)


def fmlp_forward_ex(x, gamma, eps, w_gu, w_down, gu_scales=None, down_scales=None, y=None,
                    workspace=None, stream=None, path=FMLP_PATH_AUTO, ff=None,
                    activation=FMLP_ACT_SILU, residual=None, h_out=None):
    """fmlp_forward_path with a gate activation (FMLP_ACT_*) and an optional
    residual input: then the row normalised is h = bf16(x + residual), also
    returned in h_out. Returns (y, h_out or None)."""
    return _forward(x, gamma, eps, w_gu, w_down, gu_scales, down_scales, y, workspace, stream,
                    path, ff, activation, residual, h_out)


def fmlp_forward_noalloc(x, gamma, eps, w_gu, w_down, gu_scales=None, down_scales=None, y=None,
                         stream=None, ff=None):
    """fmlp_forward with the library's fixed device scratch instead of a
    workspace (FMLP_NOALLOC_SCRATCH_BYTES); for callers that cannot allocate.
    Calls that overlap in time on one GPU race on that scratch."""
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    M, d = x.shape
    if w_gu.dtype == torch.uint8:
        _need(w_gu, torch.uint8, "w_gu")
        _need(w_down, torch.uint8, "w_down")
        _need(gu_scales, torch.float16, "gu_scales")
        _need(down_scales, torch.float16, "down_scales")
        if ff is None:
            raise ValueError("int4 weights are flat buffers: pass ff")
        wtype = FMLP_W_INT4_G32
    else:
        wtype = FMLP_W_F16 if w_gu.dtype == torch.float16 else FMLP_W_BF16
        _need(w_gu, w_gu.dtype, "w_gu")
        _need(w_down, w_gu.dtype, "w_down")
        ff = w_down.shape[1]
        if w_gu.shape != (2 * ff, d) or w_down.shape != (d, ff):
            raise ValueError("weight shapes do not match x")
    if y is None:
        y = torch.empty((M, d), dtype=torch.bfloat16, device=x.device)
    _need(y, torch.bfloat16, "y")
    if y.shape != (M, d):
        raise ValueError("y must be [M, d]")
    _check(lib().fmlp_forward_noalloc(_ptr(x), _ptr(gamma), float(eps), wtype, _ptr(w_gu),
                                      _ptr(gu_scales), _ptr(w_down), _ptr(down_scales), _ptr(y),
                                      M, d, ff, _stream(stream)), "fmlp_forward_noalloc")
    return y


def fmlp_read_probe(src, sink, workgroups: int, stream=None) -> None:
    """Read all of the device tensor src once (measurement probe); sink is
    an int32 device tensor of at least workgroups*256 elements."""
    if not (src.is_cuda and sink.is_cuda):
        raise ValueError("fmlp_read_probe takes device tensors")
    if sink.numel() * sink.element_size() < workgroups * 256 * 4:
        raise ValueError("sink too small")
    _check(lib().fmlp_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                 int(workgroups), _stream(stream)), "fmlp_read_probe")


def fmlp_kernel_names() -> list:
    """Kernel kinds known to the profiler, in kind order."""
    names, k = [], 0
    while True:
        n = lib().fmlp_kernel_name(k)
        if n is None:
            return names
        names.append(n.decode())
        k += 1


def fmlp_profile_enable(on: bool = True) -> None:
    _check(lib().fmlp_profile_enable(1 if on else 0), "fmlp_profile_enable")


def fmlp_profile_read() -> dict:
    """{kernel name: (launches, total GPU ms)} for every kind with launches."""
    out = {}
    for k, name in enumerate(fmlp_kernel_names()):
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _check(lib().fmlp_profile_read(k, ctypes.byref(n), ctypes.byref(ms)), "fmlp_profile_read")
        if n.value:
            out[name] = (int(n.value), float(ms.value))
    return out
