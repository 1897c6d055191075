"""The C ABI boundary, without a GPU: the library loads, exports every entry
point include/fmlp.h declares, and rejects bad arguments on the host before
any HIP call (so these run on a CPU-only machine)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from swiglu_mlp_rmsnorm_amd import fmlp as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmlp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F._LIB_PATH),
                                reason="libfmlp.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fmlp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(F.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", F._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fmlp_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(F.lib(), name)


# distinct, 16-byte aligned fake device addresses far apart (never dereferenced)
A = {k: ctypes.c_void_p((i + 1) << 36) for i, k in enumerate(
    ["x", "g", "wgu", "sgu", "wd", "sd", "y", "ws"])}
BIG = 1 << 34


def fwd(M=1, d=256, ff=704, eps=1e-5, wtype=0, path=0, ws_bytes=BIG, **over):
    p = dict(A)
    p.update(over)
    return F.lib().fmlp_forward_path(p["x"], p["g"], eps, wtype, p["wgu"], p["sgu"], p["wd"],
                                     p["sd"], p["y"], M, d, ff, p["ws"], ws_bytes, None, path)


@pytest.mark.parametrize("kw,status", [
    (dict(wtype=7), F.FMLP_ERR_INVALID_ARG),
    (dict(path=9), F.FMLP_ERR_INVALID_ARG),
    (dict(M=-1), F.FMLP_ERR_INVALID_ARG),
    (dict(d=48), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(ff=0), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(ff=720), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(d=65536 + 32), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(M=(1 << 24) + 1), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(eps=float("nan")), F.FMLP_ERR_INVALID_ARG),
    (dict(eps=float("inf")), F.FMLP_ERR_INVALID_ARG),
    (dict(eps=-1e-5), F.FMLP_ERR_INVALID_ARG),
    (dict(x=None), F.FMLP_ERR_INVALID_ARG),
    (dict(ws=None), F.FMLP_ERR_INVALID_ARG),
    (dict(wtype=1, sgu=None), F.FMLP_ERR_INVALID_ARG),
    (dict(y=ctypes.c_void_p((7 << 36) + 8)), F.FMLP_ERR_ALIGNMENT),
    (dict(wgu=ctypes.c_void_p((3 << 36) + 4)), F.FMLP_ERR_ALIGNMENT),
    (dict(M=33, path=1), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(M=9, path=3), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(M=1, path=3, wtype=1), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(M=1, path=3, wtype=2), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(wtype=3), F.FMLP_ERR_INVALID_ARG),
    (dict(wtype=2, ws_bytes=100), F.FMLP_ERR_WORKSPACE),
    (dict(wtype=2, y=A["wd"]), F.FMLP_ERR_INVALID_ARG),
    (dict(path=4), F.FMLP_ERR_INVALID_ARG),
    (dict(ws_bytes=100), F.FMLP_ERR_WORKSPACE),
    (dict(y=A["x"]), F.FMLP_ERR_INVALID_ARG),
    (dict(y=A["ws"]), F.FMLP_ERR_INVALID_ARG),
    (dict(ws=A["wd"]), F.FMLP_ERR_INVALID_ARG),
    # a workspace over the int4 scales (which the kernels read while they
    # write the workspace)
    (dict(wtype=1, ws=A["sgu"]), F.FMLP_ERR_INVALID_ARG),
    (dict(wtype=1, ws=A["sd"]), F.FMLP_ERR_INVALID_ARG),
    (dict(wtype=1, ws=ctypes.c_void_p((4 << 36) - 4096)), F.FMLP_ERR_INVALID_ARG),
])
def test_forward_rejects_before_any_hip_call(kw, status):
    assert fwd(**kw) == status


A_EX = dict(A, r=ctypes.c_void_p(9 << 36), h=ctypes.c_void_p(10 << 36))


def fwd_ex(M=1, d=256, ff=704, eps=1e-5, act=0, wtype=0, path=0, ws_bytes=BIG, **over):
    p = dict(A_EX)
    p.update(over)
    return F.lib().fmlp_forward_ex(p["x"], p["r"], p["h"], p["g"], eps, act, wtype, p["wgu"],
                                   p["sgu"], p["wd"], p["sd"], p["y"], M, d, ff, p["ws"],
                                   ws_bytes, None, path)


@pytest.mark.parametrize("kw,status", [
    (dict(act=3), F.FMLP_ERR_INVALID_ARG),
    (dict(act=-1), F.FMLP_ERR_INVALID_ARG),
    (dict(h=None), F.FMLP_ERR_INVALID_ARG),                  # residual without h_out
    (dict(r=None), F.FMLP_ERR_INVALID_ARG),                  # h_out without residual
    (dict(r=ctypes.c_void_p((9 << 36) + 2)), F.FMLP_ERR_ALIGNMENT),
    (dict(h=ctypes.c_void_p((10 << 36) + 8)), F.FMLP_ERR_ALIGNMENT),
    (dict(h=A["x"]), F.FMLP_ERR_INVALID_ARG),                # h_out over x
    (dict(h=A["y"]), F.FMLP_ERR_INVALID_ARG),                # h_out over y
    (dict(h=A["ws"]), F.FMLP_ERR_INVALID_ARG),               # h_out over the workspace
    (dict(h=ctypes.c_void_p((9 << 36) + 256)), F.FMLP_ERR_INVALID_ARG),  # h_out over residual
    (dict(r=A["y"]), F.FMLP_ERR_INVALID_ARG),                # y over residual
    (dict(act=1, path=3, wtype=1), F.FMLP_ERR_UNSUPPORTED_SHAPE),
    (dict(act=2, ws_bytes=100), F.FMLP_ERR_WORKSPACE),
])
def test_forward_ex_rejects_before_any_hip_call(kw, status):
    assert fwd_ex(**kw) == status


def test_forward_ex_zero_tokens_and_defaults():
    assert fwd_ex(M=0, x=None, y=None, ws=None, r=None, h=None) == F.FMLP_OK
    # without a residual and with SiLU the checks are those of fmlp_forward_path
    for kw in (dict(d=48), dict(M=33, path=1), dict(ws_bytes=100)):
        assert fwd_ex(r=None, h=None, **kw) == fwd(**kw)


def test_noalloc_host_checks():
    # fmlp_forward_noalloc: fmlp_forward's host-side checks, and a problem
    # that does not fit the fixed scratch is rejected before any HIP call
    L = F.lib()

    def na(M=1, d=256, ff=704, wtype=0, **over):
        p = dict(A)
        p.update(over)
        return L.fmlp_forward_noalloc(p["x"], p["g"], 1e-5, wtype, p["wgu"], p["sgu"], p["wd"],
                                      p["sd"], p["y"], M, d, ff, None)
    assert na(M=0, x=None, y=None) == F.FMLP_OK
    assert na(wtype=7) == F.FMLP_ERR_INVALID_ARG
    assert na(d=48) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert na(y=A["x"]) == F.FMLP_ERR_INVALID_ARG
    assert na(wtype=1, sgu=None) == F.FMLP_ERR_INVALID_ARG
    assert na(y=ctypes.c_void_p((7 << 36) + 8)) == F.FMLP_ERR_ALIGNMENT
    assert na(M=2048, d=4096, ff=14336) == F.FMLP_ERR_WORKSPACE
    assert F.fmlp_workspace_size(2048, 4096, 14336) > F.FMLP_NOALLOC_SCRATCH_BYTES
    # every decode problem up to 32 tokens with d <= 8192, ff <= 28672 fits
    # (the automatic path's own need; fmlp_workspace_size also covers the
    # forced single-pass path, which this entry point never takes)
    for d, ff in ((3072, 8192), (4096, 14336), (8192, 28672)):
        for wt in (0, 1, 2):
            for M in (1, 8, 16, 17, 32):
                assert na(M=M, d=d, ff=ff, wtype=wt) != F.FMLP_ERR_WORKSPACE, (d, ff, wt, M)


def test_read_probe_validation():
    L = F.lib()
    src, sink = ctypes.c_void_p(1 << 36), ctypes.c_void_p(2 << 36)
    assert L.fmlp_read_probe(None, 1024, sink, 256, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_read_probe(src, 0, sink, 256, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_read_probe(src, 1024, sink, 0, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_read_probe(src, 1000, sink, 256, None) == F.FMLP_ERR_ALIGNMENT
    assert L.fmlp_read_probe(ctypes.c_void_p((1 << 36) + 8), 1024, sink, 256,
                             None) == F.FMLP_ERR_ALIGNMENT


def test_int4_prefill_passes_the_host_checks():
    # int4 weights at M > 32 take the prefill path: the host-side checks
    # accept them exactly as they accept bf16 (the call then needs a GPU)
    assert fwd(M=64, wtype=1) == fwd(M=64, wtype=0)
    assert fwd(M=64, wtype=1) != F.FMLP_ERR_UNSUPPORTED_SHAPE


def test_f16_weights_pass_the_host_checks():
    # fp16 weights: same buffer sizes as bf16, scales ignored (may be NULL),
    # on either path; the workspace matches bf16's except for the single pass
    for M in (1, 16, 17, 64):
        assert fwd(M=M, wtype=2, sgu=None, sd=None) == fwd(M=M, wtype=0)
    ws = F.fmlp_workspace_size
    assert ws(2048, 4096, 14336, 2) == ws(2048, 4096, 14336, 0)
    for M in (9, 33):  # no single-pass partials (the bf16 size keeps them at every M)
        assert ws(M, 4096, 14336, 2) < ws(M, 4096, 14336, 0)
    # int4 prefill dequantises inside the GEMMs: no weight expansion in the
    # workspace, so int4 needs what fp16 needs on every path but the
    # single pass (bf16 only)
    for M in (1, 16, 32, 33, 512, 2048):
        assert ws(M, 8192, 28672, 1) == ws(M, 8192, 28672, 2)
    # the 70B decode configuration: well under 8 MB (was 1.41 GB with the
    # fp16 expansion)
    assert ws(16, 8192, 28672, 1) < 8 << 20
    assert ws(1, 8192, 28672, 1) < 8 << 20


def test_convert_f16_validation():
    L = F.lib()
    a, c = A["x"], A["y"]
    assert L.fmlp_convert_f16(None, c, 64, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_convert_f16(a, None, 64, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_convert_f16(a, c, 0, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_convert_f16(a, c, 60, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_convert_f16(a, c, 0x7FFFFFFF * 2048 + 8, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_convert_f16(a, ctypes.c_void_p(A["y"].value + 2), 64,
                              None) == F.FMLP_ERR_ALIGNMENT
    assert L.fmlp_convert_f16(a, a, 64, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_convert_f16(a, ctypes.c_void_p(A["x"].value + 64), 64,
                              None) == F.FMLP_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op():
    assert fwd(M=0, x=None, y=None, ws=None) == F.FMLP_OK


def test_workspace_size():
    ws = F.fmlp_workspace_size
    assert ws(1, 256, 704) > 0
    assert ws(32, 4096, 14336) >= ws(1, 4096, 14336)
    assert ws(2048, 4096, 14336) >= 2 * 2048 * (4096 + 14336)
    assert ws(1, 48, 704) == 0 and ws(-1, 256, 704) == 0 and ws(1, 256, 704, 5) == 0
    # the reported size covers either path; at M=1 the prefill path (tokens
    # padded to 32) is the larger, so one byte under it (beyond the 256-byte
    # alignment slack) is rejected there
    need = ws(1, 256, 704)
    assert fwd(ws_bytes=need - 256 - 1, path=F.FMLP_PATH_PREFILL) == F.FMLP_ERR_WORKSPACE
    # the single-pass decode keeps (ff/32) * M * d fp32 partial sums; at
    # Phi-3 size and M = 8 that is the largest need of the three paths
    assert ws(8, 3072, 8192) >= (8192 // 32) * 8 * 3072 * 4
    need = ws(8, 3072, 8192)
    assert fwd(M=8, d=3072, ff=8192, ws_bytes=need - 256 - 1,
               path=F.FMLP_PATH_SINGLE_PASS) == F.FMLP_ERR_WORKSPACE


SHAPES = [(256, 704), (3072, 8192), (4096, 14336), (8192, 28672), (1024, 2048), (32, 3104),
          (96, 6176), (4128, 64)]


@pytest.mark.parametrize("d,ff", SHAPES)
@pytest.mark.parametrize("wtype", [0, 1, 2])
def test_workspace_size_never_decreases(d, ff, wtype):
    # a buffer sized for the largest M serves every smaller M, on every path
    ws = F.fmlp_workspace_size
    sizes = [ws(M, d, ff, wtype) for M in range(0, 4097)]
    for M in range(1, 4097):
        assert sizes[M] >= sizes[M - 1], (d, ff, wtype, M, sizes[M - 1], sizes[M])
    # and each size passes the forward's own check on every path it can take
    for M in (1, 8, 31, 32, 33, 257, 258, 1000, 4096):
        for path in (0, 1, 2, 3):
            st = fwd(M=M, d=d, ff=ff, wtype=wtype, path=path, ws_bytes=sizes[4096])
            assert st != F.FMLP_ERR_WORKSPACE, (d, ff, wtype, M, path)
            st = fwd(M=M, d=d, ff=ff, wtype=wtype, path=path, ws_bytes=sizes[M])
            assert st != F.FMLP_ERR_WORKSPACE, (d, ff, wtype, M, path)


def test_pack_quant_dequant_validation():
    L = F.lib()
    a, b, c, e = A["x"], A["g"], A["y"], A["ws"]
    assert L.fmlp_pack_interleaved(None, b, c, 704, 256, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_interleaved(a, b, c, 704, 250, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_pack_interleaved(a, b, ctypes.c_void_p(A["y"].value + 2), 704, 256,
                                   None) == F.FMLP_ERR_ALIGNMENT
    assert L.fmlp_pack_interleaved(a, b, a, 704, 256, None) == F.FMLP_ERR_INVALID_ARG
    # quantiser: row-major, any row count, K a multiple of 32
    assert L.fmlp_quantize_int4(a, 16, 48, b, c, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_quantize_int4(a, 0, 64, b, c, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_quantize_int4(a, 16, 64, None, c, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_quantize_int4(a, 16, 64, a, c, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_quantize_int4(a, 16, 64, b, ctypes.c_void_p(A["x"].value + 512),
                                None) == F.FMLP_ERR_INVALID_ARG  # scales over w
    assert L.fmlp_quantize_int4(a, 16, 64, b, ctypes.c_void_p(A["g"].value + 256),
                                None) == F.FMLP_ERR_INVALID_ARG  # scales over q
    assert L.fmlp_quantize_int4(a, 8, 64, b, ctypes.c_void_p(A["g"].value + 8),
                                None) == F.FMLP_ERR_ALIGNMENT
    # dequant: row-major in, any row count
    assert L.fmlp_dequant_int4(a, b, 0, 64, c, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_dequant_int4(a, b, 16, 48, c, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_dequant_int4(a, b, 16, 64, ctypes.c_void_p(A["y"].value + 4),
                               None) == F.FMLP_ERR_ALIGNMENT
    assert L.fmlp_dequant_int4(a, b, 16, 64, ctypes.c_void_p(A["x"].value + 256),
                               None) == F.FMLP_ERR_INVALID_ARG  # out over q
    # int4 packers: the tiled outputs need 16-row blocks
    assert L.fmlp_pack_int4_matrix(a, b, 24, 64, c, e, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_pack_int4_matrix(a, b, 16, 48, c, e, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_pack_int4_matrix(None, b, 16, 64, c, e, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_matrix(a, b, 16, 64, c, c, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_matrix(a, b, 16, 64, a, e, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_matrix(a, b, 16, 64, c, b, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_matrix(a, b, 16, 64, c, ctypes.c_void_p(A["ws"].value + 2),
                                   None) == F.FMLP_ERR_ALIGNMENT
    g2, u1, u2 = A["sgu"], A["wd"], A["sd"]
    assert L.fmlp_pack_int4_interleaved(a, b, u1, u2, 704, 250, c, e,
                                        None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_pack_int4_interleaved(a, b, u1, None, 704, 256, c, e,
                                        None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_interleaved(a, b, u1, u2, 704, 256, u1, e,
                                        None) == F.FMLP_ERR_INVALID_ARG  # codes over up
    assert L.fmlp_pack_int4_interleaved(a, b, u1, u2, 704, 256, c, b,
                                        None) == F.FMLP_ERR_INVALID_ARG  # scales over gate's
    assert L.fmlp_pack_int4_interleaved(a, b, u1, u2, 704, 256, c, c,
                                        None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_int4_interleaved(a, g2, u1, u2, 704, 256, c, ctypes.c_void_p(
        A["ws"].value + 8), None) == F.FMLP_ERR_ALIGNMENT
    assert L.fmlp_pack_matrix(a, None, 16, 64, None) == F.FMLP_ERR_INVALID_ARG
    assert L.fmlp_pack_matrix(a, c, 24, 64, None) == F.FMLP_ERR_UNSUPPORTED_SHAPE
    assert L.fmlp_pack_matrix(a, a, 16, 64, None) == F.FMLP_ERR_INVALID_ARG


def test_int4_sizes_match_the_format():
    from oracle import oracle
    for R, K in ((16, 32), (64, 704), (57344, 8192), (8192, 28672)):
        assert F.fmlp_int4_sizes(R, K) == (oracle.int4_tiled_sizes(R, K)[0],
                                           oracle.int4_tiled_sizes(R, K)[1] * 2)
    with pytest.raises(F.FmlpError):
        F.fmlp_int4_sizes(8, 64)


def test_status_strings():
    for st in range(-7, 1):
        s = F.fmlp_status_string(st)
        assert s and s != "unknown status"
    assert F.fmlp_status_string(-99) == "unknown status"
    # the thread's last recorded hipError_t: 0, or what an earlier call that
    # reached the HIP runtime on this GPU-less host left there
    assert F.lib().fmlp_last_hip_error() >= 0


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        F.fmlp_forward(x, torch.zeros(256, dtype=torch.bfloat16), 1e-5,
                       torch.zeros(1408, 256, dtype=torch.bfloat16),
                       torch.zeros(256, 704, dtype=torch.bfloat16))
    assert math.isfinite(1e-5)
