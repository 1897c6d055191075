// C ABI of libfmlp.so (declared in include/fmlp.h): argument validation,
// path choice and kernel launch. Validation is host-only and runs before any
// HIP call, so every argument error is reported without touching the GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/fmlp.h"
#include "launch.hpp"

namespace {

thread_local int t_last_hip_error = 0;

int hip_fail(hipError_t e) {
  t_last_hip_error = (int)e;
  return FMLP_ERR_HIP;
}

constexpr int64_t kMaxD = 65536, kMaxFF = 262144, kMaxM = int64_t(1) << 24;
// fmlp_convert_f16: 8 elements per thread, 256 threads per workgroup, and a
// grid of at most 2^31 - 1 workgroups
constexpr int64_t kMaxConvert = int64_t(0x7fffffff) * 2048;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Span{b, b + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool wtype_ok(int32_t wtype) {
  return wtype == FMLP_W_BF16 || wtype == FMLP_W_INT4_G32 || wtype == FMLP_W_F16;
}

bool shape_ok(int64_t d, int64_t ff) {
  return d > 0 && ff > 0 && d % 32 == 0 && ff % 32 == 0 && d <= kMaxD && ff <= kMaxFF;
}

// a logical [rows, K] weight matrix in the tiled formats
bool matrix_ok(int64_t rows, int64_t K) {
  return rows > 0 && K > 0 && rows % 16 == 0 && K % 32 == 0 && rows <= 2 * kMaxFF && K <= kMaxFF;
}

// a row-major [rows, K] matrix in the int4 exchange format (no row blocking)
bool rowmajor_ok(int64_t rows, int64_t K) {
  return rows > 0 && K > 0 && K % 32 == 0 && rows <= 2 * kMaxFF && K <= kMaxFF;
}

// Device check, cached once per device (querying properties on every launch
// costs host time in a decode loop; the V100 report in the llama.cpp digest
// measured exactly that).
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return FMLP_ERR_DEVICE;
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_ok[dev] = 0;
      return;
    }
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  return g_dev_ok[dev] ? FMLP_OK : FMLP_ERR_DEVICE;
}

std::mutex g_flag_mutex;  // the range flags are one per device

}  // namespace

extern "C" {

const char* fmlp_status_string(int status) {
  switch (status) {
    case FMLP_OK: return "ok";
    case FMLP_ERR_INVALID_ARG: return "invalid argument";
    case FMLP_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case FMLP_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case FMLP_ERR_WORKSPACE: return "workspace too small";
    case FMLP_ERR_RANGE: return "value out of fp16 range";
    case FMLP_ERR_HIP: return "HIP runtime error";
    case FMLP_ERR_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
  }
}

int fmlp_last_hip_error(void) { return t_last_hip_error; }

int fmlp_pack_interleaved(const void* w_gate, const void* w_up, void* w_gu, int64_t ff, int64_t d,
                          void* stream) {
  if (!w_gate || !w_up || !w_gu) return FMLP_ERR_INVALID_ARG;
  if (!shape_ok(d, ff)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_gu)) return FMLP_ERR_ALIGNMENT;
  const size_t in_b = (size_t)ff * d * 2;
  const Span out = span(w_gu, 2 * in_b);
  if (overlap(out, span(w_gate, in_b)) || overlap(out, span(w_up, in_b)))
    return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  hipError_t e = fmlp::launch_pack(static_cast<const uint16_t*>(w_gate),
                                   static_cast<const uint16_t*>(w_up), static_cast<uint16_t*>(w_gu),
                                   ff, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

int fmlp_pack_matrix(const void* w, void* w_tiled, int64_t rows, int64_t K, void* stream) {
  if (!w || !w_tiled) return FMLP_ERR_INVALID_ARG;
  if (!matrix_ok(rows, K)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(w) || !aligned16(w_tiled)) return FMLP_ERR_ALIGNMENT;
  if (overlap(span(w, (size_t)rows * K * 2), span(w_tiled, (size_t)rows * K * 2)))
    return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  hipError_t e = fmlp::launch_tile_matrix(static_cast<const uint16_t*>(w),
                                          static_cast<uint16_t*>(w_tiled), rows, K,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

int fmlp_int4_sizes(int64_t rows, int64_t K, size_t* code_bytes, size_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return FMLP_ERR_INVALID_ARG;
  if (!matrix_ok(rows, K)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  *code_bytes = (size_t)fmlp::int4_code_bytes(rows, K);
  *scale_bytes = (size_t)fmlp::int4_scale_bytes(rows, K);
  return FMLP_OK;
}

int fmlp_quantize_int4(const void* w, int64_t rows, int64_t K, void* q, void* scales,
                       void* stream) {
  if (!w || !q || !scales) return FMLP_ERR_INVALID_ARG;
  if (!rowmajor_ok(rows, K)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(w) || !aligned16(q) || !aligned16(scales)) return FMLP_ERR_ALIGNMENT;
  const Span sw = span(w, (size_t)rows * K * 2), sq = span(q, (size_t)rows * (K / 2)),
             ss = span(scales, (size_t)rows * (K / 32) * 2);
  if (overlap(sw, sq) || overlap(sw, ss) || overlap(sq, ss)) return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  std::lock_guard<std::mutex> lock(g_flag_mutex);
  int range_error = 0;
  hipError_t e = fmlp::launch_quantize(static_cast<const uint16_t*>(w), rows, K,
                                       static_cast<uint8_t*>(q), static_cast<uint16_t*>(scales),
                                       static_cast<hipStream_t>(stream), &range_error);
  if (e != hipSuccess) return hip_fail(e);
  return range_error ? FMLP_ERR_RANGE : FMLP_OK;
}

int fmlp_pack_int4_interleaved(const void* q_gate, const void* s_gate, const void* q_up,
                               const void* s_up, int64_t ff, int64_t d, void* q_gu, void* s_gu,
                               void* stream) {
  if (!q_gate || !s_gate || !q_up || !s_up || !q_gu || !s_gu) return FMLP_ERR_INVALID_ARG;
  if (!shape_ok(d, ff)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(q_gate) || !aligned16(s_gate) || !aligned16(q_up) || !aligned16(s_up) ||
      !aligned16(q_gu) || !aligned16(s_gu))
    return FMLP_ERR_ALIGNMENT;
  const size_t qb = (size_t)ff * (d / 2), sb = (size_t)ff * (d / 32) * 2;
  const Span oq = span(q_gu, (size_t)fmlp::int4_code_bytes(2 * ff, d)),
             os = span(s_gu, (size_t)fmlp::int4_scale_bytes(2 * ff, d));
  const Span in[4] = {span(q_gate, qb), span(s_gate, sb), span(q_up, qb), span(s_up, sb)};
  if (overlap(oq, os)) return FMLP_ERR_INVALID_ARG;
  for (const Span& i : in)
    if (overlap(oq, i) || overlap(os, i)) return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  hipError_t e = fmlp::launch_tile_int4(
      static_cast<const uint8_t*>(q_gate), static_cast<const uint16_t*>(s_gate),
      static_cast<const uint8_t*>(q_up), static_cast<const uint16_t*>(s_up), 2 * ff, d,
      static_cast<uint8_t*>(q_gu), static_cast<uint16_t*>(s_gu), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

int fmlp_pack_int4_matrix(const void* q, const void* scales, int64_t rows, int64_t K,
                          void* q_tiled, void* s_tiled, void* stream) {
  if (!q || !scales || !q_tiled || !s_tiled) return FMLP_ERR_INVALID_ARG;
  if (!matrix_ok(rows, K)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(q) || !aligned16(scales) || !aligned16(q_tiled) || !aligned16(s_tiled))
    return FMLP_ERR_ALIGNMENT;
  const Span iq = span(q, (size_t)rows * (K / 2)), is = span(scales, (size_t)rows * (K / 32) * 2);
  const Span oq = span(q_tiled, (size_t)fmlp::int4_code_bytes(rows, K)),
             os = span(s_tiled, (size_t)fmlp::int4_scale_bytes(rows, K));
  if (overlap(oq, os) || overlap(oq, iq) || overlap(oq, is) || overlap(os, iq) || overlap(os, is))
    return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  hipError_t e = fmlp::launch_tile_int4(static_cast<const uint8_t*>(q),
                                        static_cast<const uint16_t*>(scales), nullptr, nullptr,
                                        rows, K, static_cast<uint8_t*>(q_tiled),
                                        static_cast<uint16_t*>(s_tiled),
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

int fmlp_convert_f16(const void* w, void* out, int64_t n, void* stream) {
  if (!w || !out || n <= 0 || n % 8 != 0) return FMLP_ERR_INVALID_ARG;
  if (n > kMaxConvert) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(w) || !aligned16(out)) return FMLP_ERR_ALIGNMENT;
  if (overlap(span(w, (size_t)n * 2), span(out, (size_t)n * 2))) return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  std::lock_guard<std::mutex> lock(g_flag_mutex);
  int range_error = 0;
  hipError_t e = fmlp::launch_convert_f16(static_cast<const uint16_t*>(w),
                                          static_cast<uint16_t*>(out), n,
                                          static_cast<hipStream_t>(stream), &range_error);
  if (e != hipSuccess) return hip_fail(e);
  return range_error ? FMLP_ERR_RANGE : FMLP_OK;
}

int fmlp_dequant_int4(const void* q, const void* scales, int64_t rows, int64_t K, float* out,
                      void* stream) {
  if (!q || !scales || !out) return FMLP_ERR_INVALID_ARG;
  if (!rowmajor_ok(rows, K)) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(q) || !aligned16(scales) || !aligned16(out)) return FMLP_ERR_ALIGNMENT;
  const Span so = span(out, (size_t)rows * K * 4);
  if (overlap(so, span(q, (size_t)rows * (K / 2))) ||
      overlap(so, span(scales, (size_t)rows * (K / 32) * 2)))
    return FMLP_ERR_INVALID_ARG;
  if (int st = check_device()) return st;
  hipError_t e = fmlp::launch_dequant(static_cast<const uint8_t*>(q),
                                      static_cast<const uint16_t*>(scales), rows, K, out,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

size_t fmlp_workspace_size(int64_t M, int64_t d, int64_t ff, int32_t wtype) {
  if (M < 0 || M > kMaxM || !shape_ok(d, ff) || !wtype_ok(wtype)) return 0;
  // the largest need of the paths the problem may take, each the largest
  // over every smaller M as well (decode and the single pass grow with M;
  // the prefill envelope covers its split-K partials, which do not), so a
  // buffer sized for the largest M serves every call
  size_t b = fmlp::prefill_workspace_envelope(M, d, ff, wtype);
  const int64_t md = M < fmlp::kDecodeMaxM ? M : fmlp::kDecodeMaxM;
  const size_t dec = fmlp::decode_workspace_bytes(md, d, ff);
  b = dec > b ? dec : b;
  if (wtype == FMLP_W_BF16) {
    const size_t one = fmlp::fused_partial_bytes(M < fmlp::kFusedMaxM ? M : fmlp::kFusedMaxM, d, ff);
    b = one > b ? one : b;
  }
  return b + 256;  // room to align the base
}

}  // extern "C"

namespace {

// The scratch of fmlp_forward_noalloc: its workspace, a file-scope device
// array that every GPU the library runs on holds until the process ends (one
// copy per device, each at its own address). Host code reaches its memory
// only through the address hipGetSymbolAddress returns on that device.
constexpr size_t kNoAllocScratchBytes = FMLP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This device's scratch address (looked up once per device, with it current).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

// fmlp_forward_ex, and (noalloc) the same with the device scratch as the
// workspace: then `workspace` is ignored and the problem must fit in it.
int forward_impl(const void* x, const void* residual, void* h_out, const void* gamma, float eps,
                 int32_t activation, int32_t wtype, const void* w_gu, const void* gu_scales,
                 const void* w_down, const void* down_scales, void* y, int64_t M, int64_t d,
                 int64_t ff, void* workspace, size_t workspace_bytes, void* stream, int32_t path,
                 bool noalloc) {
  if (!wtype_ok(wtype)) return FMLP_ERR_INVALID_ARG;
  if (activation != FMLP_ACT_SILU && activation != FMLP_ACT_GELU_TANH &&
      activation != FMLP_ACT_GELU_ERF)
    return FMLP_ERR_INVALID_ARG;
  if ((residual == nullptr) != (h_out == nullptr)) return FMLP_ERR_INVALID_ARG;
  if (path != FMLP_PATH_AUTO && path != FMLP_PATH_DECODE && path != FMLP_PATH_PREFILL &&
      path != FMLP_PATH_SINGLE_PASS)
    return FMLP_ERR_INVALID_ARG;
  if (M < 0) return FMLP_ERR_INVALID_ARG;
  if (!shape_ok(d, ff) || M > kMaxM) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (!std::isfinite(eps) || eps < 0.0f) return FMLP_ERR_INVALID_ARG;
  const bool int4 = wtype == FMLP_W_INT4_G32;
  if (M == 0) return FMLP_OK;
  if (!x || !gamma || !w_gu || !w_down || !y || (!noalloc && !workspace))
    return FMLP_ERR_INVALID_ARG;
  if (int4 && (!gu_scales || !down_scales)) return FMLP_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(w_gu) || !aligned16(w_down) ||
      !aligned16(y) || (!noalloc && !aligned16(workspace)) ||
      (int4 && (!aligned16(gu_scales) || !aligned16(down_scales))) ||
      !aligned16(residual) || !aligned16(h_out))
    return FMLP_ERR_ALIGNMENT;

  const bool single = path == FMLP_PATH_SINGLE_PASS ||
                      (path == FMLP_PATH_AUTO && fmlp::single_pass_auto(M, d, ff, wtype));
  const bool decode = single || path == FMLP_PATH_DECODE ||
                      (path == FMLP_PATH_AUTO && M <= fmlp::kDecodeMaxM);
  if (decode && M > fmlp::kDecodeMaxM) return FMLP_ERR_UNSUPPORTED_SHAPE;
  if (single && (wtype != FMLP_W_BF16 || M > fmlp::kFusedMaxM)) return FMLP_ERR_UNSUPPORTED_SHAPE;

  const size_t need = single   ? fmlp::fused_partial_bytes(M, d, ff)
                      : decode ? fmlp::decode_workspace_bytes(M, d, ff)
                               : fmlp::prefill_workspace_bytes(M, d, ff, wtype);
  if (noalloc) {
    if (need > kNoAllocScratchBytes) return FMLP_ERR_WORKSPACE;
    workspace = nullptr;  // set below, once the device is known
    workspace_bytes = 0;
  }
  // align the workspace base to 256 bytes inside the caller's buffer
  uintptr_t wbase = reinterpret_cast<uintptr_t>(workspace);
  uintptr_t abase = (wbase + 255) & ~uintptr_t(255);
  if (!noalloc && workspace_bytes < need + (abase - wbase)) return FMLP_ERR_WORKSPACE;

  const size_t wgu_b = int4 ? (size_t)fmlp::int4_code_bytes(2 * ff, d) : (size_t)2 * ff * d * 2;
  const size_t wd_b = int4 ? (size_t)fmlp::int4_code_bytes(d, ff) : (size_t)d * ff * 2;
  const Span sy = span(y, (size_t)M * d * 2);
  if (overlap(sy, span(x, (size_t)M * d * 2)) || overlap(sy, span(gamma, (size_t)d * 2)) ||
      overlap(sy, span(w_gu, wgu_b)) || overlap(sy, span(w_down, wd_b)) ||
      overlap(sy, span(workspace, workspace_bytes)))
    return FMLP_ERR_INVALID_ARG;
  if (int4 && (overlap(sy, span(gu_scales, (size_t)fmlp::int4_scale_bytes(2 * ff, d))) ||
               overlap(sy, span(down_scales, (size_t)fmlp::int4_scale_bytes(d, ff)))))
    return FMLP_ERR_INVALID_ARG;
  const Span sw = span(workspace, workspace_bytes);
  if (overlap(sw, span(x, (size_t)M * d * 2)) || overlap(sw, span(gamma, (size_t)d * 2)) ||
      overlap(sw, span(w_gu, wgu_b)) || overlap(sw, span(w_down, wd_b)))
    return FMLP_ERR_INVALID_ARG;
  if (int4 && (overlap(sw, span(gu_scales, (size_t)fmlp::int4_scale_bytes(2 * ff, d))) ||
               overlap(sw, span(down_scales, (size_t)fmlp::int4_scale_bytes(d, ff)))))
    return FMLP_ERR_INVALID_ARG;
  if (residual) {
    // the residual stream is written while x and the residual are still read
    const Span sr = span(residual, (size_t)M * d * 2), sh = span(h_out, (size_t)M * d * 2);
    if (overlap(sh, span(x, (size_t)M * d * 2)) || overlap(sh, sr) ||
        overlap(sh, span(gamma, (size_t)d * 2)) || overlap(sh, span(w_gu, wgu_b)) ||
        overlap(sh, span(w_down, wd_b)) || overlap(sh, sy) || overlap(sh, sw) ||
        overlap(sy, sr) || overlap(sw, sr))
      return FMLP_ERR_INVALID_ARG;
    if (int4 && (overlap(sh, span(gu_scales, (size_t)fmlp::int4_scale_bytes(2 * ff, d))) ||
                 overlap(sh, span(down_scales, (size_t)fmlp::int4_scale_bytes(d, ff)))))
      return FMLP_ERR_INVALID_ARG;
  }

  if (int st = check_device()) return st;
  if (noalloc) {
    void* sp = nullptr;
    if (hipError_t e = scratch_address(&sp)) return hip_fail(e);
    workspace_bytes = kNoAllocScratchBytes;
    wbase = abase = reinterpret_cast<uintptr_t>(sp);
  }

  fmlp::Problem p;
  p.x = static_cast<const uint16_t*>(x);
  p.gamma = static_cast<const uint16_t*>(gamma);
  p.eps = eps;
  p.wtype = wtype;
  p.w_gu = w_gu;
  p.s_gu = static_cast<const uint16_t*>(gu_scales);
  p.w_down = w_down;
  p.s_down = static_cast<const uint16_t*>(down_scales);
  p.y = static_cast<uint16_t*>(y);
  p.M = (int)M;
  p.d = (int)d;
  p.ff = (int)ff;
  p.ws = reinterpret_cast<char*>(abase);
  p.ws_bytes = workspace_bytes - (abase - wbase);
  p.act = activation;
  p.res = static_cast<const uint16_t*>(residual);
  p.hout = static_cast<uint16_t*>(h_out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = single   ? fmlp::launch_decode_fused(p, s)
                 : decode ? fmlp::launch_decode(p, s)
                          : fmlp::launch_prefill(p, s);
  return e == hipSuccess ? FMLP_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int fmlp_forward_ex(const void* x, const void* residual, void* h_out, const void* gamma,
                    float eps, int32_t activation, int32_t wtype, const void* w_gu,
                    const void* gu_scales, const void* w_down, const void* down_scales, void* y,
                    int64_t M, int64_t d, int64_t ff, void* workspace, size_t workspace_bytes,
                    void* stream, int32_t path) {
  return forward_impl(x, residual, h_out, gamma, eps, activation, wtype, w_gu, gu_scales, w_down,
                      down_scales, y, M, d, ff, workspace, workspace_bytes, stream, path, false);
}

int fmlp_forward_noalloc(const void* x, const void* gamma, float eps, int32_t wtype,
                         const void* w_gu, const void* gu_scales, const void* w_down,
                         const void* down_scales, void* y, int64_t M, int64_t d, int64_t ff,
                         void* stream) {
  return forward_impl(x, nullptr, nullptr, gamma, eps, FMLP_ACT_SILU, wtype, w_gu, gu_scales,
                      w_down, down_scales, y, M, d, ff, nullptr, 0, stream, FMLP_PATH_AUTO, true);
}

int fmlp_forward_path(const void* x, const void* gamma, float eps, int32_t wtype,
                      const void* w_gu, const void* gu_scales, const void* w_down,
                      const void* down_scales, void* y, int64_t M, int64_t d, int64_t ff,
                      void* workspace, size_t workspace_bytes, void* stream, int32_t path) {
  return fmlp_forward_ex(x, nullptr, nullptr, gamma, eps, FMLP_ACT_SILU, wtype, w_gu, gu_scales,
                         w_down, down_scales, y, M, d, ff, workspace, workspace_bytes, stream,
                         path);
}

int fmlp_forward(const void* x, const void* gamma, float eps, int32_t wtype, const void* w_gu,
                 const void* gu_scales, const void* w_down, const void* down_scales, void* y,
                 int64_t M, int64_t d, int64_t ff, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return fmlp_forward_path(x, gamma, eps, wtype, w_gu, gu_scales, w_down, down_scales, y, M, d,
                           ff, workspace, workspace_bytes, stream, FMLP_PATH_AUTO);
}

}  // extern "C"
