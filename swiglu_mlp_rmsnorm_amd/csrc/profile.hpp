// Optional per-kernel timing: while enabled (fmlp_profile_enable), every
// kernel launch is bracketed by HIP events recorded on its own stream.
#pragma once

#include <hip/hip_runtime.h>

namespace fmlp {

enum KernelKind {
  KK_PACK = 0,
  KK_QUANTIZE,
  KK_DEQUANT,
  KK_ACT_PREP,
  KK_DECODE_GATEUP_BF16,
  KK_DECODE_DOWN_BF16,
  KK_DECODE_GATEUP_INT4,
  KK_DECODE_DOWN_INT4,
  KK_RMS_PREP,
  KK_GEMM_GATEUP,
  KK_GEMM_DOWN,
  KK_COUNT
};

bool profiling_enabled();
void profile_record(int kind, hipStream_t stream, bool start);

// RAII bracket around one launch; costs one relaxed atomic load when disabled.
struct ProfileScope {
  int kind;
  hipStream_t stream;
  bool on;
  ProfileScope(int k, hipStream_t s) : kind(k), stream(s), on(profiling_enabled()) {
    if (on) profile_record(kind, stream, true);
  }
  ~ProfileScope() {
    if (on) profile_record(kind, stream, false);
  }
};

}  // namespace fmlp
