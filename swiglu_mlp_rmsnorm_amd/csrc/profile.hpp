// Optional per-kernel timing: while enabled (fmlp_profile_enable), every
// kernel is launched with hipExtLaunchKernelGGL and a start/stop event pair,
// which the runtime timestamps at the dispatch's own begin and end on the
// launch stream (so the figure is the kernel's execution time, the same
// quantity a kernel trace reports, without the gap between launches).
#pragma once

#include <hip/hip_ext.h>
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
  KK_GEMM_GATEUP,
  KK_GEMM_DOWN,
  KK_RMS_NORM,
  KK_SPLITK_REDUCE,
  KK_DECODE_FUSED_BF16,
  KK_READ_PROBE,
  KK_CONVERT_F16,
  KK_COUNT
};

bool profiling_enabled();
// Two fresh timing events, or false (then the launch goes untimed).
bool profile_events(hipEvent_t* start, hipEvent_t* stop);
void profile_push(int kind, hipEvent_t start, hipEvent_t stop);

// Launch `kernel`; timed under `kind` while profiling is enabled. Costs one
// relaxed atomic load when it is not. Launch errors are left for the caller's
// hipGetLastError().
template <typename... Params, typename... Args>
inline void launch_kernel(int kind, void (*kernel)(Params...), dim3 grid, dim3 block,
                          uint32_t shmem, hipStream_t stream, Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  if (profiling_enabled() && profile_events(&start, &stop)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, stop, 0, args...);
    profile_push(kind, start, stop);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  }
}

}  // namespace fmlp
