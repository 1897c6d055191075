// Measurement support: per-kernel timing with HIP events (see profile.hpp),
// and a plain streaming-read probe that gives the HBM read rate a kernel can
// reach for a given number of bytes per launch.
#include "profile.hpp"

#include "device_common.hpp"

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/fmlp.h"

namespace fmlp {
namespace {

struct Record {
  int kind;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;

void clear_locked() {
  for (Record& r : g_records) {
    (void)hipEventDestroy(r.start);  // best-effort cleanup
    (void)hipEventDestroy(r.stop);
  }
  g_records.clear();
}

}  // namespace

bool profiling_enabled() { return g_on.load(std::memory_order_relaxed); }

bool profile_events(hipEvent_t* start, hipEvent_t* stop) {
  if (hipEventCreate(start) != hipSuccess) return false;
  if (hipEventCreate(stop) != hipSuccess) {
    (void)hipEventDestroy(*start);
    return false;
  }
  return true;
}

void profile_push(int kind, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_records.push_back(Record{kind, start, stop});
}

// Every thread reads 16-byte chunks of src in a grid-stride loop (four
// chunks in flight, nontemporal like the weight streams) and stores the XOR
// of what it read to sink[thread], so that no read can be dropped.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4* __restrict__ src, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 e = __builtin_nontemporal_load(src + i + 3 * stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= a[j] ^ b[j] ^ c[j] ^ e[j];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= a[j];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace fmlp

extern "C" {

int fmlp_read_probe(const void* src, int64_t bytes, void* sink, int32_t workgroups,
                    void* stream) {
  if (!src || !sink || bytes <= 0 || workgroups < 1 || workgroups > 65536)
    return FMLP_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u) ||
      (bytes & 15))
    return FMLP_ERR_ALIGNMENT;
  fmlp::launch_kernel(fmlp::KK_READ_PROBE, fmlp::k_read_probe, dim3(workgroups), dim3(256), 0,
                      static_cast<hipStream_t>(stream),
                      static_cast<const fmlp::u32x4*>(src), bytes / 16,
                      static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? FMLP_OK : FMLP_ERR_HIP;
}

static const char* const kKernelNames[fmlp::KK_COUNT] = {
    "pack_tile", "quantize_int4", "dequant_int4", "act_prep", "decode_gateup_bf16",
    "decode_down_bf16", "decode_gateup_int4", "decode_down_int4",
    "gemm_gateup_silu_f16", "gemm_down_f16", "rms_norm_f16", "splitk_reduce",
    "decode_fused_bf16", "read_probe", "convert_f16"};

int fmlp_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(fmlp::g_mu);
  fmlp::clear_locked();
  fmlp::g_on.store(on != 0, std::memory_order_relaxed);
  return FMLP_OK;
}

int fmlp_profile_read(int32_t kind, int64_t* launches, double* total_ms) {
  if (kind < 0 || kind >= fmlp::KK_COUNT || !launches || !total_ms) return FMLP_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(fmlp::g_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (const fmlp::Record& r : fmlp::g_records) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return FMLP_ERR_HIP;
    float e = 0.f;
    if (hipEventElapsedTime(&e, r.start, r.stop) != hipSuccess) return FMLP_ERR_HIP;
    ms += e;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return FMLP_OK;
}

const char* fmlp_kernel_name(int32_t kind) {
  return (kind >= 0 && kind < fmlp::KK_COUNT) ? kKernelNames[kind] : nullptr;
}

}  // extern "C"
