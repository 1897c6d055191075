// Per-kernel timing with HIP events (see profile.hpp). Host code only.
#include "profile.hpp"

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
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  g_records.clear();
}

}  // namespace

bool profiling_enabled() { return g_on.load(std::memory_order_relaxed); }

bool profile_events(hipEvent_t* start, hipEvent_t* stop) {
  if (hipEventCreate(start) != hipSuccess) return false;
  if (hipEventCreate(stop) != hipSuccess) {
    hipEventDestroy(*start);
    return false;
  }
  return true;
}

void profile_push(int kind, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_records.push_back(Record{kind, start, stop});
}

}  // namespace fmlp

extern "C" {

static const char* const kKernelNames[fmlp::KK_COUNT] = {
    "pack_tile", "quantize_int4", "dequant_int4", "act_prep", "decode_gateup_bf16",
    "decode_down_bf16", "decode_gateup_int4", "decode_down_int4", "rms_scale",
    "gemm_gateup_silu_f16", "gemm_down_f16", "rms_tile_f16", "splitk_reduce",
    "decode_fused_bf16", "partial_reduce"};

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
