// Internal host-side interface between the C ABI (fmlp_api.hip) and the
// kernel translation units. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fmlp {

// One forward problem after argument validation.
struct Problem {
  const uint16_t* x;       // bf16 [M, d]
  const uint16_t* gamma;   // bf16 [d]
  float eps;
  int wtype;               // 0 bf16, 1 int4 group-32, 2 fp16
  const void* w_gu;        // tiled bf16 or fp16 [2ff, d] | tiled int4 codes
  const uint16_t* s_gu;    // tiled fp16 scales (int4)
  const void* w_down;      // tiled bf16 or fp16 [d, ff] | tiled int4 codes
  const uint16_t* s_down;  // tiled fp16 scales (int4)
  uint16_t* y;             // bf16 [M, d]
  int M, d, ff;
  char* ws;                // workspace base (256-byte aligned)
  size_t ws_bytes;
  int act = 0;             // gate activation (enum fmlp_activation)
  const uint16_t* res = nullptr;  // bf16 [M, d] residual input, or null
  uint16_t* hout = nullptr;       // bf16 [M, d] residual stream x + res (when res)
};

constexpr int kDecodeMaxM = 32;
// Largest M of the single-pass decode (bf16 weights): its fp32 partials grow
// as (ff/32) * M * d * 4 bytes.
constexpr int kFusedMaxM = 8;

// Sizes of the tiled int4 format for a logical [R, K] matrix.
inline int64_t int4_code_bytes(int64_t R, int64_t K) { return (R / 16) * ((K + 127) / 128) * 1024; }
inline int64_t int4_scale_bytes(int64_t R, int64_t K) { return (R / 16) * ((K + 127) / 128) * 128; }

// Workspace layout, shared by the sizing query and the launchers.
size_t decode_workspace_bytes(int64_t M, int64_t d, int64_t ff);
size_t fused_partial_bytes(int64_t M, int64_t d, int64_t ff);
size_t prefill_workspace_bytes(int64_t M, int64_t d, int64_t ff, int wtype);
// The largest prefill_workspace_bytes(M', d, ff, wtype) over 1 <= M' <= M.
size_t prefill_workspace_envelope(int64_t M, int64_t d, int64_t ff, int wtype);

hipError_t launch_pack(const uint16_t* w_gate, const uint16_t* w_up, uint16_t* w_gu, int64_t ff,
                       int64_t d, hipStream_t stream);
hipError_t launch_tile_matrix(const uint16_t* w, uint16_t* out, int64_t R, int64_t K,
                              hipStream_t stream);
hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, uint8_t* q,
                           uint16_t* scales, hipStream_t stream, int* range_error);
hipError_t launch_convert_f16(const uint16_t* w, uint16_t* out, int64_t n, hipStream_t stream,
                              int* range_error);
hipError_t launch_dequant(const uint8_t* q, const uint16_t* scales, int64_t rows, int64_t K,
                          float* out, hipStream_t stream);
// Row-major int4 [R, K] (or the row interleave of two [R/2, K] matrices when
// qb is non-null) -> the tiled int4 layout.
hipError_t launch_tile_int4(const uint8_t* qa, const uint16_t* sa, const uint8_t* qb,
                            const uint16_t* sb, int64_t R, int64_t K, uint8_t* qt, uint16_t* st,
                            hipStream_t stream);

hipError_t launch_decode(const Problem& p, hipStream_t stream);
hipError_t launch_decode_fused(const Problem& p, hipStream_t stream);
// Whether FMLP_PATH_AUTO takes the single-pass decode for this problem.
bool single_pass_auto(int64_t M, int64_t d, int64_t ff, int wtype);
hipError_t launch_prefill(const Problem& p, hipStream_t stream);

}  // namespace fmlp
