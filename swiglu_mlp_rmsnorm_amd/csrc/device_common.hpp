// Device helpers shared by the fmlp kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmlp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

// ---- raw 16-byte global loads / stores ------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming (read-once) weight load: nontemporal hint so weights do not evict
// the small reused operands from L2.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---- bf16 / fp16 bit conversions -------------------------------------------

// The two bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua = __builtin_bit_cast(uint16_t, a), ub = __builtin_bit_cast(uint16_t, b);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Split fp32 values into bf16 hi + bf16 lo with hi + lo == v to ~2^-17
// relative (exactly, when v carries at most 16 significant bits, as the
// product of two bf16 values does). Packs pairs (v0, v1).
__device__ __forceinline__ void split_bf16_pair(float v0, float v1, uint32_t& hi,
                                                uint32_t& lo) {
  hi = pack_bf16_rne(v0, v1);
  const float r0 = v0 - bf16_lo(hi);
  const float r1 = v1 - bf16_hi(hi);
  lo = pack_bf16_rne(r0, r1);
}

// bf16 pair -> fp16 pair. Exact for |w| in the fp16 normal range
// [2^-14, 65504]; smaller magnitudes are truncated to fp16 subnormals
// (absolute error < 2^-24).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef __attribute__((ext_vector_type(2))) __fp16 fp16x2_t;
  const fp16x2_t h = __builtin_amdgcn_cvt_pkrtz(bf16_lo(w), bf16_hi(w));
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 h;
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = bf16x2_to_f16x2(v[j]);
  return h;
}

// ---- MFMA wrappers (v_mfma_f32_16x16x32_{bf16,f16}) ------------------------
// Operand layout (wave64): lane l supplies row (l % 16) of A and column
// (l % 16) of B, each as 8 consecutive K-slots of the group (l / 16); the
// accumulator lane l holds D[4*(l/16) + j][l % 16], j = 0..3.

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// sigma(z) = 1 / (1 + e^-z) with the hardware exponential and reciprocal
// (about 1 ulp each; the results are rounded to fp16 or bf16 afterwards).
// Limits: 0 for z -> -inf (e^-z = inf), 1 for z -> +inf.
__device__ __forceinline__ float fast_sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// SiLU(t) * u in fp32, SiLU(t) = t sigma(t). For finite t -> -inf it tends
// to -0 (sigma underflows to 0) without producing NaN.
__device__ __forceinline__ float silu_mul(float t, float u) { return t * fast_sigmoid(t) * u; }

// erf(x) by the rational approximation of Abramowitz and Stegun, Handbook
// of Mathematical Functions, formula 7.1.26: 1 - (a1 k + ... + a5 k^5)
// e^(-x^2) with k = 1 / (1 + p x) for x >= 0, odd in x. Absolute error
// below 1.5e-7 (about 5e-7 evaluated in fp32), far below the fp16 rounding
// of the product it feeds. Branch-free: one hardware reciprocal and one
// exponential, the sigmoid's cost. Limits: +-1 for x -> +-inf, NaN for NaN.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float k = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float q =
      k * (0.254829592f +
           k * (-0.284496736f + k * (1.421413741f + k * (-1.453152027f + k * 1.061405429f))));
  return copysignf(1.0f - q * __expf(-ax * ax), x);
}

// Gate activations (enum fmlp_activation): 0 SiLU; 1 GELU, tanh form
// 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))), evaluated through the
// identity 0.5 (1 + tanh y) = sigma(2 y); 2 GELU, erf form
// 0.5 t (1 + erf(t / sqrt 2)), erf as above. Both GELU forms tend to -0 for
// t -> -inf.
__device__ __forceinline__ float act_mul(int act, float t, float u) {
  if (act == 1)
    return t * fast_sigmoid(1.5957691216057308f * (t + 0.044715f * t * t * t)) * u;
  if (act == 2) return 0.5f * t * (1.0f + erf_as7126(t * 0.7071067811865476f)) * u;
  return silu_mul(t, u);
}

// The residual stream: eight bf16 sums x + r, each rounded to bf16 (nearest
// even). The binary32 sum of two bf16 values rounded to bf16 is the correctly
// rounded sum (24 >= 2*8 + 2 bits, so the double rounding is innocuous).
__device__ __forceinline__ u32x4 add_bf16x8(u32x4 x, u32x4 r) {
  u32x4 h;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    h[j] = pack_bf16_rne(bf16_lo(x[j]) + bf16_lo(r[j]), bf16_hi(x[j]) + bf16_hi(r[j]));
  return h;
}

}  // namespace fmlp
