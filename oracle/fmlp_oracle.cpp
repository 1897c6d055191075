// CPU oracle for the fused gated (SwiGLU) MLP with an RMSNorm prologue.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
// load or call this file; only the test suite, the smoke check and the
// benchmark's CPU-baseline leg use it. It shares no code, header, table or
// helper with the HIP library: every conversion below is written out here.
//
// What it computes (all arithmetic in IEEE double unless stated):
//   FastTPS review (xllm-io paper-review blog), section 3 "technical
//   architecture", Eq(1): O = W_down( SiLU(W_gate h) * (W_up h) ), where '*'
//   is the element-wise product ("elewMul"), and the MLP-block flow on the
//   same page: RMSNorm -> interleaved gate-up matmul -> SiLU*mul -> down
//   projection (Figure 4: part1 RMSNorm, part2 interleaved gate/up fusion,
//   part3 down projection). So h = RMSNorm(x).
//   Readings where the pages are silent:
//     RMSNorm(x)_k = gamma_k * x_k / sqrt(mean_k(x^2) + eps)   (no mean
//       subtraction, no bias, gamma is a plain multiplier);
//     SiLU(t) = t / (1 + exp(-t))  (Swish with beta = 1; SwiGLU);
//     interleave: packed row 2i is gate row i, packed row 2i+1 is up row i
//       (llama.cpp PR digest, blog.cecily.jp: gate/up rows alternate);
//     weights are nn.Linear-shaped [out, in], row-major;
//     int4: symmetric, groups of 32 consecutive elements along K, one fp16
//       scale per group, s = fp16_rne(fp32(max|w| / 7)),
//       q = clamp(round_half_even(fp32(w / s)), -8, 7), q = 0 when s == 0,
//       two's-complement nibbles, even k in the low nibble.
//
//   Variants beyond Eq(1) (also readings):
//     activation of the gate branch: SiLU (Eq(1)), or GELU, the activation the
//       Together AI fusion post (blog.hotdry.top) names for its fused MLP;
//       the pages give no GELU formula, so both usual forms are offered:
//       erf form t * Phi(t) = 0.5 t (1 + erf(t / sqrt 2)), and tanh form
//       0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3)));
//     fp16 weight storage: a bf16 weight becomes the fp16 value of largest
//       magnitude not above its own, with its sign (truncation toward zero).
//       Every bf16 value in the fp16 normal range [2^-14, 65504] is exact in
//       fp16 (8 significant bits of 11); only the subnormal range rounds, and
//       non-finite values or magnitudes above 65504 are range errors. The
//       forward then reads those fp16 values as the weights;
//     residual prologue: with a residual input r (the previous sublayer's
//       output), the residual stream h = bf16_rne(x + r) is formed, written
//       out, and normalised in place of x (the residual add fused with the
//       following RMSNorm; same post, where the add/all-reduce is fused into
//       the next normalisation).
//
// Summation order is fixed (k ascending), and OpenMP only splits independent
// outputs, so results do not depend on the thread count.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cfenv>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

// ---------------------------------------------------------------- scalars

// bf16 -> double: a bf16 is the top 16 bits of an IEEE binary32.
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return (double)f;
}

// IEEE binary16 -> double, decoded field by field (exact).
static double f16_value(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = std::ldexp((double)m, -24);              // zero / subnormal
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = std::ldexp((double)(m | 0x400), e - 25);  // 1.m * 2^(e-15)
  return sign ? -v : v;
}

// binary32 -> binary16 with round-to-nearest-even, written from the format
// definition: scale the magnitude so the kept bits are the integer part,
// round that integer half-to-even, rebuild the fields.
static uint16_t f16_bits_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (std::isnan(f)) return (uint16_t)(sign | 0x7e00u);
  const double a = std::fabs((double)f);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);  // rounds past 65504
  const int old_mode = std::fegetround();
  std::fesetround(FE_TONEAREST);
  uint16_t bits;
  if (a < std::ldexp(1.0, -14)) {
    // subnormal range: unit is 2^-24; rounding up may reach 0x400 (min normal)
    bits = (uint16_t)std::nearbyint(std::ldexp(a, 24));
  } else {
    int e2;
    std::frexp(a, &e2);            // a = f * 2^e2, f in [0.5, 1)
    const int e = e2 - 1;          // a in [2^e, 2^(e+1))
    double mant = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
    int ee = e;
    if (mant >= 2048.0) { mant = 1024.0; ee += 1; }
    bits = (uint16_t)(((ee + 15) << 10) | ((int)mant - 1024));
  }
  std::fesetround(old_mode);
  return (uint16_t)(sign | bits);
}

// double -> bf16 with round-to-nearest-even, written from the format
// definition (8 significant bits, exponent range of binary32): scale the
// magnitude so the kept bits are the integer part, round that integer
// half-to-even, scale back; the rounded value is exact in binary32, whose
// top 16 bits are the bf16 pattern.
static uint16_t bf16_bits_rne(double v) {
  if (std::isnan(v)) return std::signbit(v) ? 0xffc0u : 0x7fc0u;
  const double a = std::fabs(v);
  const int old_mode = std::fegetround();
  std::fesetround(FE_TONEAREST);
  double r;
  if (a < std::ldexp(1.0, -126)) {
    r = std::ldexp(std::nearbyint(std::ldexp(a, 133)), -133);  // subnormal unit 2^-133
  } else {
    int e2;
    std::frexp(a, &e2);                                   // a in [2^(e2-1), 2^e2)
    r = std::ldexp(std::nearbyint(std::ldexp(a, 8 - e2)), e2 - 8);  // 8 significant bits
  }
  std::fesetround(old_mode);
  const float f = (float)(std::signbit(v) ? -r : r);      // exact, or +-inf past the range
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

double oracle_bf16_to_double(uint16_t b) { return bf16_value(b); }
uint16_t oracle_bf16_rne(double v) { return bf16_bits_rne(v); }
double oracle_f16_to_double(uint16_t h) { return f16_value(h); }
uint16_t oracle_f32_to_f16_rne(float f) { return f16_bits_rne(f); }

// SiLU(t) = t * sigmoid(t) = t / (1 + e^-t). For t -> -inf, e^-t overflows to
// +inf and the quotient is -0, the correct limit.
double oracle_silu(double t) { return t / (1.0 + std::exp(-t)); }

// GELU, erf form: t * Phi(t), Phi the standard normal distribution function.
double oracle_gelu_erf(double t) { return 0.5 * t * (1.0 + std::erf(t / std::sqrt(2.0))); }

// GELU, tanh form: Phi(t) approximated by 0.5 (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))).
double oracle_gelu_tanh(double t) {
  const double c = std::sqrt(2.0 / std::acos(-1.0));
  return 0.5 * t * (1.0 + std::tanh(c * (t + 0.044715 * t * t * t)));
}

// Gate activation by code: 0 SiLU, 1 GELU (tanh form), 2 GELU (erf form).
static double gate_act(int act, double t) {
  if (act == 1) return oracle_gelu_tanh(t);
  if (act == 2) return oracle_gelu_erf(t);
  return oracle_silu(t);
}

// h[i] = bf16_rne(x[i] + r[i]) over n elements (bit patterns); the sum of
// two bf16 values is exact in double.
void oracle_residual_add(const uint16_t* x, const uint16_t* r, int64_t n, uint16_t* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = bf16_bits_rne(bf16_value(x[i]) + bf16_value(r[i]));
}

// ---------------------------------------------------------------- RMSNorm

// r[m] = 1 / sqrt(mean_k x[m,k]^2 + eps)
void oracle_rms_scale(const uint16_t* x, int64_t M, int64_t d, double eps,
                      double* r) {
  for (int64_t m = 0; m < M; ++m) {
    double ss = 0.0;
    for (int64_t k = 0; k < d; ++k) {
      const double v = bf16_value(x[m * d + k]);
      ss += v * v;
    }
    r[m] = 1.0 / std::sqrt(ss / (double)d + eps);
  }
}

// n[m,k] = x[m,k] * r[m] * gamma[k]
void oracle_rmsnorm(const uint16_t* x, const uint16_t* gamma, double eps,
                    int64_t M, int64_t d, double* n) {
  for (int64_t m = 0; m < M; ++m) {
    double r;
    oracle_rms_scale(x + m * d, 1, d, eps, &r);
    for (int64_t k = 0; k < d; ++k)
      n[m * d + k] = bf16_value(x[m * d + k]) * r * bf16_value(gamma[k]);
  }
}

// ---------------------------------------------------------------- packing

// w_gu[2i, :] = w_gate[i, :], w_gu[2i+1, :] = w_up[i, :]   (bf16 bit copies)
void oracle_pack_interleaved(const uint16_t* w_gate, const uint16_t* w_up,
                             uint16_t* w_gu, int64_t ff, int64_t d) {
  for (int64_t i = 0; i < ff; ++i) {
    for (int64_t k = 0; k < d; ++k) {
      w_gu[(2 * i) * d + k] = w_gate[i * d + k];
      w_gu[(2 * i + 1) * d + k] = w_up[i * d + k];
    }
  }
}

// ---------------------------------------------------------------- tiled layouts
// The library stores weights fragment-tiled (a storage permutation only; the
// logical matrices are unchanged). For a logical bf16 matrix W [R, K]
// (R % 16 == 0, K % 32 == 0), element (r, k) sits at
//   ((r/16)*(K/32) + k/32)*512 + (((k%32)/8)*16 + r%16)*8 + k%8.
static int64_t tiled_bf16_index(int64_t r, int64_t k, int64_t K) {
  return ((r / 16) * (K / 32) + k / 32) * 512 + (((k % 32) / 8) * 16 + r % 16) * 8 + k % 8;
}

void oracle_tile_bf16(const uint16_t* w, int64_t R, int64_t K, uint16_t* out) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) out[tiled_bf16_index(r, k, K)] = w[r * K + k];
}

void oracle_untile_bf16(const uint16_t* t, int64_t R, int64_t K, uint16_t* w) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) w[r * K + k] = t[tiled_bf16_index(r, k, K)];
}

// Tiled int4: groups of 32 along K are taken four at a time ("super-tiles",
// nq = ceil(K/128) per 16-row block, 1024 bytes each). Code (r, k) with group
// g = k/32 lives in super-tile ((r/16)*nq + g/4), 16-byte lane slot
// L = ((k%32)/8)*16 + r%16, 32-bit word g%4 of that slot, nibble k%8 (bits
// 4*(k%8)). Scale (r, g) is fp16 element ((r/16)*nq + g/4)*64 + (r%16)*4 + g%4.
// Groups past K/32 in the last super-tile hold zero codes and zero scales.
int64_t oracle_int4_tiled_code_bytes(int64_t R, int64_t K) { return (R / 16) * ((K + 127) / 128) * 1024; }
int64_t oracle_int4_tiled_scale_count(int64_t R, int64_t K) { return (R / 16) * ((K + 127) / 128) * 64; }

static void int4_tiled_pos(int64_t r, int64_t k, int64_t K, int64_t* byte, int* shift) {
  const int64_t nq = (K + 127) / 128, g = k / 32;
  const int64_t lane = ((k % 32) / 8) * 16 + r % 16;
  const int64_t word = ((r / 16) * nq + g / 4) * 256 + lane * 4 + g % 4;
  const int nib = (int)(k % 8);
  *byte = word * 4 + nib / 2;
  *shift = (nib % 2) * 4;
}
static int64_t int4_tiled_scale_index(int64_t r, int64_t g, int64_t K) {
  const int64_t nq = (K + 127) / 128;
  return ((r / 16) * nq + g / 4) * 64 + (r % 16) * 4 + g % 4;
}

// row-major (q [R, K/2] even k low nibble, s [R, K/32]) -> tiled
void oracle_tile_int4(const uint8_t* q, const uint16_t* s, int64_t R, int64_t K, uint8_t* qt,
                      uint16_t* st) {
  std::memset(qt, 0, (size_t)oracle_int4_tiled_code_bytes(R, K));
  std::memset(st, 0, (size_t)oracle_int4_tiled_scale_count(R, K) * 2);
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = q[r * (K / 2) + k / 2];
      const int nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
      int64_t b;
      int sh;
      int4_tiled_pos(r, k, K, &b, &sh);
      qt[b] = (uint8_t)(qt[b] | (nib << sh));
    }
    for (int64_t g = 0; g < K / 32; ++g) st[int4_tiled_scale_index(r, g, K)] = s[r * (K / 32) + g];
  }
}

// tiled -> row-major
void oracle_untile_int4(const uint8_t* qt, const uint16_t* st, int64_t R, int64_t K, uint8_t* q,
                        uint16_t* s) {
  std::memset(q, 0, (size_t)(R * (K / 2)));
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      int64_t b;
      int sh;
      int4_tiled_pos(r, k, K, &b, &sh);
      const int nib = (qt[b] >> sh) & 0xF;
      q[r * (K / 2) + k / 2] = (uint8_t)(q[r * (K / 2) + k / 2] | ((k & 1) ? nib << 4 : nib));
    }
    for (int64_t g = 0; g < K / 32; ++g) s[r * (K / 32) + g] = st[int4_tiled_scale_index(r, g, K)];
  }
}

// ---------------------------------------------------------------- int4

// Returns 0, or -5 when a group's scale is not a finite fp16 (a non-finite
// weight, or max|w|/7 rounding past 65504).
int oracle_quantize_int4(const uint16_t* w, int64_t rows, int64_t K,
                         uint8_t* q, uint16_t* scales) {
  const int old_mode = std::fegetround();
  std::fesetround(FE_TONEAREST);
  int status = 0;
  const int64_t groups = K / 32;
  for (int64_t r = 0; r < rows && status == 0; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const uint16_t* src = w + r * K + g * 32;
      float mx = 0.0f;
      bool finite = true;
      for (int j = 0; j < 32; ++j) {
        const float v = (float)bf16_value(src[j]);
        if (!std::isfinite(v)) finite = false;
        const float a = std::fabs(v);
        if (a > mx) mx = a;
      }
      const float ratio = mx / 7.0f;          // IEEE binary32 division
      const uint16_t sh = f16_bits_rne(ratio);
      if (!finite || (sh & 0x7c00u) == 0x7c00u) { status = -5; break; }
      scales[r * groups + g] = sh;
      const float s = (float)f16_value(sh);
      for (int j = 0; j < 32; j += 2) {
        int qq[2];
        for (int t = 0; t < 2; ++t) {
          int v = 0;
          if (s != 0.0f) {
            const float ratio_k = (float)bf16_value(src[j + t]) / s;
            float rq = std::nearbyint(ratio_k);  // ties to even
            if (rq > 7.0f) rq = 7.0f;
            if (rq < -8.0f) rq = -8.0f;
            v = (int)rq;
          }
          qq[t] = v;
        }
        q[r * (K / 2) + (g * 32 + j) / 2] =
            (uint8_t)((qq[0] & 0xF) | ((qq[1] & 0xF) << 4));
      }
    }
  }
  std::fesetround(old_mode);
  return status;
}

// Signed value of nibble k of a packed int4 row.
static int int4_at(const uint8_t* qrow, int64_t k) {
  const uint8_t byte = qrow[k / 2];
  const int nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
  return nib >= 8 ? nib - 16 : nib;
}

// out[r,k] = float(s[r, k/32]) * float(q[r,k]); exact in binary32
// (an 11-bit significand times a 4-bit integer).
void oracle_dequant_int4(const uint8_t* q, const uint16_t* scales,
                         int64_t rows, int64_t K, float* out) {
  const int64_t groups = K / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = (float)f16_value(scales[r * groups + k / 32]) *
                       (float)int4_at(q + r * (K / 2), k);
}

// bf16 -> fp16 by truncation toward zero, over n elements (bit patterns),
// written from the binary16 format: the magnitude in units of the fp16 spacing
// at its binade (2^-24 below 2^-14), rounded down, fields rebuilt, sign kept.
// Returns how many elements are not finite or exceed 65504 in magnitude;
// their outputs are set to 0.
int64_t oracle_bf16_to_f16_trunc(const uint16_t* w, int64_t n, uint16_t* out) {
  int64_t bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    const double v = bf16_value(w[i]);
    const double a = std::fabs(v);
    if (!std::isfinite(v) || a > 65504.0) {
      ++bad;
      out[i] = 0;
      continue;
    }
    uint16_t bits;
    if (a < std::ldexp(1.0, -14)) {
      bits = (uint16_t)std::floor(std::ldexp(a, 24));  // subnormal: unit 2^-24
    } else {
      int e2;
      std::frexp(a, &e2);                                        // a in [2^(e2-1), 2^e2)
      const double mant = std::floor(std::ldexp(a, 11 - e2));  // in [1024, 2047]
      bits = (uint16_t)(((e2 - 1 + 15) << 10) | ((int)mant - 1024));
    }
    out[i] = (uint16_t)((w[i] & 0x8000u) | bits);
  }
  return bad;
}

// ---------------------------------------------------------------- forward

// Weight access: one callback-free struct per storage kind keeps the three
// forward variants on the same arithmetic.
// Every binary16 pattern's value, decoded once by f16_value (a cache of that
// function: the forward reads the same doubles it would compute).
static const double* f16_table() {
  static double* t = [] {
    double* v = new double[65536];
    for (uint32_t h = 0; h < 65536; ++h) v[h] = f16_value((uint16_t)h);
    return v;
  }();
  return t;
}

struct WeightView {
  int kind;                 // 0 bf16, 1 int4 group-32, 2 fp16
  const uint16_t* bf;       // bf16 (kind 0) or fp16 (kind 2) [rows, K]
  const uint8_t* q;         // int4 [rows, K/2]
  const uint16_t* s;        // fp16 [rows, K/32]
  int64_t K;
  const double* f16 = f16_table();
  double at(int64_t row, int64_t k) const {
    if (kind == 0) return bf16_value(bf[row * K + k]);
    if (kind == 2) return f16[bf[row * K + k]];
    return f16[s[row * (K / 32) + k / 32]] * (double)int4_at(q + row * (K / 2), k);
  }
};

// y[m, :] = Wd (act(Wg n_m) * (Wu n_m)), n_m = RMSNorm(h_m), with h = x, or
// h = bf16_rne(x + res) when res is given (then also written to h_out when
// that is given). gate row i is (g_view, g_row0 + g_stride*i), up row i
// likewise.
//
// Every output is one sum over k ascending. Tokens are taken kTokenChunk at a
// time; within a chunk the loops run over weight rows outermost, so each row's
// values are read once per chunk and used for each of its tokens. The sum of
// each (token, output) pair is the same sequence of operations whatever the
// loop order or the thread that runs it.
static void forward_core(const uint16_t* x, const uint16_t* res, uint16_t* h_out,
                         const uint16_t* gamma, double eps, int act,
                         const WeightView& gv, int64_t g_row0, int64_t g_stride,
                         const WeightView& uv, int64_t u_row0, int64_t u_stride,
                         const WeightView& dv, int64_t M, int64_t d, int64_t ff,
                         double* y) {
  constexpr int64_t kTokenChunk = 16;
  std::vector<double> n((size_t)(kTokenChunk * d));
  std::vector<double> a((size_t)(kTokenChunk * ff));
  std::vector<uint16_t> h((size_t)d);
  for (int64_t m0 = 0; m0 < M; m0 += kTokenChunk) {
    const int64_t mc = M - m0 < kTokenChunk ? M - m0 : kTokenChunk;
    for (int64_t m = 0; m < mc; ++m) {
      const uint16_t* xm = x + (m0 + m) * d;
      if (res) {
        oracle_residual_add(xm, res + (m0 + m) * d, d, h.data());
        if (h_out) std::memcpy(h_out + (m0 + m) * d, h.data(), (size_t)d * sizeof(uint16_t));
        xm = h.data();
      }
      oracle_rmsnorm(xm, gamma, eps, 1, d, n.data() + m * d);
    }
#pragma omp parallel
    {
      std::vector<double> wg((size_t)d), wu((size_t)d);
#pragma omp for schedule(static)
      for (int64_t i = 0; i < ff; ++i) {
        const int64_t gr = g_row0 + g_stride * i, ur = u_row0 + u_stride * i;
        for (int64_t k = 0; k < d; ++k) wg[k] = gv.at(gr, k);
        for (int64_t k = 0; k < d; ++k) wu[k] = uv.at(ur, k);
        for (int64_t m = 0; m < mc; ++m) {
          const double* nm = n.data() + m * d;
          double g = 0.0, u = 0.0;
          for (int64_t k = 0; k < d; ++k) {
            g += wg[k] * nm[k];
            u += wu[k] * nm[k];
          }
          a[m * ff + i] = gate_act(act, g) * u;
        }
      }
    }
#pragma omp parallel
    {
      std::vector<double> wd((size_t)ff);
#pragma omp for schedule(static)
      for (int64_t j = 0; j < d; ++j) {
        for (int64_t i = 0; i < ff; ++i) wd[i] = dv.at(j, i);
        for (int64_t m = 0; m < mc; ++m) {
          const double* am = a.data() + m * ff;
          double acc = 0.0;
          for (int64_t i = 0; i < ff; ++i) acc += wd[i] * am[i];
          y[(m0 + m) * d + j] = acc;
        }
      }
    }
  }
}

// Eq(1) from separate gate and up matrices (the unfused ordering), with the
// activation `act` and the optional residual prologue (res, h_out nullable).
void oracle_forward_unfused_ex(const uint16_t* x, const uint16_t* res, uint16_t* h_out,
                               const uint16_t* gamma, double eps, int act,
                               const uint16_t* w_gate, const uint16_t* w_up,
                               const uint16_t* w_down, int64_t M, int64_t d, int64_t ff,
                               double* y) {
  WeightView g{0, w_gate, nullptr, nullptr, d};
  WeightView u{0, w_up, nullptr, nullptr, d};
  WeightView dn{0, w_down, nullptr, nullptr, ff};
  forward_core(x, res, h_out, gamma, eps, act, g, 0, 1, u, 0, 1, dn, M, d, ff, y);
}

void oracle_forward_unfused(const uint16_t* x, const uint16_t* gamma,
                            double eps, const uint16_t* w_gate,
                            const uint16_t* w_up, const uint16_t* w_down,
                            int64_t M, int64_t d, int64_t ff, double* y) {
  oracle_forward_unfused_ex(x, nullptr, nullptr, gamma, eps, 0, w_gate, w_up, w_down, M, d, ff,
                            y);
}

// Eq(1) from the interleaved matrix w_gu [2ff, d] (gate at even rows).
void oracle_forward_bf16(const uint16_t* x, const uint16_t* gamma, double eps,
                         const uint16_t* w_gu, const uint16_t* w_down,
                         int64_t M, int64_t d, int64_t ff, double* y) {
  WeightView gu{0, w_gu, nullptr, nullptr, d};
  WeightView dn{0, w_down, nullptr, nullptr, ff};
  forward_core(x, nullptr, nullptr, gamma, eps, 0, gu, 0, 2, gu, 1, 2, dn, M, d, ff, y);
}

// Eq(1) with int4 weights: w = s * q, widened exactly to double; activation
// and residual prologue as in oracle_forward_unfused_ex.
void oracle_forward_int4_ex(const uint16_t* x, const uint16_t* res, uint16_t* h_out,
                            const uint16_t* gamma, double eps, int act, const uint8_t* q_gu,
                            const uint16_t* s_gu, const uint8_t* q_down,
                            const uint16_t* s_down, int64_t M, int64_t d, int64_t ff,
                            double* y) {
  WeightView gu{1, nullptr, q_gu, s_gu, d};
  WeightView dn{1, nullptr, q_down, s_down, ff};
  forward_core(x, res, h_out, gamma, eps, act, gu, 0, 2, gu, 1, 2, dn, M, d, ff, y);
}

void oracle_forward_int4(const uint16_t* x, const uint16_t* gamma, double eps,
                         const uint8_t* q_gu, const uint16_t* s_gu,
                         const uint8_t* q_down, const uint16_t* s_down,
                         int64_t M, int64_t d, int64_t ff, double* y) {
  oracle_forward_int4_ex(x, nullptr, nullptr, gamma, eps, 0, q_gu, s_gu, q_down, s_down, M, d,
                         ff, y);
}

// Eq(1) with fp16 weights: the interleaved w_gu [2ff, d] and w_down [d, ff]
// hold fp16 values (oracle_bf16_to_f16_trunc of the bf16 matrices), widened
// exactly to double; activation and residual prologue as in
// oracle_forward_unfused_ex.
void oracle_forward_f16_ex(const uint16_t* x, const uint16_t* res, uint16_t* h_out,
                           const uint16_t* gamma, double eps, int act, const uint16_t* w_gu,
                           const uint16_t* w_down, int64_t M, int64_t d, int64_t ff, double* y) {
  WeightView gu{2, w_gu, nullptr, nullptr, d};
  WeightView dn{2, w_down, nullptr, nullptr, ff};
  forward_core(x, res, h_out, gamma, eps, act, gu, 0, 2, gu, 1, 2, dn, M, d, ff, y);
}

// Threads the parallel loops above will use.
int oracle_omp_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// Set that thread count (results do not depend on it).
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

}  // extern "C"
