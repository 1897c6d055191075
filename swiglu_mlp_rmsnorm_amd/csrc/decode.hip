// Decode path (M <= 32 tokens): two weight-streaming kernels.
//
//   1. gate/up: z = W_gu v (v = gamma * x, unnormalised), the RMS scale r of
//      each token folded in afterwards (z * r = W_gu (gamma * x * r)), then
//      a = SiLU(z_gate) * z_up on the interleaved row pairs, in registers
//      (FastTPS review section 3: RMSNorm -> interleaved gate-up matmul ->
//      SiLU*mul; llama.cpp PR digest: GLU applied in the same matmul pass).
//   2. down: y = W_down a.
//
// Both are bound by HBM reads of the weights (decode arithmetic intensity is
// ~M flop/byte, far under the bf16 ridge of ~315 flop/byte), so the design
// goal is to keep enough 16-byte loads in flight and spend little VALU time.
// The dot products run on MFMA 16x16x32 bf16: weights are the A operand
// (16 rows per block, loaded straight from HBM into registers in the MFMA
// lane layout), tokens are the B operand (16 columns, zero-padded above M).
// The B operand carries the activation as an exact bf16 hi + lo split, so the
// contraction has fp32-equivalent precision in the activation (the product
// of two bf16 values has 16 significant bits, which hi + lo hold exactly).
// K is split across the waves of a workgroup and reduced through LDS in a
// fixed order: results are deterministic.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace fmlp {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(int64_t M, int64_t d, int64_t ff) {
  (void)d;
  // a_hi, a_lo: bf16 [M, ff] each
  return 2 * align256((size_t)M * (size_t)ff * 2);
}

// ---------------------------------------------------------------------------
// gate/up + RMSNorm + SiLU*mul.
// Workgroup: S waves, RB row blocks of 16 W_gu rows (RB*8 gate/up pairs).
// Wave w handles K32 blocks w, w+S, w+2S, ... of all RB row blocks, so the S
// waves of a workgroup together read contiguous spans of each row.
// Output: a = a_hi + a_lo (bf16 pair, fp32-equivalent), [M, ff].
template <int NCB, int RB, int S>
__global__ __launch_bounds__(64 * S) void k_decode_gateup_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, float eps,
    const uint16_t* __restrict__ wgu, uint16_t* __restrict__ a_hi, uint16_t* __restrict__ a_lo,
    int M, int d, int ff) {
  __shared__ f32x4 red[S * RB * NCB * 64];
  __shared__ float ssred[S * NCB * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (RB * 16);
  const int nkb = d >> 5;

  const uint16_t* wrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) wrow[rb] = wgu + (row0 + rb * 16 + col) * (int64_t)d + grp * 8;
  const uint16_t* xrow[NCB];
  bool tok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int t = cb * 16 + col;
    tok[cb] = t < M;
    xrow[cb] = x + (int64_t)(tok[cb] ? t : 0) * d + grp * 8;
  }
  const uint16_t* grow = gamma + grp * 8;

  f32x4 acc[RB][NCB];
  float ss[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    ss[cb] = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int kb = wave;
  u32x4 wn[RB];
  if (kb < nkb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) wn[rb] = ld16_stream(wrow[rb] + kb * 32);
  }
  for (; kb < nkb; kb += S) {
    u32x4 w[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) w[rb] = wn[rb];
    if (kb + S < nkb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wn[rb] = ld16_stream(wrow[rb] + (kb + S) * 32);
    }
    const int k = kb * 32;
    const u32x4 gv = ld16(grow + k);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      u32x4 xv = {0u, 0u, 0u, 0u};
      if (tok[cb]) xv = ld16(xrow[cb] + k);
      u32x4 hi, lo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = bf16_lo(xv[j]), x1 = bf16_hi(xv[j]);
        ss[cb] = fmaf(x0, x0, ss[cb]);
        ss[cb] = fmaf(x1, x1, ss[cb]);
        uint32_t h, l;
        split_bf16_pair(x0 * bf16_lo(gv[j]), x1 * bf16_hi(gv[j]), h, l);
        hi[j] = h;
        lo[j] = l;
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][cb] = mfma_bf16(w[rb], hi, acc[rb][cb]);
        acc[rb][cb] = mfma_bf16(w[rb], lo, acc[rb][cb]);
      }
    }
  }

  // sum of squares: lanes col, col+16, col+32, col+48 hold the same token
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    ss[cb] += __shfl_xor(ss[cb], 16);
    ss[cb] += __shfl_xor(ss[cb], 32);
    if (grp == 0) ssred[(wave * NCB + cb) * 16 + col] = ss[cb];
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) red[((wave * RB + rb) * NCB + cb) * 64 + lane] = acc[rb][cb];
  __syncthreads();

  // epilogue: one thread per (pair, token); pairs fastest for coalesced stores
  constexpr int kPairs = RB * 8;
  const float inv_d = 1.0f / (float)d;
  for (int o = threadIdx.x; o < kPairs * NCB * 16; o += 64 * S) {
    const int p = o % kPairs, t = o / kPairs;
    if (t >= M) continue;
    const int cb = t >> 4, c = t & 15;
    const int rb = p >> 3, lr = (p & 7) * 2;  // gate row within the block
    const int L = (lr >> 2) * 16 + c, e = lr & 3;
    float g = 0.f, u = 0.f, sst = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const f32x4 v = red[((s * RB + rb) * NCB + cb) * 64 + L];
      g += v[e];
      u += v[e + 1];
      sst += ssred[(s * NCB + cb) * 16 + c];
    }
    const float r = 1.0f / sqrtf(sst * inv_d + eps);
    const float av = silu_mul(g * r, u * r);
    const uint16_t h = bf16_rne(av);
    const int64_t idx = (int64_t)t * ff + row0 / 2 + p;
    a_hi[idx] = h;
    a_lo[idx] = bf16_rne(av - __uint_as_float((uint32_t)h << 16));
  }
}

// ---------------------------------------------------------------------------
// down projection: y[t, j] = sum_i W_down[j, i] a[t, i], a = a_hi + a_lo.
template <int NCB, int RB, int S>
__global__ __launch_bounds__(64 * S) void k_decode_down_bf16(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const uint16_t* __restrict__ wd, uint16_t* __restrict__ y, int M, int d, int ff) {
  __shared__ f32x4 red[S * RB * NCB * 64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (RB * 16);
  const int nkb = ff >> 5;

  const uint16_t* wrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) wrow[rb] = wd + (row0 + rb * 16 + col) * (int64_t)ff + grp * 8;
  const uint16_t* ahr[NCB];
  const uint16_t* alr[NCB];
  bool tok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int t = cb * 16 + col;
    tok[cb] = t < M;
    const int64_t off = (int64_t)(tok[cb] ? t : 0) * ff + grp * 8;
    ahr[cb] = a_hi + off;
    alr[cb] = a_lo + off;
  }

  f32x4 acc[RB][NCB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int kb = wave;
  u32x4 wn[RB];
  if (kb < nkb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) wn[rb] = ld16_stream(wrow[rb] + kb * 32);
  }
  for (; kb < nkb; kb += S) {
    u32x4 w[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) w[rb] = wn[rb];
    if (kb + S < nkb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wn[rb] = ld16_stream(wrow[rb] + (kb + S) * 32);
    }
    const int k = kb * 32;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
      if (tok[cb]) {
        hi = ld16(ahr[cb] + k);
        lo = ld16(alr[cb] + k);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][cb] = mfma_bf16(w[rb], hi, acc[rb][cb]);
        acc[rb][cb] = mfma_bf16(w[rb], lo, acc[rb][cb]);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) red[((wave * RB + rb) * NCB + cb) * 64 + lane] = acc[rb][cb];
  __syncthreads();

  constexpr int kRows = RB * 16;
  for (int o = threadIdx.x; o < kRows * NCB * 16; o += 64 * S) {
    const int rl = o % kRows, t = o / kRows;
    if (t >= M) continue;
    const int cb = t >> 4, c = t & 15;
    const int rb = rl >> 4, lr = rl & 15;
    const int L = (lr >> 2) * 16 + c, e = lr & 3;
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) sum += red[((s * RB + rb) * NCB + cb) * 64 + L][e];
    y[(int64_t)t * d + row0 + rl] = bf16_rne(sum);
  }
}

// ---------------------------------------------------------------------------

template <int NCB>
static hipError_t launch_decode_bf16_t(const Problem& p, hipStream_t stream) {
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.ws);
  uint16_t* a_lo = reinterpret_cast<uint16_t*>(p.ws + align256((size_t)p.M * p.ff * 2));
  constexpr int RB_GU = (NCB == 1) ? 4 : 2, S_GU = 8;
  constexpr int RB_D = 1, S_D = 16;
  const int gu_blocks = (2 * p.ff) / (16 * RB_GU);
  {
    ProfileScope prof(KK_DECODE_GATEUP_BF16, stream);
    hipLaunchKernelGGL((k_decode_gateup_bf16<NCB, RB_GU, S_GU>), dim3(gu_blocks), dim3(64 * S_GU),
                       0, stream, p.x, p.gamma, p.eps, reinterpret_cast<const uint16_t*>(p.w_gu),
                       a_hi, a_lo, p.M, p.d, p.ff);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int d_blocks = p.d / (16 * RB_D);
  ProfileScope prof(KK_DECODE_DOWN_BF16, stream);
  hipLaunchKernelGGL((k_decode_down_bf16<NCB, RB_D, S_D>), dim3(d_blocks), dim3(64 * S_D), 0,
                     stream, a_hi, a_lo, reinterpret_cast<const uint16_t*>(p.w_down), p.y, p.M,
                     p.d, p.ff);
  return hipGetLastError();
}

hipError_t launch_decode_int4(const Problem& p, hipStream_t stream);

hipError_t launch_decode(const Problem& p, hipStream_t stream) {
  if (p.wtype == 1) return launch_decode_int4(p, stream);
  if (p.M <= 16) return launch_decode_bf16_t<1>(p, stream);
  return launch_decode_bf16_t<2>(p, stream);
}

}  // namespace fmlp
