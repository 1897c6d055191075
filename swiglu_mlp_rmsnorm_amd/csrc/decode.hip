// Decode path (M <= 32 tokens): two kernels per forward (three for int4,
// and for bf16 weights at M > 16).
//
//   0. (int4; bf16 at M > 16) act prep: r = 1/sqrt(mean(x^2) + eps) per token
//      and the normalised input n = gamma * x * r as fp16, in the int4
//      operand order or in natural order (FastTPS review, section 3, Figure 4
//      part1). On the bf16 path at M <= 16 the RMSNorm is folded into step 1
//      instead.
//   1. gate/up: z = W_gu n over the interleaved rows, then a = SiLU(z_gate) *
//      z_up on each (2i, 2i+1) pair in registers (Figure 4 part2; llama.cpp
//      PR digest: the GLU is applied in the same pass as the gate/up matmul).
//      Only a (M x ff) leaves the kernel.
//   2. down: y = W_down a (Figure 4 part3).
//
// Steps 1 and 2 are bound by HBM reads of the weights (decode arithmetic
// intensity is about M flop/byte against a bf16 ridge of ~315 flop/byte), so
// they are built to stream: weights arrive in the fragment-tiled layout, one
// contiguous 1 KB tile per 16-row x 32-column block, read by one 16-byte load
// per lane straight into the MFMA operand layout; each wave keeps a P-deep
// register ring of upcoming tiles in flight; the S waves of a workgroup split
// K and reduce through LDS in a fixed order (deterministic results).
//
// Dot products run on MFMA 16x16x32 with A = activations (16 token rows, zero
// above M) and B = weights (16 weight rows), so lane l accumulates weight row
// l%16 for tokens 4*(l/16) .. +3.
//
// bf16 weights: the activation is an exact-to-2^-17 bf16 hi + lo pair (two
// bf16 MFMAs per tile), so the normalised input and the SiLU*mul
// intermediate keep fp32-like precision (rounding either to bf16 alone
// breaks the accuracy bar at the larger shapes). At M > 16 (two token blocks)
// the activations are fp16 instead, as on the prefill path: one f16 MFMA per
// tile against the weight tile converted to fp16 in registers (exact in the
// fp16 normal range), and half the activation bytes per workgroup, which at
// that M match the weight bytes.
//
// int4 weights: one fp16 MFMA per group. The conversion is the published
// magic-number int4 -> fp16 method (Kim et al., "Who Says Elephants Can't
// Run", arXiv 2211.10017): a 4-bit field placed under the fp16 exponent of
// 1024 is an exact fp16 integer. A word holds the 8 codes a lane needs; with
// u = word ^ 0x88888888 each nibble is q+8, and
//   (u & 0x000F000F) | 0x64006400 -> fp16 (1032 + q0, 1032 + q4)
//   (u & 0x00F000F0) | 0x64006400 -> fp16 (1152 + 16 q1, 1152 + 16 q5)
// (and the same on u >> 8 for codes 2,6 / 3,7): six VALU operations per 8
// weights, all exact. The activation slots facing the x16 codes carry n/16,
// and a second MFMA of the activations against the constant offsets
// (-1032 / -1152) seeds the accumulator, so the pair of MFMAs returns
// sum_k q_k n_k for the group exactly up to fp32 rounding; the lane then
// scales it by its row's fp16 group scale. Activation and intermediate are
// fp16 on this path (inside the accuracy bar).
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace fmlp {

// Launch settings, each chosen by measurement on MI355X.
constexpr int kGuRb = 2;          // 16-row blocks per gate/up workgroup
constexpr int kGuS = 8;           // waves per gate/up workgroup (split K)
constexpr int kGuP = 2;           // ring depth (tiles in flight per wave and row block)
constexpr int kGuSMany = 4;       // waves per gate/up workgroup when there are many workgroups
constexpr int kGuManyWgs = 768;   // "many": at least this many gate/up workgroups
constexpr int kDnS = 16;          // waves per down workgroup
constexpr int kDnP = 1;           // down ring depth
constexpr int kQ4P = 1;           // int4 ring depth (super-tiles of 4 groups), both kernels
constexpr int kQ4GuRb = 2;        // int4 gate/up row blocks per workgroup
constexpr int kDnSplitS = 8;      // waves per workgroup of a K-split down launch
constexpr int kDnRb = 1;          // down row blocks per workgroup (bf16)
constexpr int kQ4DnRb = 2;        // down row blocks per workgroup (int4)
constexpr int kFuS = 16;          // waves per single-pass workgroup
constexpr int kFuP = 1;           // single-pass gate/up ring depth
constexpr int kFuDq = 8;          // single-pass down tiles in flight per wave
// Above kBigM tokens the activation loads of each K unit are shared by more
// weight rows (the settings below).
constexpr int kBigM = 4;
constexpr int kBigDnM = 1;        // the down kernel's large-M settings above this M
constexpr int kBigGuRb = 4;       // bf16 gate/up row blocks per workgroup for M > kBigM
constexpr int kBigDnRb = 4;       // down row blocks per workgroup for M > kBigDnM (split K)
constexpr int kBigDnS = 8;        // and its waves (M <= 16)
constexpr int kBigDnS2 = 8;       // and its waves (M > 16; 16 measured 3-9% slower)
constexpr int kBigGuRb2 = 4;      // bf16 gate/up row blocks per workgroup for M > 16 ...
constexpr int kBigGuRb2w = 8;     // ... or this many, where that adds no row blocks to the
                                  // most any CU streams (gu_wide below)
constexpr int kQ4BigGuRb = 4;     // int4 gate/up row blocks per workgroup for 4 < M <= 16
// bf16 weights: from this M on, fp16 activations (WK_BF16H); measured -10% at
// Llama-8B M=32, no gain at M=16 (the prep launch costs what the kernels
// save), a loss at M=8.
constexpr int kH16MinM = 17;

// Weight kinds: bf16 weights with the bf16 hi + lo activation pair; int4
// weights; bf16 weights with fp16 activations (several tokens: one MFMA per
// tile instead of two and half the activation bytes, the weight tile
// converted to fp16 in registers).
enum { WK_BF16 = 0, WK_INT4 = 1, WK_BF16H = 2, WK_F16 = 3 };
// bf16 or fp16 weights read with fp16 activations
constexpr bool wk_h16(int wk) { return wk == WK_BF16H || wk == WK_F16; }

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Down-projection split along K (see k_decode_down): with `blocks` row-block
// groups (d/16 over the row blocks per workgroup), split each into k slices
// when that spreads the work more evenly over the 256 CUs (time ~ rounds of
// workgroups / k), keeping at least min_units K units per slice; at most
// kMaxSplit. The kernel gives each slice ceil(nu / splits) units, so the
// count is taken as ceil(nu / ceil(nu / k)): then (splits - 1) slices of that
// length cover fewer than nu units and no slice is empty.
constexpr int kMaxSplit = 8;
static int down_splits(int64_t blocks, int64_t ff, bool int4) {
  const int64_t nu = int4 ? (ff + 127) / 128 : ff / 32;
  const int64_t min_units = int4 ? 4 : 16;
  int best = 1;
  double tb = (double)((blocks + 255) / 256);
  for (int k = 2; k <= kMaxSplit; ++k) {
    if (nu / k < min_units) break;
    const int64_t per = (nu + k - 1) / k;
    const int s = (int)((nu + per - 1) / per);
    const double t = (double)((blocks * s + 255) / 256) / s;
    if (t < tb - 1e-9) tb = t, best = s;
  }
  return best;
}

size_t decode_workspace_bytes(int64_t M, int64_t d, int64_t ff) {
  // n fp16 [M, d] (int4 only); a: bf16 hi + lo [M, ff] (int4: fp16 in the
  // first half); split-K partials fp32 [kMaxSplit, M, d]; counters [d/16]
  return align256((size_t)M * d * 2) + 2 * align256((size_t)M * ff * 2) +
         align256((size_t)kMaxSplit * M * d * 4) + align256((size_t)(d / 16) * 4);
}

struct DecodeWs {
  uint16_t *n0, *a0, *a1;
  float* part;
  int* cnt;
};

static DecodeWs decode_ws(const Problem& p) {
  const size_t nb = align256((size_t)p.M * p.d * 2), ab = align256((size_t)p.M * p.ff * 2);
  const size_t pb = align256((size_t)kMaxSplit * p.M * p.d * 4);
  char* b = p.ws;
  return DecodeWs{reinterpret_cast<uint16_t*>(b), reinterpret_cast<uint16_t*>(b + nb),
                  reinterpret_cast<uint16_t*>(b + nb + ab),
                  reinterpret_cast<float*>(b + nb + 2 * ab),
                  reinterpret_cast<int*>(b + nb + 2 * ab + pb)};
}

// ------------------------------------------------------------ int4 helpers

// 8 codes -> fp16 operand words (see the file comment for the slot order).
// (w ^ 0x88888888) & m | 0x64006400 equals (w & m) ^ (0x64006400 | (0x88888888
// & m)), the nibble field and the fp16 exponent bits being disjoint: one
// 3-input bit operation per word pair.
__device__ __forceinline__ u32x4 int4_to_f16_magic(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = (w & 0x000F000Fu) ^ 0x64086408u;
  r[1] = (w & 0x00F000F0u) ^ 0x64806480u;
  r[2] = (w8 & 0x000F000Fu) ^ 0x64086408u;
  r[3] = (w8 & 0x00F000F0u) ^ 0x64806480u;
  return r;
}

// Negated magic offsets per slot: -1032 for slots of codes 0,4,2,6 and -1152
// for slots of codes 1,5,3,7 (fp16 0xE408 / 0xE480).
constexpr uint32_t kNegOffA = 0xE408E408u, kNegOffB = 0xE480E480u;

// Position of logical element m (0..7) of an 8-block in the int4 operand
// order, and whether that slot carries the value divided by 16.
__device__ __forceinline__ int q4_slot(int m) { return (m & 1) ? 2 + ((m >> 1) & 1) * 4 + (m >> 2) : (m >> 1 & 1) * 4 + (m >> 2); }

// ------------------------------------------------------------ act prep
// (int4; bf16 weights at M > 16.) One 512-thread workgroup per token:
// r = 1/sqrt(mean(x^2) + eps), then n = x * gamma * r stored as fp16 [M, d],
// either in the int4 slot order with the slots of odd elements carrying
// n/16, or in natural order. Each thread issues all its x and gamma
// loads at once and keeps x in registers between the two steps (d up to
// kActPrepChunks * 8 * 512; larger d takes a second pass over x).
constexpr int kActPrepChunks = 4;

__device__ __forceinline__ u32x4 act_q4_chunk(u32x4 v, u32x4 g, float r) {
  float n[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    n[2 * j] = bf16_lo(v[j]) * bf16_lo(g[j]) * r;
    n[2 * j + 1] = bf16_hi(v[j]) * bf16_hi(g[j]) * r;
  }
  _Float16 h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[q4_slot(e)] = (_Float16)((e & 1) ? n[e] * 0.0625f : n[e]);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, h[2 * j]) |
           ((uint32_t)__builtin_bit_cast(uint16_t, h[2 * j + 1]) << 16);
  return o;
}

// The same in natural order (no slot permutation, no 1/16 slots): the fp16
// activations of the bf16-weight several-token path.
__device__ __forceinline__ u32x4 act_f16_chunk(u32x4 v, u32x4 g, float r) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)(bf16_lo(v[j]) * bf16_lo(g[j]) * r);
    const _Float16 hi = (_Float16)(bf16_hi(v[j]) * bf16_hi(g[j]) * r);
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

// With res, the row normalised is the residual stream h = bf16_rne(x + res),
// which is also stored to hout. Q4: the int4 slot order, else natural order.
template <bool Q4>
__global__ __launch_bounds__(512) void k_act_prep(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ gamma,
                                                     float eps, uint16_t* __restrict__ n0, int d,
                                                     const uint16_t* __restrict__ res,
                                                     uint16_t* __restrict__ hout) {
  __shared__ float part[8];
  const int64_t m = blockIdx.x;
  const uint16_t* xr = x + m * d;
  const int chunks = d >> 3, tid = threadIdx.x;
  // chunk c of the row being normalised
  auto row = [&](int c) {
    const u32x4 xv = ld16(xr + c * 8);
    return res ? add_bf16x8(xv, ld16(res + m * d + c * 8)) : xv;
  };
  u32x4 v[kActPrepChunks], g[kActPrepChunks];
#pragma unroll
  for (int i = 0; i < kActPrepChunks; ++i) {
    const int c = tid + i * 512;
    v[i] = c < chunks ? row(c) : u32x4{0u, 0u, 0u, 0u};
    g[i] = c < chunks ? ld16(gamma + c * 8) : u32x4{0u, 0u, 0u, 0u};
    if (hout && c < chunks) st16(hout + m * d + c * 8, v[i]);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kActPrepChunks; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(v[i][j]), b = bf16_hi(v[i][j]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  for (int c = tid + kActPrepChunks * 512; c < chunks; c += 512) {  // only for very large d
    const u32x4 w = row(c);
    if (hout) st16(hout + m * d + c * 8, w);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(w[j]), b = bf16_hi(w[j]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < 8; ++w) tot += part[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int i = 0; i < kActPrepChunks; ++i) {
    const int c = tid + i * 512;
    if (c < chunks)
      st16(n0 + m * d + c * 8, Q4 ? act_q4_chunk(v[i], g[i], r) : act_f16_chunk(v[i], g[i], r));
  }
  for (int c = tid + kActPrepChunks * 512; c < chunks; c += 512) {
    const u32x4 xv = row(c), gv = ld16(gamma + c * 8);
    st16(n0 + m * d + c * 8, Q4 ? act_q4_chunk(xv, gv, r) : act_f16_chunk(xv, gv, r));
  }
}

// ------------------------------------------------------------ GEMV core
// acc[rb][cb] += W[row block rb0+rb] . act for the K range owned by this wave.
// Activation operand modes:
//   ACT_X      : bf16 weights; act = gamma * x (unnormalised, exact in fp32),
//                split hi/lo here from act0 = x [M, K] and act1 = gamma [K];
//                also accumulates sum x^2 per token into ss (RMS folded later)
//   ACT_HL     : bf16 weights; act0 / act1 = hi / lo bf16 [M, K], natural order
//   ACT_Q4     : int4 weights; act0 = fp16 [M, K] in the int4 slot order
//   ACT_HL_LDS : as ACT_HL, act0 / act1 staged in LDS by the workgroup
//   ACT_Q4_LDS : as ACT_Q4, act0 staged in LDS by the workgroup
//   ACT_XR     : as ACT_X on the residual stream h = bf16_rne(x + res) (res
//                [M, K] like x); h is also stored to hout when that is given
//   ACT_F16    : bf16 weights, each tile converted to fp16 in registers;
//                act0 = fp16 [M, K], natural order; one f16 MFMA per tile
//   ACT_F16W   : as ACT_F16 on fp16 weights (no conversion)
// Global activations are read into the ring with the weights. Staged ones
// are [M, astride] rows whose first element is k = kbase; they are read
// from LDS as they are used. stage_load() issues the workgroup's loads of
// them before the first weight loads (they hit L2, so they return first),
// stage_store() writes them to LDS once those are issued; then a
// workgroup barrier.
// Weights: bf16 tiles (1 KB per 16 x 32 block) or int4 super-tiles (1 KB per
// 16 rows x 4 groups) + scales. The K units u0 .. u0+ucnt-1 are covered;
// each wave walks units u0+wave, u0+wave+S, ...
// with a P-deep ring of weight tiles (and global activation chunks) in flight.
enum {
  ACT_X = 0, ACT_HL = 1, ACT_Q4 = 2, ACT_HL_LDS = 3, ACT_Q4_LDS = 4, ACT_XR = 5, ACT_F16 = 6,
  ACT_F16W = 7
};

// EMAX: accumulator rows per lane that can hold a token (int4 scale FMAs;
// 1 when M = 1).
template <int MODE, int NCB, int RB, int S, int P, int EMAX = 4, class StageLoad,
          class StageStore>
__device__ __forceinline__ void gemv_core(const void* __restrict__ w,
                                          const uint16_t* __restrict__ sc,
                                          const uint16_t* __restrict__ act0,
                                          const uint16_t* __restrict__ act1, int64_t rb0, int K,
                                          int M, int u0, int ucnt, f32x4 (&acc)[RB][NCB],
                                          float (&ss)[NCB], int astride, int kbase,
                                          StageLoad&& stage_load, StageStore&& stage_store,
                                          const uint16_t* __restrict__ res = nullptr,
                                          uint16_t* __restrict__ hout = nullptr) {
  constexpr bool kLds = MODE == ACT_HL_LDS || MODE == ACT_Q4_LDS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nkb = K >> 5;
  int64_t aoff[NCB];
  bool tok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int t = cb * 16 + col;
    tok[cb] = t < M;
    aoff[cb] = (int64_t)(tok[cb] ? t : 0) * astride + grp * 8 - kbase;
    ss[cb] = 0.f;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr bool kX = MODE == ACT_X || MODE == ACT_XR;  // activations from x (and res)
  if constexpr (kX || MODE == ACT_HL || MODE == ACT_HL_LDS || MODE == ACT_F16 ||
                MODE == ACT_F16W) {
    // unit = one 32-column group
    const uint16_t* wt = static_cast<const uint16_t*>(w) + lane * 8;
    const int nit = wave < ucnt ? (ucnt - wave + S - 1) / S : 0;
    u32x4 wb[P][RB], hb[P][NCB], lb[P][NCB];
    u32x4 gb[P];
    // units past this wave's range (prologue slots beyond nit) re-read its
    // last unit, or unit 0 when it has none: in bounds, and never consumed
    const int klast = nit > 0 ? u0 + wave + (nit - 1) * S : 0;
    // weights (and global activations) of ring slot `slot`
    auto issue = [&](int slot, int it) {
      const int kb = it < nit ? u0 + wave + it * S : klast;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wb[slot][rb] = ld16_stream(wt + ((rb0 + rb) * nkb + kb) * 512);
      if constexpr (!kLds) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          hb[slot][cb] = ld16(act0 + aoff[cb] + kb * 32);
          if (MODE == ACT_HL) lb[slot][cb] = ld16(act1 + aoff[cb] + kb * 32);
          if (MODE == ACT_XR) lb[slot][cb] = ld16(res + aoff[cb] + kb * 32);  // residual
        }
        if (kX) gb[slot] = ld16(act1 + grp * 8 + kb * 32);
      }
    };
    // no branches around the first loads, so that the compiler's wait for
    // the staged chunks leaves the weight loads behind them in flight
    if constexpr (kLds) {
      stage_load();
      __builtin_amdgcn_sched_barrier(0);  // keep the staged loads ahead of the weights
    }
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p, p);
    if constexpr (kLds) {
      __builtin_amdgcn_sched_barrier(0);
      stage_store();
      __syncthreads();
    }
    for (int i0 = 0; i0 < nit; i0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int it = i0 + p;
        if (it < nit) {
          const int kb = u0 + wave + it * S;
          u32x4 wv[RB], h[NCB], l[NCB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) wv[rb] = wb[p][rb];
          const u32x4 gv = gb[p];
          // (lanes of absent tokens read token 0's activations: MFMA rows
          // are independent, so they only fill accumulator rows that are
          // never reduced into a stored output; no masking needed)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            if constexpr (kLds) {
              h[cb] = *reinterpret_cast<const u32x4*>(act0 + aoff[cb] + kb * 32);
              l[cb] = *reinterpret_cast<const u32x4*>(act1 + aoff[cb] + kb * 32);
            } else {
              h[cb] = hb[p][cb];
              l[cb] = lb[p][cb];
            }
          }
          if constexpr (MODE == ACT_F16 || MODE == ACT_F16W) {
            if constexpr (MODE == ACT_F16) {
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) wv[rb] = bf16x8_to_f16x8(wv[rb]);
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) acc[rb][cb] = mfma_f16(h[cb], wv[rb], acc[rb][cb]);
          } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              if (kX) {
                // h holds x (l the residual); build the hi/lo pair of gamma * x in place
                u32x4 xv = h[cb];
                if (MODE == ACT_XR) {
                  xv = add_bf16x8(xv, l[cb]);
                  if (hout != nullptr && tok[cb]) st16(hout + aoff[cb] + kb * 32, xv);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float x0 = bf16_lo(xv[j]), x1 = bf16_hi(xv[j]);
                  ss[cb] = fmaf(x0, x0, ss[cb]);
                  ss[cb] = fmaf(x1, x1, ss[cb]);
                  uint32_t hh, ll;
                  split_bf16_pair(x0 * bf16_lo(gv[j]), x1 * bf16_hi(gv[j]), hh, ll);
                  h[cb][j] = hh;
                  l[cb][j] = ll;
                }
              }
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) {
                acc[rb][cb] = mfma_bf16(h[cb], wv[rb], acc[rb][cb]);
                acc[rb][cb] = mfma_bf16(l[cb], wv[rb], acc[rb][cb]);
              }
            }
          }
          // the slot's next tile is issued once this one has been consumed,
          // so its registers are reused in place rather than copied out
          // (measured 0.5-2% faster than issuing before the MFMAs)
          if (it + P < nit) issue(p, it + P);
        }
      }
    }
  } else {
    // unit = one super-tile of 4 groups
    const int nq = (K + 127) >> 7;
    const uint8_t* qt = static_cast<const uint8_t*>(w) + lane * 16;
    const uint16_t* stl = sc + col * 4;
    const int nit = wave < ucnt ? (ucnt - wave + S - 1) / S : 0;
    const u32x4 negoff = {kNegOffA, kNegOffB, kNegOffA, kNegOffB};
    u32x4 qb[P][RB], ab[P][4][NCB];
    uint64_t sb[P][RB];
    const int qlast = nit > 0 ? u0 + wave + (nit - 1) * S : 0;  // as in the bf16 branch
    auto issue = [&](int slot, int it) {
      const int q = it < nit ? u0 + wave + it * S : qlast;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t st = (rb0 + rb) * nq + q;
        qb[slot][rb] = ld16_stream(qt + st * 1024);
        sb[slot][rb] = *reinterpret_cast<const uint64_t*>(stl + st * 64);
      }
      if constexpr (!kLds) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kb = q * 4 + j < nkb ? q * 4 + j : nkb - 1;  // padding groups are skipped
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            ab[slot][j][cb] = ld16(act0 + aoff[cb] + kb * 32);
        }
      }
    };
    // no branches around the first loads, so that the compiler's wait for
    // the staged chunks leaves the weight loads behind them in flight
    if constexpr (kLds) {
      stage_load();
      __builtin_amdgcn_sched_barrier(0);  // keep the staged loads ahead of the weights
    }
#pragma unroll
    for (int p = 0; p < P; ++p) issue(p, p);
    if constexpr (kLds) {
      __builtin_amdgcn_sched_barrier(0);
      stage_store();
      __syncthreads();
    }
    for (int i0 = 0; i0 < nit; i0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int it = i0 + p;
        if (it < nit) {
          const int q = u0 + wave + it * S;
          u32x4 qv[RB], av[4][NCB];
          uint64_t sv[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            qv[rb] = qb[p][rb];
            sv[rb] = sb[p][rb];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kb = q * 4 + j < nkb ? q * 4 + j : nkb - 1;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              // (absent tokens: as in the bf16 branch, no masking needed)
              if constexpr (kLds)
                av[j][cb] = *reinterpret_cast<const u32x4*>(act0 + aoff[cb] + kb * 32);
              else
                av[j][cb] = ab[p][j][cb];
            }
          }
          // (unstaged activations: the next tile is issued after this one is
          // consumed, as in the bf16 branch; measured: down 6% faster at
          // M = 16, while the staged kernels at M <= 4 keep the early issue)
          if (kLds && it + P < nit) issue(p, it + P);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (q * 4 + j >= nkb) break;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const f32x4 c = mfma_f16(av[j][cb], negoff, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int rb = 0; rb < RB; ++rb) {
                const f32x4 dq = mfma_f16(av[j][cb], int4_to_f16_magic(qv[rb][j]), c);
                const float s = (float)__builtin_bit_cast(
                    _Float16, (uint16_t)(sv[rb] >> (16 * j)));
#pragma unroll
                for (int e = 0; e < EMAX; ++e) acc[rb][cb][e] = fmaf(s, dq[e], acc[rb][cb][e]);
              }
            }
          }
          if (!kLds && it + P < nit) issue(p, it + P);
        }
      }
    }
  }
}

// Cross-wave reduction of the accumulators through LDS (fixed wave order).
// Afterwards red[((w*RB + rb)*NCB + cb)*64 + lane] holds wave w's values.
template <int RB, int NCB>
__device__ __forceinline__ void stash(f32x4* red, const f32x4 (&acc)[RB][NCB]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) red[((wave * RB + rb) * NCB + cb) * 64 + lane] = acc[rb][cb];
}

// ------------------------------------------------------------ gate/up kernel
// Workgroup: RB blocks of 16 W_gu rows (RB*8 gate/up pairs), S waves split K.
// bf16: activations come straight from x and gamma (ACT_X); each wave also
// sums x^2 over its K units, the sums are reduced with the dot products and
// r = 1/sqrt(mean(x^2) + eps) scales z before SiLU*mul (z * r = W (gamma x r)).
// Writes a = a0 + a1 (bf16 hi/lo, natural order, [M, ff]).
// int4: activations are the prepared fp16 n (ACT_Q4); writes a0 = fp16 a in
// the int4 slot order, [M, ff]. bf16 weights with fp16 activations
// (WK_BF16H), or fp16 weights (WK_F16): the prepared fp16 n in natural order
// (ACT_F16, ACT_F16W); writes a0 = fp16 a, [M, ff].
// LDS: the workgroup first stages its activations in LDS (dynamic shared
// memory): gamma * x as the bf16 hi + lo pair with the per-token sums of x^2
// (bf16), or a copy of n (int4); for small M, where the per-wave activation
// loads would carry mostly duplicated lanes.
// Workgroup 0 also clears the down kernel's split-K arrival counters (ncnt of
// them; agent-coherent stores, read by that kernel's atomics).
constexpr int kLdsMaxM = 4;           // staged activations: at most this many tokens
constexpr int kStageRegs = 2;         // staged chunks a gate/up thread holds in registers (8 waves)
constexpr int kStageRegsDown = 4;     // the same for the down kernel

// RES (bf16): the activations are the residual stream h = bf16_rne(x + res);
// workgroup 0 stores h to hout. act: the gate activation.
template <int WK, int NCB, int RB, int S, int P, bool LDS, bool RES, int EMAX = 4>
__global__ __launch_bounds__(64 * S) void k_decode_gateup(
    const void* __restrict__ w, const uint16_t* __restrict__ sc, const uint16_t* __restrict__ act0,
    const uint16_t* __restrict__ act1, float eps, uint16_t* __restrict__ a0,
    uint16_t* __restrict__ a1, int M, int d, int ff, int* __restrict__ cnt, int ncnt, int act,
    const uint16_t* __restrict__ res, uint16_t* __restrict__ hout) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < ncnt; i += 64 * S)
      __hip_atomic_store(cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __shared__ f32x4 red[S * RB * NCB * 64];
  __shared__ float ssred[S * NCB * 16];
  extern __shared__ __align__(16) uint16_t stage_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rb0 = (int64_t)blockIdx.x * RB;
  f32x4 acc[RB][NCB];
  float ss[NCB];
  const int units = WK == WK_INT4 ? (d + 127) >> 7 : d >> 5;
  if constexpr (LDS) {
    uint16_t* lhi = stage_lds;
    uint16_t* llo = stage_lds + (int64_t)M * d;
    const int cpt = d >> 3, nch = M * cpt;  // 16-byte chunks per token, in all
    constexpr int kSR = kStageRegs * 8 / S > 0 ? kStageRegs * 8 / S : 1;  // chunks per thread
    u32x4 sx[kSR], sg[kSR];
    auto stage_load = [&]() {
#pragma unroll
      for (int i = 0; i < kSR; ++i) {
        int c = threadIdx.x + i * 64 * S;
        c = c < nch ? c : nch - 1;  // loaded, not stored
        const int t = c / cpt, kc = c - t * cpt;
        sx[i] = ld16(act0 + (int64_t)t * d + kc * 8);
        if constexpr (WK == WK_BF16) sg[i] = ld16(act1 + kc * 8);
      }
    };
    auto stage_store = [&]() {
      float sp[kLdsMaxM] = {0.f, 0.f, 0.f, 0.f};
      // valid: c is this thread's own chunk (a clamped duplicate rewrites
      // the last chunk with the same value and adds nothing to the sums)
      auto put = [&](int c, u32x4 xv, u32x4 gv, bool valid) {
        const int t = c / cpt, kc = c - t * cpt;
        if constexpr (WK == WK_BF16) {
          u32x4 hv, lv;
          float sacc = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = bf16_lo(xv[j]), x1 = bf16_hi(xv[j]);
            sacc = fmaf(x0, x0, sacc);
            sacc = fmaf(x1, x1, sacc);
            uint32_t hh, ll;
            split_bf16_pair(x0 * bf16_lo(gv[j]), x1 * bf16_hi(gv[j]), hh, ll);
            hv[j] = hh;
            lv[j] = ll;
          }
          *reinterpret_cast<u32x4*>(lhi + t * d + kc * 8) = hv;
          *reinterpret_cast<u32x4*>(llo + t * d + kc * 8) = lv;
#pragma unroll
          for (int tt = 0; tt < kLdsMaxM; ++tt)
            if (valid && t == tt) sp[tt] += sacc;
        } else {
          *reinterpret_cast<u32x4*>(lhi + t * d + kc * 8) = xv;
        }
      };
      // unconditional stores keep the compiler from sinking the staged
      // loads below the weight loads
#pragma unroll
      for (int i = 0; i < kSR; ++i) {
        const int c = threadIdx.x + i * 64 * S;
        put(c < nch ? c : nch - 1, sx[i], sg[i], c < nch);
      }
      for (int c = threadIdx.x + kSR * 64 * S; c < nch; c += 64 * S) {
        const int kc = c % cpt;
        put(c, ld16(act0 + (int64_t)(c / cpt) * d + kc * 8),
            WK == WK_BF16 ? ld16(act1 + kc * 8) : u32x4{0u, 0u, 0u, 0u}, true);
      }
      if constexpr (WK == WK_BF16) {
#pragma unroll
        for (int tt = 0; tt < kLdsMaxM; ++tt) {
          float v = sp[tt];
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
          if (lane == 0) ssred[wave * 16 + tt] = v;
        }
      }
    };
    gemv_core<WK == WK_BF16 ? ACT_HL_LDS : ACT_Q4_LDS, NCB, RB, S, P, EMAX>(
        w, sc, lhi, llo, rb0, d, M, 0, units, acc, ss, d, 0, stage_load, stage_store);
    stash<RB, NCB>(red, acc);
  } else {
    gemv_core<WK == WK_BF16    ? (RES ? ACT_XR : ACT_X)
              : WK == WK_BF16H ? ACT_F16
              : WK == WK_F16   ? ACT_F16W
                               : ACT_Q4,
              NCB,
              RB, S, P>(w, sc, act0, act1, rb0, d, M, 0, units, acc, ss, d, 0, [] {}, [] {}, res,
                        blockIdx.x == 0 ? hout : nullptr);
    stash<RB, NCB>(red, acc);
    if (WK == WK_BF16) {
      // lanes col, col+16, col+32, col+48 hold the same token
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float v = ss[cb];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 16) ssred[(wave * NCB + cb) * 16 + lane] = v;
      }
    }
  }
  __syncthreads();
  // one thread per (pair, token), pairs fastest
  constexpr int kPairs = RB * 8;
  const float inv_d = 1.0f / (float)d;
  for (int o = threadIdx.x; o < kPairs * M; o += 64 * S) {
    const int p = o % kPairs, t = o / kPairs;
    const int cb = t >> 4, c = t & 15;
    const int rb = p >> 3, lr = (p & 7) * 2;
    const int L = (c >> 2) * 16 + lr, e = c & 3;
    float g = 0.f, u = 0.f, sst = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int base = ((s * RB + rb) * NCB + cb) * 64 + L;
      g += red[base][e];
      u += red[base + 1][e];
      if (WK == WK_BF16) sst += ssred[(s * NCB + cb) * 16 + c];
    }
    const int i = (int)(rb0 * 8) + p;  // index along ff
    if (WK == WK_BF16) {
      const float r = 1.0f / sqrtf(sst * inv_d + eps);
      const float av = act_mul(act, g * r, u * r);
      const uint16_t h = bf16_rne(av);
      a0[(int64_t)t * ff + i] = h;
      a1[(int64_t)t * ff + i] = bf16_rne(av - __uint_as_float((uint32_t)h << 16));
    } else if (wk_h16(WK)) {
      a0[(int64_t)t * ff + i] = __builtin_bit_cast(uint16_t, (_Float16)act_mul(act, g, u));
    } else {
      const float av = act_mul(act, g, u);
      const int mm = i & 7;
      const _Float16 hv = (_Float16)((mm & 1) ? av * 0.0625f : av);
      a0[(int64_t)t * ff + (i & ~7) + q4_slot(mm)] = __builtin_bit_cast(uint16_t, hv);
    }
  }
}

// ------------------------------------------------------------ down kernel
// Workgroup: RB blocks of 16 W_down rows, S waves split its K range.
// gridDim.y > 1 splits K = ff across workgroups as well (for layers with
// fewer 16-row blocks than CUs): slice ks of gridDim.y equal ranges of K
// units. Each slice stores its fp32 partial sums with agent-coherent stores,
// waits for them to complete and counts itself in on an agent-scope atomic;
// the last of a block's slices to arrive reads all partials back (agent-
// coherent loads) and writes y = bf16(sum over slices in slice order), so
// the result does not depend on arrival order. No workgroup waits for
// another.
// LDS: the workgroup stages its K range of a in LDS first (small M).
template <int WK, int NCB, int RB, int S, int P, bool LDS, int EMAX = 4>
__global__ __launch_bounds__(64 * S) void k_decode_down(
    const void* __restrict__ w, const uint16_t* __restrict__ sc, const uint16_t* __restrict__ a0,
    const uint16_t* __restrict__ a1, uint16_t* __restrict__ y, int M, int d, int ff,
    float* __restrict__ part, int* __restrict__ cnt) {
  __shared__ f32x4 red[S * RB * NCB * 64];
  __shared__ int last;
  extern __shared__ __align__(16) uint16_t stage_lds[];
  const int64_t rb0 = (int64_t)blockIdx.x * RB;
  const int splits = gridDim.y, ks = blockIdx.y;
  constexpr int UK = WK == WK_INT4 ? 128 : 32;  // K per unit
  const int nu = (ff + UK - 1) / UK;            // K units
  const int per = (nu + splits - 1) / splits;
  const int u0 = ks * per, ucnt = nu - u0 < per ? nu - u0 : per;
  f32x4 acc[RB][NCB];
  float ss[NCB];
  if constexpr (LDS) {
    // rows of per * UK elements, first element k = u0 * UK
    const int astride = per * UK, kbeg = u0 * UK;
    const int kend = (u0 + (ucnt > 0 ? ucnt : 0)) * UK < ff ? (u0 + (ucnt > 0 ? ucnt : 0)) * UK : ff;
    uint16_t* lhi = stage_lds;
    uint16_t* llo = stage_lds + (int64_t)M * astride;
    const int cpt = (kend - kbeg) >> 3, nch = M * cpt;
    u32x4 sh[kStageRegsDown], sl[kStageRegsDown];
    auto src = [&](int c) { return (int64_t)(c / cpt) * ff + kbeg + (c % cpt) * 8; };
    auto dst = [&](int c) { return (c / cpt) * astride + (c % cpt) * 8; };
    auto stage_load = [&]() {
#pragma unroll
      for (int i = 0; i < kStageRegsDown; ++i) {
        int c = threadIdx.x + i * 64 * S;
        c = c < nch ? c : nch - 1;  // loaded, not stored
        sh[i] = ld16(a0 + src(c));
        if constexpr (WK == WK_BF16) sl[i] = ld16(a1 + src(c));
      }
    };
    auto stage_store = [&]() {
      // unconditional (a clamped duplicate rewrites the last chunk with the
      // same value), which keeps the compiler from sinking the staged loads
#pragma unroll
      for (int i = 0; i < kStageRegsDown; ++i) {
        int c = threadIdx.x + i * 64 * S;
        c = c < nch ? c : nch - 1;
        *reinterpret_cast<u32x4*>(lhi + dst(c)) = sh[i];
        if constexpr (WK == WK_BF16) *reinterpret_cast<u32x4*>(llo + dst(c)) = sl[i];
      }
      for (int c = threadIdx.x + kStageRegsDown * 64 * S; c < nch; c += 64 * S) {
        *reinterpret_cast<u32x4*>(lhi + dst(c)) = ld16(a0 + src(c));
        if constexpr (WK == WK_BF16) *reinterpret_cast<u32x4*>(llo + dst(c)) = ld16(a1 + src(c));
      }
    };
    gemv_core<WK == WK_BF16 ? ACT_HL_LDS : ACT_Q4_LDS, NCB, RB, S, P, EMAX>(
        w, sc, lhi, llo, rb0, ff, M, u0, ucnt > 0 ? ucnt : 0, acc, ss, astride, kbeg, stage_load,
        stage_store);
  } else {
    gemv_core<WK == WK_BF16    ? ACT_HL
              : WK == WK_BF16H ? ACT_F16
              : WK == WK_F16   ? ACT_F16W
                               : ACT_Q4,
              NCB, RB, S, P>(
        w, sc, a0, a1, rb0, ff, M, u0, ucnt > 0 ? ucnt : 0, acc, ss, ff, 0, [] {}, [] {});
  }
  stash<RB, NCB>(red, acc);
  __syncthreads();
  for (int o = threadIdx.x; o < RB * 16 * M; o += 64 * S) {
    const int rl = o % (RB * 16), t = o / (RB * 16);
    const int rb = rl >> 4, r = rl & 15;
    const int cb = t >> 4, c = t & 15;
    const int L = (c >> 2) * 16 + r, e = c & 3;
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) sum += red[((s * RB + rb) * NCB + cb) * 64 + L][e];
    const int64_t yi = (int64_t)t * d + rb0 * 16 + rl;
    if (splits == 1)
      y[yi] = bf16_rne(sum);
    else
      __hip_atomic_store(part + (int64_t)ks * M * d + yi, sum, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  if (splits == 1) return;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(cnt + blockIdx.x, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
  __syncthreads();
  if (!last) return;
  for (int o = threadIdx.x; o < RB * 16 * M; o += 64 * S) {
    const int rl = o % (RB * 16), t = o / (RB * 16);
    const int64_t yi = (int64_t)t * d + rb0 * 16 + rl;
    // all slices' loads in flight before the first add (one load and its
    // wait per slice would chain their latencies): unconditional within each
    // group of four (the second group only when there are more than four
    // slices), slices past the last re-read it and are masked out; summed in
    // slice order
    static_assert(kMaxSplit == 8, "two groups of four partial loads");
    float pv[kMaxSplit];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      pv[k] = __hip_atomic_load(part + (int64_t)(k < splits ? k : splits - 1) * M * d + yi,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (splits > 4) {
#pragma unroll
      for (int k = 4; k < 8; ++k)
        pv[k] = __hip_atomic_load(part + (int64_t)(k < splits ? k : splits - 1) * M * d + yi,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
#pragma unroll
      for (int k = 4; k < 8; ++k) pv[k] = 0.f;
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxSplit; ++k) sum += k < splits ? pv[k] : 0.f;
    y[yi] = bf16_rne(sum);
  }
}

// ------------------------------------------------------------ single pass
// Gate/up, SiLU*mul and down in one launch (FastTPS review, section 3: the
// Fusion MLP keeps the intermediate on chip and moves only the input and the
// output). Workgroup w owns the 32 features [32w, 32w + 32) of ff:
//   1. their 64 interleaved W_gu rows (row blocks 4w .. 4w+3) against
//      gamma * x, S waves splitting K, the RMS factor folded into the
//      epilogue exactly as in k_decode_gateup;
//   2. a = SiLU(gate) * up for the 32 features, kept in LDS as the bf16
//      hi + lo operand pair;
//   3. the matching 32 columns of W_down (K unit w of every 16-row block,
//      one 1 KB tile each) against a, each wave taking every S-th row block,
//      giving the fp32 partial  part[w][t][j] = sum_{i in slice w}
//      W_down[j][i] a[t][i];
//   4. the cross-workgroup sum of the nw = ff/32 partials, by arrival, in
//      two levels: slices are grouped G = ceil(sqrt(nw)) at a time; the last
//      workgroup of a group to arrive sums its group's partials in slice
//      order into grp[g], and the last of those sums grp[0 .. ng-1] in group
//      order into y. The result does not depend on arrival order, and no
//      workgroup ever waits for another.
// The down tiles do not depend on a, so each wave issues its first DQ of
// them as soon as its gate/up loads have landed, before the cross-wave
// reduction.
//
// Ordering across workgroups (which may sit on different XCDs, whose L2
// caches are not coherent with each other): partials and group sums are
// written with agent-scope atomic stores, which the hardware writes through
// to the device-coherent level and acknowledges only once they are there;
// each thread then waits for its stores' acknowledgements (s_waitcnt
// vmcnt(0): on gfx9 the vector memory counter covers stores), the workgroup
// meets a barrier, and only then does one thread count it in with an
// agent-scope atomic add, performed at that same level. A workgroup that
// draws the last ticket therefore counts only after every other member's
// data is in device-coherent memory, and it reads them with agent-scope
// atomic loads, which are served from there rather than from a stale line
// of its own L2. This is the release / acquire pair made explicit per
// access: a fence instead would write back and invalidate the whole L2.
//
// The arrival counters need to start at zero: they live in a library-owned
// device array (zero when the library loads), and the workgroup that draws a
// counter's last ticket, the last to touch it in the launch, sets it back to
// zero. Launches of this path that overlap in time on one GPU would share
// the counters, so they must not overlap (the path's documented contract).
// RES: on the residual stream h = bf16_rne(x + res), which workgroup 0 stores
// to hout; act: the gate activation.
constexpr int kSpMaxGroups = 128;  // ceil(sqrt(ff/32)) + 1 <= 92 for ff <= 262144
__device__ unsigned int g_sp_count[kSpMaxGroups + 1];  // per group, then the final level

__host__ __device__ inline int sp_group_size(int nw) {
  int g = 1;
  while (g * g < nw) ++g;
  return g;
}

// dst[o] (or y[o] as bf16) = sum over k < n of src[k * stride + o], in k
// order, for o < len; agent-scope loads and stores. A thread takes kSpE
// outputs at a time (strided by the workgroup size) and keeps 8 loads of each
// in flight, 8 * kSpE in all, before adding them in order.
constexpr int kSpE = 4;
__device__ __forceinline__ void sp_sum(const float* src, int64_t stride, int n, int64_t len,
                                       float* dst, uint16_t* y) {
  const int64_t nt = blockDim.x;
  for (int64_t o0 = threadIdx.x; o0 < len; o0 += nt * kSpE) {
    float acc[kSpE];
#pragma unroll
    for (int e = 0; e < kSpE; ++e) acc[e] = 0.f;
    for (int k0 = 0; k0 < n; k0 += 8) {
      float v[kSpE][8];
#pragma unroll
      for (int e = 0; e < kSpE; ++e) {
        const int64_t o = o0 + e * nt < len ? o0 + e * nt : o0;  // re-read, not stored
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int kk = k0 + k < n ? k0 + k : n - 1;  // re-read, not summed
          v[e][k] = __hip_atomic_load(src + kk * stride + o, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int e = 0; e < kSpE; ++e)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k0 + k < n) acc[e] += v[e][k];
    }
#pragma unroll
    for (int e = 0; e < kSpE; ++e) {
      const int64_t o = o0 + e * nt;
      if (o >= len) break;
      if (y)
        y[o] = bf16_rne(acc[e]);
      else
        __hip_atomic_store(dst + o, acc[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// This workgroup's arrival at counter c of `members`: true for the last one,
// which also resets the counter. Call after the workgroup's stores have been
// issued; all threads must call it.
__device__ __forceinline__ bool sp_arrive(unsigned int* c, unsigned int members) {
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int prev =
        __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == members - 1;
    if (last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return last;
}

template <int S, int P, int DQ, bool RES>
__global__ __launch_bounds__(64 * S) void k_decode_fused(
    const uint16_t* __restrict__ w_gu, const uint16_t* __restrict__ w_down,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, float eps,
    float* __restrict__ part, float* __restrict__ grp, uint16_t* __restrict__ y, int M, int d,
    int ff, int act, const uint16_t* __restrict__ res, uint16_t* __restrict__ hout) {
  constexpr int RB = 4;  // 4 x 16 W_gu rows = 32 gate/up pairs
  __shared__ f32x4 red[S * RB * 64];
  __shared__ float ssred[S * 16];
  __shared__ uint32_t abuf[2][16][17];  // [hi, lo][token][feature pair], padded
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp_l = lane >> 4;
  const int sl = blockIdx.x;
  f32x4 acc[RB][1];
  float ss[1];
  gemv_core<RES ? ACT_XR : ACT_X, 1, RB, S, P>(w_gu, nullptr, x, gamma, (int64_t)sl * RB, d, M, 0,
                                               d >> 5, acc, ss, d, 0, [] {}, [] {}, res,
                                               blockIdx.x == 0 ? hout : nullptr);

  // down tiles (row block wave + j*S, K unit sl), j < nt
  const int64_t tstride = (int64_t)(ff >> 5) * 512 * S;  // elements between a wave's tiles
  const int nbd = d >> 4;
  const int nt = wave < nbd ? (nbd - wave + S - 1) / S : 0;
  const uint16_t* wd = w_down + ((int64_t)wave * (ff >> 5) + sl) * 512 + lane * 8;
  u32x4 db[DQ];
#pragma unroll
  for (int q = 0; q < DQ; ++q)
    if (q < nt) db[q] = ld16_stream(wd + q * tstride);

  stash<RB, 1>(red, acc);
  {
    float v = ss[0];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < 16) ssred[wave * 16 + lane] = v;
  }
  __syncthreads();
  const float inv_d = 1.0f / (float)d;
  for (int o = threadIdx.x; o < 16 * 16; o += 64 * S) {
    const int pp = o & 15, t = o >> 4;  // features 2pp, 2pp+1 of the slice
    uint32_t h = 0u, l = 0u;
    if (t < M) {
      const int L0 = (t >> 2) * 16, e = t & 3;
      float sst = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s) sst += ssred[s * 16 + t];
      const float r = 1.0f / sqrtf(sst * inv_d + eps);
      float av[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int p = 2 * pp + k;
        const int rb = p >> 3, lr = (p & 7) * 2;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int base = (s * RB + rb) * 64 + L0 + lr;
          g += red[base][e];
          u += red[base + 1][e];
        }
        av[k] = act_mul(act, g * r, u * r);
      }
      split_bf16_pair(av[0], av[1], h, l);
    }
    abuf[0][t][pp] = h;
    abuf[1][t][pp] = l;
  }
  __syncthreads();
  // A operand: token col, features 8*grp_l .. 8*grp_l+7 of the slice
  u32x4 ah, al;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ah[i] = abuf[0][col][grp_l * 4 + i];
    al[i] = abuf[1][col][grp_l * 4 + i];
  }
  const int64_t md = (int64_t)M * d;
  float* pw = part + (int64_t)sl * md;
  for (int j0 = 0; j0 < nt; j0 += DQ) {
#pragma unroll
    for (int q = 0; q < DQ; ++q) {
      const int j = j0 + q;
      if (j < nt) {
        const u32x4 wv = db[q];
        if (j + DQ < nt) db[q] = ld16_stream(wd + (j + DQ) * tstride);
        f32x4 c = mfma_bf16(ah, wv, f32x4{0.f, 0.f, 0.f, 0.f});
        c = mfma_bf16(al, wv, c);
        const int row = (wave + j * S) * 16 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = grp_l * 4 + e;
          if (t < M)
            __hip_atomic_store(pw + (int64_t)t * d + row, c[e], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }

  // step 4: the two-level arrival-ordered, order-independent reduction
  const int nw = (int)gridDim.x, G = sp_group_size(nw), ng = (nw + G - 1) / G;
  const int g = sl / G, g0 = g * G, members = nw - g0 < G ? nw - g0 : G;
  if (!sp_arrive(&g_sp_count[g], (unsigned)members)) return;
  sp_sum(part + (int64_t)g0 * md, md, members, md, grp + (int64_t)g * md, nullptr);
  if (!sp_arrive(&g_sp_count[kSpMaxGroups], (unsigned)ng)) return;
  sp_sum(grp, md, ng, md, nullptr, y);
}

bool single_pass_auto(int64_t M, int64_t d, int64_t ff, int wtype) {
  (void)M, (void)d, (void)ff, (void)wtype;
  return false;
}

// Single-pass workspace: fp32 partial sums [ff/32, M, d] and group sums
// [ng, M, d] from the start of the workspace.
size_t fused_partial_bytes(int64_t M, int64_t d, int64_t ff) {
  const int nw = (int)(ff / 32), G = sp_group_size(nw), ng = (nw + G - 1) / G;
  return align256((size_t)nw * M * d * 4) + (size_t)ng * M * d * 4;
}

hipError_t launch_decode_fused(const Problem& p, hipStream_t stream) {
  const int nw = p.ff / 32;
  float* part = reinterpret_cast<float*>(p.ws);
  float* grp = reinterpret_cast<float*>(p.ws + align256((size_t)nw * p.M * p.d * 4));
  auto go = [&](auto kern) {
    launch_kernel(KK_DECODE_FUSED_BF16, kern, dim3(nw), dim3(64 * kFuS), 0, stream,
                  static_cast<const uint16_t*>(p.w_gu), static_cast<const uint16_t*>(p.w_down),
                  p.x, p.gamma, p.eps, part, grp, p.y, p.M, p.d, p.ff, p.act, p.res, p.hout);
  };
  if (p.res)
    go(k_decode_fused<kFuS, kFuP, kFuDq, true>);
  else
    go(k_decode_fused<kFuS, kFuP, kFuDq, false>);
  return hipGetLastError();
}

// ------------------------------------------------------------ launch

// Down projection with DRB row blocks and S waves per workgroup, K split
// `splits` ways across workgroups; activations staged in LDS when `lds`.
template <int WK, int NCB, int DRB, int S, bool STAGE>
static void launch_down(const Problem& p, const DecodeWs& ws, int splits, bool lds,
                        int64_t lds_bytes, hipStream_t stream) {
  constexpr int DP = WK == WK_INT4 ? kQ4P : kDnP;
  const int kind = WK == WK_INT4 ? KK_DECODE_DOWN_INT4 : KK_DECODE_DOWN_BF16;
  const dim3 grid(p.d / (16 * DRB), splits), block(64 * S);
  // int4 at M = 1: one accumulator row per lane holds the token
  constexpr int kEmax1 = WK == WK_INT4 ? 1 : 4;
  if (STAGE && lds && WK == WK_INT4 && p.M == 1)
    launch_kernel(kind, k_decode_down<WK, NCB, DRB, S, DP, STAGE, kEmax1>, grid, block,
                  (uint32_t)lds_bytes, stream, p.w_down, p.s_down, ws.a0, ws.a1, p.y, p.M, p.d,
                  p.ff, ws.part, ws.cnt);
  else if (STAGE && lds)
    launch_kernel(kind, k_decode_down<WK, NCB, DRB, S, DP, STAGE>, grid, block,
                  (uint32_t)lds_bytes, stream, p.w_down, p.s_down, ws.a0, ws.a1, p.y, p.M, p.d,
                  p.ff, ws.part, ws.cnt);
  else
    launch_kernel(kind, k_decode_down<WK, NCB, DRB, S, DP, false>, grid, block, 0, stream,
                  p.w_down, p.s_down, ws.a0, ws.a1, p.y, p.M, p.d, p.ff, ws.part, ws.cnt);
}

template <int WK, int NCB, int RB, int S>
static void launch_gateup_s(const Problem& p, const DecodeWs& ws, const uint16_t* act0,
                            const uint16_t* act1, int ncnt, bool lds, int64_t lds_bytes,
                            hipStream_t stream) {
  constexpr int GP = WK == WK_INT4 ? kQ4P : kGuP;
  constexpr bool kStage =
      NCB == 1 && (WK == WK_INT4 || WK == WK_BF16);
  const int kind = WK == WK_INT4 ? KK_DECODE_GATEUP_INT4 : KK_DECODE_GATEUP_BF16;
  // 2ff is a multiple of 64, so RB <= 4 divides the gate/up row blocks; a
  // larger RB is launched only where launch_decode_t checked that it does
  const dim3 grid((2 * p.ff) / (16 * RB)), block(64 * S);
  auto go = [&](auto kern, uint32_t shmem) {
    launch_kernel(kind, kern, grid, block, shmem, stream, p.w_gu, p.s_gu, act0, act1, p.eps, ws.a0,
                  ws.a1, p.M, p.d, p.ff, ws.cnt, ncnt, p.act, p.res, p.hout);
  };
  // the int4 path has added the residual in its prep kernel already
  // int4 at M = 1: one accumulator row per lane holds the token
  constexpr int kEmax1 = WK == WK_INT4 ? 1 : 4;
  if (kStage && lds && WK == WK_INT4 && p.M == 1)
    go(k_decode_gateup<WK, NCB, RB, S, GP, kStage, false, kEmax1>, (uint32_t)lds_bytes);
  else if (kStage && lds)
    go(k_decode_gateup<WK, NCB, RB, S, GP, kStage, false>, (uint32_t)lds_bytes);
  else if (WK == WK_BF16 && p.res)
    go(k_decode_gateup<WK, NCB, RB, S, GP, false, WK == WK_BF16>, 0);
  else
    go(k_decode_gateup<WK, NCB, RB, S, GP, false, false>, 0);
}

// Waves per workgroup: with many bf16 workgroups (Llama-8B-sized layers and
// up) fewer waves per CU stream faster (measured on MI355X: Llama-8B gate/up
// 44 -> 41 us at 4 waves, M = 1 and 4); Phi-3-sized layers, and int4 (whose
// 4-wave version measured 10 % slower), keep 8.
template <int WK, int NCB, int RB>
static void launch_gateup(const Problem& p, const DecodeWs& ws, const uint16_t* act0,
                          const uint16_t* act1, int ncnt, bool lds, int64_t lds_bytes,
                          hipStream_t stream) {
  if (WK != WK_INT4 && NCB == 1 && (2 * p.ff) / (16 * RB) >= kGuManyWgs)
    launch_gateup_s<WK, NCB, RB, kGuSMany>(p, ws, act0, act1, ncnt, lds, lds_bytes, stream);
  else
    launch_gateup_s<WK, NCB, RB, kGuS>(p, ws, act0, act1, ncnt, lds, lds_bytes, stream);
}

template <int WK, int NCB>
static hipError_t launch_decode_t(const Problem& p, hipStream_t stream) {
  const DecodeWs ws = decode_ws(p);
  constexpr int GRB = WK == WK_INT4 ? kQ4GuRb : kGuRb;
  constexpr int RB = (NCB == 1) ? GRB : (GRB > 2 ? 2 : GRB);
  constexpr int DRB = WK == WK_INT4 ? kQ4DnRb : kDnRb;
  constexpr bool kStage = NCB == 1 && WK == WK_INT4;
  constexpr bool kStageDn =
      NCB == 1 && WK == WK_INT4;
  hipError_t e;
  if constexpr (WK != WK_BF16) {
    launch_kernel(KK_ACT_PREP, k_act_prep<WK == WK_INT4>, dim3(p.M), dim3(512), 0, stream, p.x,
                  p.gamma, p.eps, ws.n0, p.d, p.res, p.hout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // bf16 reads x and gamma directly; the others read the prepared fp16 n
  const uint16_t* act0 = WK == WK_BF16 ? p.x : ws.n0;
  const uint16_t* act1 = WK == WK_BF16 ? p.gamma : nullptr;
  // Larger M: every K unit's activation loads (M tokens per wave) cost as
  // much as its weight loads, so more weight rows share them: bf16 gate/up
  // takes kBigGuRb row blocks per workgroup, and the down projection
  // kBigDnRb, split along K to keep enough workgroups.
  const bool big = p.M > kBigM;
  // down: BDRB row blocks per workgroup, split along K, from M > kBigDnM
  // (two tokens on: measured 4-10% faster down kernels at M = 2..4 on the
  // Phi-3, Llama-8B and 70B int4 shapes); otherwise DRB row blocks per
  // workgroup when they divide d and leave enough workgroups to cover the
  // CUs; else one, split along K when that helps
  constexpr int BDRB = kBigDnRb;
  const bool bdrb = p.M > kBigDnM && p.d % (16 * BDRB) == 0;
  const bool drb = !bdrb && DRB > 1 && p.d % (16 * DRB) == 0 && p.d / (16 * DRB) >= 256;
  const int dn_rb = bdrb ? BDRB : drb ? DRB : 1;
  const int splits = drb ? 1 : down_splits(p.d / (16 * dn_rb), p.ff, WK == WK_INT4);
  // Activations staged in LDS for small M, when they fit without lowering
  // the number of workgroups resident per CU (bytes per workgroup).
  // Measured on MI355X at M=1: int4 (70B shape) gains 13 % in gate/up and
  // 10 % in down; bf16 gate/up gains 3-4 % (Phi-3, Llama-8B), while bf16
  // down loses up to 14 %, so the bf16 down kernel reads its a per wave.
  auto lds_budget = [](int64_t wgs) -> int64_t { return wgs <= 256 ? 96 * 1024 : 32 * 1024; };
  constexpr int BGRB = NCB == 1 ? kBigGuRb : kBigGuRb2, BGRBW = kBigGuRb2w;
  constexpr int Q4B = kQ4BigGuRb;
  // int4 takes Q4B row blocks from M > kBigM up to 16 tokens (its
  // registers hold RB at two token blocks); bf16 / fp16 at two token blocks
  // take BGRBW instead of BGRB where that divides the row blocks and adds none
  // to the most any CU streams (rounds of 256 workgroups times row blocks):
  // measured 4-7% faster at Llama-8B M=17..32 (224 workgroups), while at
  // Phi-3 (128 of them) it would double the largest share
  // bf16 / fp16 also take BGRB from two tokens on where that still leaves
  // more than one round of workgroups (Llama-8B: 448; measured 3-20% faster
  // at M = 2..4, while at Phi-3's 256 it is slower)
  const int64_t gblocks = (2 * p.ff) / 16;
  const bool gu_big = WK == WK_INT4 ? big && NCB == 1
                                    : big || (p.M > 1 && gblocks / BGRB > 256);
  auto most_per_cu = [gblocks](int64_t rb) { return (gblocks / rb + 255) / 256 * rb; };
  const bool gu_wide = gu_big && WK != WK_INT4 && NCB == 2 && gblocks % BGRBW == 0 &&
                       most_per_cu(BGRBW) <= most_per_cu(BGRB);
  // small layers (a tensor-parallel share of ff): one row block per
  // workgroup where RB of them would leave CUs without a workgroup
  const bool gu_small = !gu_big && NCB == 1 && RB > 1 && gblocks / RB < 256;
  const int gu_rb = gu_wide ? BGRBW : gu_big ? (WK == WK_INT4 ? Q4B : BGRB) : gu_small ? 1 : RB;
  const int64_t gu_wgs = gblocks / gu_rb;
  const int64_t gu_lds = (int64_t)(WK == WK_BF16 ? 4 : 2) * p.M * p.d;
  // (bf16 gate/up staging, when enabled, does not cover the residual prologue)
  constexpr bool kStageGu =
      NCB == 1 && (WK == WK_INT4 || WK == WK_BF16);
  const bool gl = kStageGu && (WK == WK_INT4 || !p.res) && p.M <= kLdsMaxM &&
                  gu_lds <= lds_budget(gu_wgs);
  const int ukd = WK == WK_INT4 ? 128 : 32, nud = (p.ff + ukd - 1) / ukd;
  const int64_t dn_wgs = (p.d / (16 * dn_rb)) * splits;
  const int64_t dn_lds = (int64_t)(WK == WK_BF16 ? 4 : 2) * p.M * ((nud + splits - 1) / splits) * ukd;
  const bool dl = kStage && p.M <= kLdsMaxM && dn_lds <= lds_budget(dn_wgs);

  const int ncnt = splits > 1 ? (int)(p.d / 16) : 0;
  if (gu_wide) {
    if constexpr (WK != WK_INT4 && NCB == 2)
      launch_gateup<WK, NCB, BGRBW>(p, ws, act0, act1, ncnt, gl, gu_lds, stream);
  } else if (gu_big) {
    if constexpr (WK != WK_INT4)
      launch_gateup<WK, NCB, BGRB>(p, ws, act0, act1, ncnt, gl, gu_lds, stream);
    else if constexpr (NCB == 1)
      launch_gateup<WK, NCB, Q4B>(p, ws, act0, act1, ncnt, gl, gu_lds, stream);
  } else if (gu_small) {
    // and 16 waves: each wave then walks half as many K units, so fewer
    // load round trips in a row (Llama-8B's 8-way share, ff = 1792, M = 1:
    // gate/up 13.6 -> 9.9 us)
    if constexpr (NCB == 1)
      launch_gateup_s<WK, NCB, 1, 16>(p, ws, act0, act1, ncnt, gl, gu_lds, stream);
  } else {
    launch_gateup<WK, NCB, RB>(p, ws, act0, act1, ncnt, gl, gu_lds, stream);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (bdrb)
    // (int4 with two token blocks keeps 8 waves: its registers do not fit 16)
    launch_down<WK, NCB, BDRB, (NCB == 1 || WK == WK_INT4) ? kBigDnS : kBigDnS2,
                kStageDn>(p, ws, splits, dl, dn_lds, stream);
  else if (drb)
    launch_down<WK, NCB, DRB, (NCB == 2 && WK == WK_INT4) ? 8 : kDnS, kStageDn>(
        p, ws, splits, dl, dn_lds, stream);
  else if (splits == 1)
    launch_down<WK, NCB, 1, kDnS, kStageDn>(p, ws, splits, dl, dn_lds, stream);
  else  // split slices are short: 8 waves each, so that more of them are resident per CU
    launch_down<WK, NCB, 1, kDnSplitS, kStageDn>(p, ws, splits, dl, dn_lds, stream);
  return hipGetLastError();
}

hipError_t launch_decode(const Problem& p, hipStream_t stream) {
  if (p.wtype == 1)
    return p.M <= 16 ? launch_decode_t<WK_INT4, 1>(p, stream)
                     : launch_decode_t<WK_INT4, 2>(p, stream);
  if (p.wtype == 2)
    return p.M <= 16 ? launch_decode_t<WK_F16, 1>(p, stream)
                     : launch_decode_t<WK_F16, 2>(p, stream);
  if (p.M >= kH16MinM)
    return p.M <= 16 ? launch_decode_t<WK_BF16H, 1>(p, stream)
                     : launch_decode_t<WK_BF16H, 2>(p, stream);
  return p.M <= 16 ? launch_decode_t<WK_BF16, 1>(p, stream) : launch_decode_t<WK_BF16, 2>(p, stream);
}

}  // namespace fmlp
