// Decode path for int4 weights (symmetric, groups of 32 along K, fp16
// scales): the same two-kernel structure as the bf16 decode path, with the
// weights expanded in registers (the llama.cpp PR digest describes the
// gate/up + GLU fusion inside its quantised matmul; the format here is the
// library's own group-32 layout).
//
// Per 32-element group g of row r the kernels compute
//     z_r += s[r,g] * sum_k q[r,k] v[k]
// on MFMA 16x16x32 bf16 with the operands swapped relative to the bf16 path:
// A = activations (16 tokens x 32 k), B = weights (32 k x 16 rows), so each
// lane's four accumulators belong to ONE weight row and one scale per lane
// per group suffices, and only the accumulator slots of real tokens are
// scaled (one VALU op per group per lane at M <= 1).
//
// In-register expansion: a 32-bit word holds 8 codes. XOR with 0x88888888
// turns each two's-complement nibble into q + 8 in [0, 15]; OR-ing that into
// the mantissa of bf16 128.0 (0x4300) gives the exact bf16 value 136 + q.
// The constant offset is removed through the MFMA accumulator input:
// C = -136 * sum_k v[k], computed per group with one MFMA against a matrix of
// ones, so sum_k (136 + q_k) v_k + C = sum_k q_k v_k. The activation enters as
// an exact bf16 hi + lo pair (two MFMAs), as on the bf16 path.
//
// K-slot order inside one lane's 8 codes: word bits [4j, 4j+4) hold code
// k = 8*grp + j; extracting with shifts of 0, 4, 8, 12 and the mask
// 0x000F000F yields the pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7). The activation
// fragment is built in the same order.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace fmlp {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// 8 codes (one word) -> 4 words of bf16 pairs (136 + q), in (k0,k4)..(k3,k7) order.
__device__ __forceinline__ u32x4 int4_to_bf16_offset(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  u32x4 r;
  r[0] = (u & 0x000F000Fu) | 0x43004300u;
  r[1] = ((u >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((u >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((u >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 1.0 pair

// One group of 32 K for RB weight row blocks and NCB token blocks.
// act_hi/act_lo: activation fragments (tokens x k), permuted K order.
template <int RB, int NCB>
__device__ __forceinline__ void int4_group_mfma(const u32x4 (&act_hi)[NCB],
                                                const u32x4 (&act_lo)[NCB], const uint32_t (&qw)[RB],
                                                const float (&s)[RB], f32x4 (&acc)[RB][NCB],
                                                int jmax) {
  const u32x4 ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    // C = -136 * (sum_k v_k) for each token slot of this lane
    f32x4 vs = mfma_bf16(act_hi[cb], ones, f32x4{0.f, 0.f, 0.f, 0.f});
    vs = mfma_bf16(act_lo[cb], ones, vs);
    const f32x4 c = vs * -136.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const u32x4 wq = int4_to_bf16_offset(qw[rb]);
      f32x4 dq = mfma_bf16(act_hi[cb], wq, c);
      dq = mfma_bf16(act_lo[cb], wq, dq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < jmax) acc[rb][cb][j] = fmaf(s[rb], dq[j], acc[rb][cb][j]);
    }
  }
}

// ---------------------------------------------------------------------------
// gate/up (int4) + RMSNorm + SiLU*mul. Writes a_hi/a_lo [M, ff] with every
// aligned block of 8 stored in (k0,k4),(k1,k5),(k2,k6),(k3,k7) order, which
// is the fragment order the int4 down kernel consumes.
template <int NCB, int RB, int S>
__global__ __launch_bounds__(64 * S) void k_decode_gateup_int4(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, float eps,
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ sc, uint16_t* __restrict__ a_hi,
    uint16_t* __restrict__ a_lo, int M, int d, int ff) {
  __shared__ f32x4 red[S * RB * NCB * 64];
  __shared__ float ssred[S * NCB * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (RB * 16);
  const int nkb = d >> 5;
  const int jmax = M >= 4 ? 4 : M;

  const uint8_t* qrow[RB];
  const uint16_t* srow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t r = row0 + rb * 16 + col;
    qrow[rb] = q + r * (int64_t)(d / 2) + grp * 4;
    srow[rb] = sc + r * (int64_t)(d / 32);
  }
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
    ss[cb] = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int kb = wave;
  uint32_t qn[RB];
  uint16_t sn[RB];
  if (kb < nkb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      qn[rb] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(qrow[rb] + kb * 16));
      sn[rb] = srow[rb][kb];
    }
  }
  for (; kb < nkb; kb += S) {
    uint32_t qw[RB];
    float s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      qw[rb] = qn[rb];
      s[rb] = (float)__builtin_bit_cast(_Float16, sn[rb]);
    }
    if (kb + S < nkb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        qn[rb] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(qrow[rb] + (kb + S) * 16));
        sn[rb] = srow[rb][kb + S];
      }
    }
    const int k = kb * 32;
    const u32x4 gv = ld16(grow + k);
    u32x4 ah[NCB], al[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      u32x4 xv = {0u, 0u, 0u, 0u};
      if (tok[cb]) xv = ld16(xrow[cb] + k);
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = bf16_lo(xv[j]), x1 = bf16_hi(xv[j]);
        ss[cb] = fmaf(x0, x0, ss[cb]);
        ss[cb] = fmaf(x1, x1, ss[cb]);
        v[2 * j] = x0 * bf16_lo(gv[j]);
        v[2 * j + 1] = x1 * bf16_hi(gv[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h, l;
        split_bf16_pair(v[j], v[j + 4], h, l);
        ah[cb][j] = h;
        al[cb][j] = l;
      }
    }
    int4_group_mfma<RB, NCB>(ah, al, qw, s, acc, jmax);
  }

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

  // D layout (swapped operands): lane L holds rows (L % 16), tokens 4*(L/16)+e.
  constexpr int kPairs = RB * 8;
  const float inv_d = 1.0f / (float)d;
  for (int o = threadIdx.x; o < kPairs * NCB * 16; o += 64 * S) {
    const int p = o % kPairs, t = o / kPairs;
    if (t >= M) continue;
    const int cb = t >> 4, c = t & 15;
    const int rb = p >> 3, lr = (p & 7) * 2;
    const int L = (c >> 2) * 16 + lr, e = c & 3;
    float g = 0.f, u = 0.f, sst = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      g += red[((s * RB + rb) * NCB + cb) * 64 + L][e];
      u += red[((s * RB + rb) * NCB + cb) * 64 + L + 1][e];
      sst += ssred[(s * NCB + cb) * 16 + c];
    }
    const float r = 1.0f / sqrtf(sst * inv_d + eps);
    const float av = silu_mul(g * r, u * r);
    const uint16_t h = bf16_rne(av);
    const int i = (int)(row0 / 2) + p;  // logical index along ff
    const int ib = i & ~7, ii = i & 7;
    const int spos = ib + (ii < 4 ? 2 * ii : 2 * (ii - 4) + 1);
    const int64_t idx = (int64_t)t * ff + spos;
    a_hi[idx] = h;
    a_lo[idx] = bf16_rne(av - __uint_as_float((uint32_t)h << 16));
  }
}

// ---------------------------------------------------------------------------
// down projection (int4): y[t, j] = sum_i W_down[j, i] a[t, i].
template <int NCB, int RB, int S>
__global__ __launch_bounds__(64 * S) void k_decode_down_int4(
    const uint16_t* __restrict__ a_hi, const uint16_t* __restrict__ a_lo,
    const uint8_t* __restrict__ q, const uint16_t* __restrict__ sc, uint16_t* __restrict__ y,
    int M, int d, int ff) {
  __shared__ f32x4 red[S * RB * NCB * 64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (RB * 16);
  const int nkb = ff >> 5;
  const int jmax = M >= 4 ? 4 : M;

  const uint8_t* qrow[RB];
  const uint16_t* srow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t r = row0 + rb * 16 + col;
    qrow[rb] = q + r * (int64_t)(ff / 2) + grp * 4;
    srow[rb] = sc + r * (int64_t)(ff / 32);
  }
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
  uint32_t qn[RB];
  uint16_t sn[RB];
  if (kb < nkb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      qn[rb] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(qrow[rb] + kb * 16));
      sn[rb] = srow[rb][kb];
    }
  }
  for (; kb < nkb; kb += S) {
    uint32_t qw[RB];
    float s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      qw[rb] = qn[rb];
      s[rb] = (float)__builtin_bit_cast(_Float16, sn[rb]);
    }
    if (kb + S < nkb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        qn[rb] = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(qrow[rb] + (kb + S) * 16));
        sn[rb] = srow[rb][kb + S];
      }
    }
    const int k = kb * 32;
    u32x4 ah[NCB], al[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      ah[cb] = u32x4{0u, 0u, 0u, 0u};
      al[cb] = u32x4{0u, 0u, 0u, 0u};
      if (tok[cb]) {
        ah[cb] = ld16(ahr[cb] + k);
        al[cb] = ld16(alr[cb] + k);
      }
    }
    int4_group_mfma<RB, NCB>(ah, al, qw, s, acc, jmax);
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
    const int L = (c >> 2) * 16 + lr, e = c & 3;
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) sum += red[((s * RB + rb) * NCB + cb) * 64 + L][e];
    y[(int64_t)t * d + row0 + rl] = bf16_rne(sum);
  }
}

template <int NCB>
static hipError_t launch_decode_int4_t(const Problem& p, hipStream_t stream) {
  uint16_t* a_hi = reinterpret_cast<uint16_t*>(p.ws);
  uint16_t* a_lo = reinterpret_cast<uint16_t*>(p.ws + align256((size_t)p.M * p.ff * 2));
  constexpr int RB_GU = (NCB == 1) ? 4 : 2, S_GU = 8;
  constexpr int RB_D = 1, S_D = 16;
  {
    ProfileScope prof(KK_DECODE_GATEUP_INT4, stream);
    hipLaunchKernelGGL((k_decode_gateup_int4<NCB, RB_GU, S_GU>),
                       dim3((2 * p.ff) / (16 * RB_GU)), dim3(64 * S_GU), 0, stream, p.x, p.gamma,
                       p.eps, reinterpret_cast<const uint8_t*>(p.w_gu), p.s_gu, a_hi, a_lo, p.M,
                       p.d, p.ff);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProfileScope prof(KK_DECODE_DOWN_INT4, stream);
  hipLaunchKernelGGL((k_decode_down_int4<NCB, RB_D, S_D>), dim3(p.d / (16 * RB_D)),
                     dim3(64 * S_D), 0, stream, a_hi, a_lo,
                     reinterpret_cast<const uint8_t*>(p.w_down), p.s_down, p.y, p.M, p.d, p.ff);
  return hipGetLastError();
}

hipError_t launch_decode_int4(const Problem& p, hipStream_t stream) {
  if (p.M <= 16) return launch_decode_int4_t<1>(p, stream);
  return launch_decode_int4_t<2>(p, stream);
}

}  // namespace fmlp
