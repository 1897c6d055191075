// Prefill path (M > 32 tokens): the MLP is a dense contraction here, so it
// runs as two LDS-tiled MFMA GEMMs.
//
//   0. RMS pre-pass: n = fp16(gamma * x * r), r = 1/sqrt(mean(x^2) + eps)
//      (FastTPS review section 3, Figure 4 part1).
//   1. C = n W_gu^T on fp16 MFMA; the epilogue pairs interleaved columns
//      (gate 2i, up 2i+1) inside each lane and writes a = SiLU(g) * u as
//      fp16 (Figure 4 part2; the [M, 2ff] gate/up product never reaches HBM).
//   2. y = a W_down^T on fp16 MFMA, stored bf16 (Figure 4 part3).
//
// Operands are fp16 rather than bf16: rounding n to bf16 alone costs about
// 2e-2 max / 3.3e-3 mean relative error on Llama-8B-shaped layers, over the
// accuracy bar, while bf16 weights convert to fp16 exactly in the fp16 normal
// range and fp16 MFMA runs at the bf16 rate. Weights are converted while
// they are staged into LDS.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

#include <mutex>

namespace fmlp {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t prefill_workspace_bytes(int64_t M, int64_t d, int64_t ff) {
  // n fp16 [M, d], a fp16 [M, ff]
  return align256((size_t)M * d * 2) + align256((size_t)M * ff * 2);
}

// ---------------------------------------------------------------- RMS pre-pass
// One 256-thread workgroup per token row.
__global__ __launch_bounds__(256) void k_rms_prep_f16(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ gamma,
                                                      float eps, uint16_t* __restrict__ n, int d) {
  __shared__ float part[4];
  const int64_t m = blockIdx.x;
  const uint16_t* xr = x + m * d;
  uint16_t* nr = n + m * d;
  const int chunks = d >> 3;
  float ss = 0.f;
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 v = ld16(xr + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(v[j]), b = bf16_hi(v[j]);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const u32x4 v = ld16(xr + c * 8);
    const u32x4 g = ld16(gamma + c * 8);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(bf16_lo(v[j]) * bf16_lo(g[j]) * r);
      const _Float16 hi = (_Float16)(bf16_hi(v[j]) * bf16_hi(g[j]) * r);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    st16(nr + c * 8, o);
  }
}

// ---------------------------------------------------------------- GEMM
// C[f, t] = sum_k W[f, k] * Act[t, k]; W in the fragment-tiled bf16 layout
// (converted to fp16 on its way into LDS), Act fp16 [M, K] row-major.
//
// MFMA 32x32x16 f16: measured on MI355X it sustains ~2.0 PFLOP/s from a
// single wave per SIMD with two independent accumulators, where 16x16x32
// needs several waves and many chains to pass ~1.3 PFLOP/s.
// Operands: A = weights (32 rows x 16 K per fragment), B = activations
// (32 tokens x 16 K); lane l supplies row/token l % 32, K slots
// 8*(l/32) .. +7; the accumulator lane l holds column (token) l % 32 and
// rows 8i + 4*(l/32) + j in register 4i + j, so each lane owns whole
// gate/up pairs (rows 2p, 2p+1) for the SiLU*mul epilogue.
//
// Block tile BN features x BM tokens x 64 K, WGN x WGM waves each owning a
// (BN/WGN) x (BM/WGM) sub-tile. LDS holds both operands in fragment order
// (1 KB per 32 x 16 fragment, slot L at byte 16 L) in two stages; every MFMA
// operand read is one contiguous ds_read_b128 per wave. Weights pass through
// registers (bf16 -> fp16, and the 16 x 32 storage tile is re-cut into two
// 32 x 16 fragments); activations are loaded straight into LDS in fragment
// order (global_load_lds). Stage k+1 is filled while step k computes.
// Tiles are assigned XCD-major: each of the 8 XCDs takes a contiguous range
// of tile indices, token tiles fastest, so workgroups sharing a weight band
// run on the same XCD and share its L2.
enum { EPI_SILU_MUL_F16 = 0, EPI_STORE_BF16 = 1 };

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int NB, int MB, int WGN, int WGM>  // 32-row blocks per tile; wave grid
struct GemmCfg {
  static constexpr int W = WGN * WGM, THREADS = 64 * W;
  static constexpr int BN = NB * 32, BM = MB * 32;
  static constexpr int WNB = NB / WGN, WMB = MB / WGM;     // 32-row blocks per wave
  // per stage: NB*2 storage tiles of weights, MB*4 fragments of activations
  static constexpr int A_PER_T = NB * 2 * 2 / W, B_PER_T = MB * 4 / W;  // 16-byte chunks
  static constexpr int A_ELEMS = NB * 4 * 512, B_ELEMS = MB * 4 * 512;  // fp16 per stage
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr size_t LDS_BYTES = 2 * STAGE_ELEMS * 2;
  static_assert(A_PER_T >= 2 && A_PER_T % 2 == 0 && B_PER_T >= 4 && B_PER_T % 4 == 0, "tile");
};

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

// LDS fragment index of (32-row block, 16-column chunk q of the 64-column step).
__device__ __forceinline__ int frag_at(int blk32, int q) { return blk32 * 4 + q; }

template <int NB, int MB, int WGN, int WGM, int EPI>
__global__ __launch_bounds__(64 * WGN * WGM) void k_gemm_wf16(const uint16_t* __restrict__ Wt,
                                                              const uint16_t* __restrict__ Act,
                                                              uint16_t* __restrict__ out, int M,
                                                              int N, int K) {
  using C = GemmCfg<NB, MB, WGN, WGM>;
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WGN, wm = wave / WGN;

  const int nN = (N + C::BN - 1) / C::BN, nM = (M + C::BM - 1) / C::BM;
  const int T = nN * nM;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, idx = pid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int tn = tile / nM, tm = tile % nM;
  const int n0 = tn * C::BN, m0 = tm * C::BM;
  const int nkb = K >> 5, nrb = N >> 4;

  // Weight chunk i of a thread: storage tile (16-row block rbl, K block kbl),
  // slot = lane; rbl = W*(i >> 1) + wave, kbl = i & 1. Its 8 values (row r'
  // = lane % 16, columns 8*(lane/16) ..) land in fragment (rbl/2, 2 kbl +
  // lane/32), slot 32*((lane/16) % 2) + 16*(rbl % 2) + lane % 16.
  const uint16_t* wbase = Wt + (int64_t)(n0 >> 4) * nkb * 512;
  uint32_t woff[C::A_PER_T];
  int wdst[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int rbl = C::W * (i >> 1) + wave, kbl = i & 1;
    const int rbc = (n0 >> 4) + rbl < nrb ? rbl : nrb - 1 - (n0 >> 4);  // rows past N clamped
    woff[i] = (uint32_t)((rbc * nkb + kbl) * 512 + lane * 8);
    const int g = lane >> 4;
    wdst[i] = (frag_at(rbl >> 1, 2 * kbl + (g >> 1)) * 64 + 32 * (g & 1) + 16 * (rbl & 1) +
               (lane & 15)) * 8;
  }
  // Activation chunk i: fragment (token block tb = W*(i >> 2) + wave... ) see below;
  // fragment (tb, q) slot = lane covers token 32 tb + lane % 32, columns 16 q + 8 (lane/32).
  const uint16_t* abase = Act + (int64_t)m0 * K;
  uint32_t aoff[C::B_PER_T];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int f = C::W * i + wave;  // fragment index within the stage: tb = f / 4, q = f % 4
    int tl = (f >> 2) * 32 + (lane & 31);
    tl = m0 + tl < M ? tl : M - 1 - m0;  // tokens past M clamped
    aoff[i] = (uint32_t)(tl * K + (f & 3) * 16 + (lane >> 5) * 8);
  }

  f32x16 acc[C::WNB][C::WMB];
#pragma unroll
  for (int i = 0; i < C::WNB; ++i)
#pragma unroll
    for (int j = 0; j < C::WMB; ++j) acc[i][j] = f32x16{};

  const int nkt = (nkb + 1) >> 1;
  u32x4 rw[C::A_PER_T];
  // weights of step kt -> registers (K block kb + 1 may not exist on the last step)
  auto a_load = [&](int kt) {
    const int kb = kt * 2;
    const bool full = kb + 1 < nkb;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      rw[i] = ((i & 1) == 0 || full) ? ld16(wbase + woff[i] + kb * 512) : u32x4{0u, 0u, 0u, 0u};
  };
  // registers -> LDS stage, bf16 -> fp16, re-cut into 32 x 16 fragments
  auto a_store = [&](int stage) {
    uint16_t* sA = lds + stage * C::STAGE_ELEMS;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      u32x4 h;
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = bf16x2_to_f16x2(rw[i][j]);
      *reinterpret_cast<u32x4*>(&sA[wdst[i]]) = h;
    }
  };
  // activations of step kt -> LDS stage directly; a missing last K block
  // (fragments q = 2, 3) is zero-filled from registers instead
  auto b_load = [&](int kt, int stage) {
    const int kb = kt * 2;
    const bool full = kb + 1 < nkb;
    uint16_t* sB = lds + stage * C::STAGE_ELEMS + C::A_ELEMS;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int f = C::W * i + wave;
      uint16_t* dst = &sB[f * 512];
      if ((f & 3) < 2 || full)
        __builtin_amdgcn_global_load_lds((gptr_t)(abase + aoff[i] + kb * 32), (lptr_t)dst, 16, 0, 0);
      else
        *reinterpret_cast<u32x4*>(dst + lane * 8) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // prologue: stage 0 <- step 0; registers <- weights of step 1
  a_load(0);
  b_load(0, 0);
  a_store(0);
  if (nkt > 1) a_load(1);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    // stage nxt was released by the last barrier: fill it for step kt+1 while
    // this step computes; the weights of step kt+2 start loading right away
    if (kt + 1 < nkt) {
      a_store(nxt);
      if (kt + 2 < nkt) a_load(kt + 2);
      b_load(kt + 1, nxt);
    }
    const uint16_t* sA = lds + cur * C::STAGE_ELEMS;
    const uint16_t* sB = sA + C::A_ELEMS;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4 af[C::WNB], bf[C::WMB];
#pragma unroll
      for (int i = 0; i < C::WNB; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&sA[frag_at(wn * C::WNB + i, q) * 512 + lane * 8]);
#pragma unroll
      for (int j = 0; j < C::WMB; ++j)
        bf[j] = *reinterpret_cast<const u32x4*>(&sB[frag_at(wm * C::WMB + j, q) * 512 + lane * 8]);
#pragma unroll
      for (int i = 0; i < C::WNB; ++i)
#pragma unroll
        for (int j = 0; j < C::WMB; ++j) acc[i][j] = mfma32_f16(af[i], bf[j], acc[i][j]);
    }
    // stage nxt complete (direct loads and this wave's writes) before the barrier
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  // epilogue: lane holds token t = col of block (i, j) and rows 8r + 4 grp + e
  const int col = lane & 31, grp = lane >> 5;
#pragma unroll
  for (int i = 0; i < C::WNB; ++i) {
#pragma unroll
    for (int j = 0; j < C::WMB; ++j) {
      const int t = m0 + (wm * C::WMB + j) * 32 + col;
      if (t >= M) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f0 = n0 + (wn * C::WNB + i) * 32 + 8 * r + 4 * grp;
        if (f0 >= N) continue;
        const float v0 = acc[i][j][4 * r], v1 = acc[i][j][4 * r + 1];
        const float v2 = acc[i][j][4 * r + 2], v3 = acc[i][j][4 * r + 3];
        if (EPI == EPI_SILU_MUL_F16) {
          const _Float16 a0 = (_Float16)silu_mul(v0, v1);
          const _Float16 a1 = (_Float16)silu_mul(v2, v3);
          const uint32_t packed = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          *reinterpret_cast<uint32_t*>(out + (int64_t)t * (N / 2) + f0 / 2) = packed;
        } else {
          uint32_t* dst = reinterpret_cast<uint32_t*>(out + (int64_t)t * N + f0);
          dst[0] = pack_bf16_rne(v0, v1);
          dst[1] = pack_bf16_rne(v2, v3);
        }
      }
    }
  }
}

// Launch one GEMM with a given block tile and wave grid.
template <int NB, int MB, int WGN, int WGM, int EPI>
static hipError_t launch_gemm_t(const uint16_t* W, const uint16_t* Act, uint16_t* out, int M,
                                int N, int K, hipStream_t stream) {
  using C = GemmCfg<NB, MB, WGN, WGM>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_wf16<NB, MB, WGN, WGM, EPI>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
  launch_kernel(EPI == EPI_SILU_MUL_F16 ? KK_GEMM_GATEUP : KK_GEMM_DOWN,
                k_gemm_wf16<NB, MB, WGN, WGM, EPI>, dim3(tiles), dim3(C::THREADS),
                (uint32_t)C::LDS_BYTES, stream, W, Act, out, M, N, K);
  return hipGetLastError();
}

// Estimated cost of a tile choice: waves of workgroups (one workgroup per CU
// for the large tiles, two for 128 x 128) times the time of one tile, which
// grows with its area and with the workgroups sharing a CU, discounted by how
// well the tile size feeds the matrix cores.
static double gemm_cost(int M, int N, int bn, int bm, double eff, int per_cu) {
  const int tiles = ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
  const int slots = 256 * per_cu;
  const int waves = (tiles + slots - 1) / slots;
  return (double)waves * bn * bm * per_cu / eff;
}

#ifndef FMLP_GEMM_TILE
#define FMLP_GEMM_TILE 0  // 0: by cost; 1: 256x256 4 waves; 2: 128x256; 3: 128x128; 4: 256x256 8 waves
#endif

template <int EPI>
static hipError_t launch_gemm(const uint16_t* W, const uint16_t* Act, uint16_t* out, int M, int N,
                              int K, hipStream_t stream) {
  if (FMLP_GEMM_TILE == 1) return launch_gemm_t<8, 8, 2, 2, EPI>(W, Act, out, M, N, K, stream);
  if (FMLP_GEMM_TILE == 2) return launch_gemm_t<4, 8, 2, 2, EPI>(W, Act, out, M, N, K, stream);
  if (FMLP_GEMM_TILE == 3) return launch_gemm_t<4, 4, 2, 2, EPI>(W, Act, out, M, N, K, stream);
  if (FMLP_GEMM_TILE == 4) return launch_gemm_t<8, 8, 2, 4, EPI>(W, Act, out, M, N, K, stream);
  const double c256 = gemm_cost(M, N, 256, 256, 1.0, 1);
  const double c128n = gemm_cost(M, N, 128, 256, 0.85, 1);
  const double c128 = gemm_cost(M, N, 128, 128, 0.7, 2);
  if (c256 <= c128n && c256 <= c128)
    return launch_gemm_t<8, 8, 2, 4, EPI>(W, Act, out, M, N, K, stream);
  if (c128n <= c128) return launch_gemm_t<4, 8, 2, 2, EPI>(W, Act, out, M, N, K, stream);
  return launch_gemm_t<4, 4, 2, 2, EPI>(W, Act, out, M, N, K, stream);
}

hipError_t launch_prefill(const Problem& p, hipStream_t stream) {
  if (p.wtype != 0) return hipErrorNotSupported;
  uint16_t* n = reinterpret_cast<uint16_t*>(p.ws);
  uint16_t* a = reinterpret_cast<uint16_t*>(p.ws + align256((size_t)p.M * p.d * 2));
  launch_kernel(KK_RMS_PREP, k_rms_prep_f16, dim3(p.M), dim3(256), 0, stream, p.x, p.gamma, p.eps,
                n, p.d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_gemm<EPI_SILU_MUL_F16>(reinterpret_cast<const uint16_t*>(p.w_gu), n, a, p.M, 2 * p.ff,
                                    p.d, stream);
  if (e != hipSuccess) return e;
  return launch_gemm<EPI_STORE_BF16>(reinterpret_cast<const uint16_t*>(p.w_down), a, p.y, p.M,
                                     p.d, p.ff, stream);
}

}  // namespace fmlp
