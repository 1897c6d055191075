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
// int4 weights: a pre-pass dequantises both matrices into fp16 in the same
// fragment-tiled geometry (w = s*q, exact in fp32, rounded once to fp16:
// relative error <= 2^-11, far inside the accuracy bar), and the GEMMs read
// those fp16 tiles without conversion.
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
#include <type_traits>

#ifndef FMLP_SETPRIO
#define FMLP_SETPRIO 0  // raise the wave priority over each sub-step's MFMA block (no gain with the
                        // reads hoisted to the sub-step's top; +1% before)
#endif

namespace fmlp {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// GEMM activations (the normalised input n and the SiLU*mul product a) live
// in the workspace "fragment-tiled": for token block tb (32 tokens) and
// column block kb (32 columns) two 1 KB MFMA fragments q = 0, 1 of 32 tokens
// x 16 columns; slot s of a fragment holds token 32 tb + s % 32, columns
// 32 kb + 16 q + 8 (s / 32) .. +7. A wave then loads any operand fragment as
// one contiguous 1 KB burst. Token blocks are padded to 32 tokens; the
// padding slots are never read into a stored output.
__device__ __forceinline__ int64_t act_tile_off(int t, int k, int K) {
  const int tb = t >> 5, kb = k >> 5, q = (k >> 4) & 1, slot = ((k >> 3) & 1) * 32 + (t & 31);
  return (((int64_t)tb * (K >> 5) + kb) * 2 + q) * 512 + slot * 8 + (k & 7);
}

static inline int64_t pad32(int64_t m) { return (m + 31) & ~(int64_t)31; }

// ---------------------------------------------------------------- RMS pre-pass
// (a) r_t = 1/sqrt(mean(x_t^2) + eps), one wave per token.
__global__ __launch_bounds__(256) void k_rms_scale(const uint16_t* __restrict__ x, float eps,
                                                   float* __restrict__ r, int M, int d,
                                                   const uint16_t* __restrict__ res) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= M) return;
  const uint16_t* xr = x + (int64_t)t * d;
  const uint16_t* rr = res ? res + (int64_t)t * d : nullptr;
  const int nch = d >> 3;
  // kU chunks per lane in flight at once (one load, then its wait, per
  // chunk would serialise the row's memory latency)
  constexpr int kU = 8;
  float ss = 0.f;
  for (int c0 = lane; c0 < nch; c0 += 64 * kU) {
    u32x4 v[kU], rv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + u * 64;
      v[u] = c < nch ? ld16(xr + c * 8) : u32x4{0u, 0u, 0u, 0u};
      if (rr) rv[u] = c < nch ? ld16(rr + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const u32x4 w = rr ? add_bf16x8(v[u], rv[u]) : v[u];  // residual stream
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) r[t] = 1.0f / sqrtf(ss / (float)d + eps);
}

// (b) n = fp16(gamma * x * r) in the fragment-tiled layout, one 16-byte slot
// per thread (consecutive threads write consecutive slots). Slots of padding
// tokens get the last token's values (finite, never stored).
__global__ __launch_bounds__(256) void k_rms_tile(const uint16_t* __restrict__ x,
                                                  const uint16_t* __restrict__ gamma,
                                                  const float* __restrict__ r,
                                                  uint16_t* __restrict__ n, int M, int d,
                                                  int64_t slots, const uint16_t* __restrict__ res,
                                                  uint16_t* __restrict__ hout) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= slots) return;
  const int slot = (int)(g & 63);
  const int64_t frag = g >> 6;                       // = tb * (d/16) + f
  const int fpb = d >> 4;                            // fragments per token block
  const int tb = (int)(frag / fpb), f = (int)(frag - (int64_t)tb * fpb);
  const int t0 = tb * 32 + (slot & 31);
  const int t = t0 < M ? t0 : M - 1;  // padding tokens repeat the last one
  const int k = (f >> 1) * 32 + (f & 1) * 16 + (slot >> 5) * 8;
  u32x4 v = ld16(x + (int64_t)t * d + k);
  if (res) {  // the residual stream h = bf16_rne(x + res), stored once per element
    v = add_bf16x8(v, ld16(res + (int64_t)t * d + k));
    if (t0 < M) st16(hout + (int64_t)t * d + k, v);
  }
  const u32x4 gm = ld16(gamma + k);
  const float rt = r[t];
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const _Float16 lo = (_Float16)(bf16_lo(v[j]) * bf16_lo(gm[j]) * rt);
    const _Float16 hi = (_Float16)(bf16_hi(v[j]) * bf16_hi(gm[j]) * rt);
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  st16(n + g * 8, o);
}

// ---------------------------------------------------------------- int4 -> fp16 tiles
// One thread per 16-byte chunk of the output (8 weights of one row): chunk
// (tile, slot) of the fragment-tiled layout holds row 16*rb + slot%16,
// columns 32*kb + 8*(slot/16) .. +7, tile = rb*(K/32) + kb. Its codes are one
// word of the int4 super-tile of (rb, kb/4), its scale one fp16.
__global__ __launch_bounds__(256) void k_dequant_f16_tiled(const uint32_t* __restrict__ qt,
                                                           const uint16_t* __restrict__ st,
                                                           int64_t R, int64_t K,
                                                           uint16_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;  // output chunk
  const int64_t nkb = K >> 5, nq = (K + 127) >> 7;
  if (c >= (R >> 4) * nkb * 64) return;
  const int slot = (int)(c & 63);
  const int64_t tile = c >> 6, rb = tile / nkb, kb = tile - rb * nkb;
  const int64_t stile = rb * nq + (kb >> 2);
  const uint32_t word = qt[stile * 256 + slot * 4 + (kb & 3)];
  const float s = (float)__builtin_bit_cast(
      _Float16, st[stile * 64 + (slot & 15) * 4 + (kb & 3)]);
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q0 = (int)((word >> (8 * j)) << 28) >> 28;      // code 2j (low nibble)
    const int q1 = (int)((word >> (8 * j + 4)) << 28) >> 28;  // code 2j+1
    const _Float16 w0 = (_Float16)(s * (float)q0), w1 = (_Float16)(s * (float)q1);
    o[j] = (uint32_t)__builtin_bit_cast(uint16_t, w0) |
           ((uint32_t)__builtin_bit_cast(uint16_t, w1) << 16);
  }
  st16(out + c * 8, o);
}

// ---------------------------------------------------------------- GEMM
// C[f, t] = sum_k W[f, k] * Act[t, k]; W in the fragment-tiled bf16 layout,
// Act fp16 in the fragment-tiled activation layout above.
//
// MFMA 32x32x16 f16: measured on MI355X it sustains ~2.0 PFLOP/s from a
// single wave per SIMD with independent accumulators, where 16x16x32 needs
// several waves and many chains to pass ~1.3 PFLOP/s.
// Operands: A = weights (32 rows x 16 K per fragment), B = activations
// (32 tokens x 16 K); lane l supplies row/token l % 32, K slots
// 8*(l/32) .. +7; the accumulator lane l holds column (token) l % 32 and
// rows 8i + 4*(l/32) + j in register 4i + j, so each lane owns whole
// gate/up pairs (rows 2p, 2p+1) for the SiLU*mul epilogue.
//
// Block tile BN features x BM tokens on a WGN x WGM grid of 4 or 8 waves,
// each owning a (BN/WGN) x (BM/WGM) sub-tile; one K step is one 32-column
// block. Both operands go from memory straight into LDS (buffer loads with
// the LDS-DMA bit, 16 bytes per lane, no register staging and no LDS writes
// by the waves), each wave instruction one contiguous 1 KB: the weights as
// their bf16 16 x 32 storage tiles, the activations as their fragments. The
// LDS is a ring of 5 stages (160 KB at 256 x 256), so the loads of step
// kt+4 are issued while step kt computes: four steps of MFMA work hide the
// memory latency.
//
// Each step has two 16-column sub-steps. Fragments are read one sub-step
// ahead into two register sets; a weight fragment gathers rows 0-15 and
// 16-31 from two storage tiles (each 16-lane group reads 256 contiguous
// bytes: no bank conflicts) and is converted bf16 -> fp16 in registers just
// before its MFMAs (exact in the fp16 normal range). Before the second
// sub-step's MFMAs each wave waits only for step kt+1's loads (vector memory
// counts retire in issue order, so later steps' loads stay in flight), meets
// the barrier, and reads step kt+1's first fragments under those MFMAs.
// Within a sub-step the LDS reads issue first and the conversions are spread
// between the MFMAs (sched_group_barrier), in the matrix pipe's shadow.
//
// Tiles are assigned XCD-major: each of the 8 XCDs takes a contiguous range
// of tile indices, token tiles fastest, so workgroups sharing a weight band
// run on the same XCD and share its L2.
// Epilogues: SiLU*mul (or a GELU form) to the fp16 tiled activations
// (gate/up), bf16 y, or an fp32 split-K partial (slice blockIdx.y of
// [splits, M, N]). The three gate epilogues differ only in the activation,
// which is a compile-time constant: a runtime choice inlines every
// activation at each of the unrolled output sites and triples the kernel's
// code.
enum {
  EPI_SILU_MUL_F16 = 0,
  EPI_STORE_BF16 = 1,
  EPI_STORE_F32 = 2,
  EPI_GELU_TANH_MUL_F16 = 3,
  EPI_GELU_ERF_MUL_F16 = 4
};
constexpr bool epi_gate(int epi) {
  return epi == EPI_SILU_MUL_F16 || epi == EPI_GELU_TANH_MUL_F16 || epi == EPI_GELU_ERF_MUL_F16;
}
constexpr int epi_act(int epi) {  // enum fmlp_activation
  return epi == EPI_GELU_TANH_MUL_F16 ? 1 : epi == EPI_GELU_ERF_MUL_F16 ? 2 : 0;
}

typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int NB, int MB, int WGN_, int WGM_>  // 32-row blocks per tile; wave grid
struct GemmCfg {
  static constexpr int WGN = WGN_, WGM = WGM_, W = WGN * WGM, THREADS = 64 * W;
  static constexpr int BN = NB * 32, BM = MB * 32;
  static constexpr int WNB = NB / WGN, WMB = MB / WGM;  // 32-row blocks per wave
  // 16-byte chunks per thread and step: weights 2*NB storage tiles of 1 KB,
  // activations 2*MB fragments of 1 KB
  static constexpr int A_PER_T = NB * 2 / W, B_PER_T = MB * 2 / W, LD_PER_T = A_PER_T + B_PER_T;
  static constexpr int A_ELEMS = NB * 1024, B_ELEMS = MB * 1024;  // 16-bit elements per stage
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int STAGES = 5;
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_ELEMS * 2;
  // one wave per SIMD when the accumulators alone fill 256 registers
  static constexpr int WAVES_PER_EU = (WNB * WMB >= 16) ? 1 : 2;
  static_assert((W == 4 || W == 8) && WNB >= 1 && WMB >= 1 && A_PER_T * W == NB * 2 &&
                B_PER_T * W == MB * 2, "tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(3 * LD_PER_T < 64, "vmcnt field");
};

typedef void __attribute__((address_space(3)))* lptr_t;

// Buffer descriptor word 3 for CDNA raw (unswizzled, stride 0) buffers: a
// 32-bit data format; the extent (num_records) is in bytes.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ int buf_extent(int64_t bytes) {
  return bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
}
// One 16-byte-per-lane LDS DMA through a raw buffer descriptor over
// [base, base + extent): lane l's 16 bytes at byte offset voff + soff land at
// dst + 16 l. (The descriptor is built here, not in the kernel body: its
// loop-invariant scalar setup is hoisted by the compiler.)
__device__ __forceinline__ void buf_load_lds16(const uint16_t* base, int extent, lptr_t dst,
                                               int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, extent, kBufWord3),
      dst, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate for vmcnt(vm) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] |
// expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]). The builtin, unlike
// inline asm, is seen by the compiler's own wait insertion, which then adds
// no redundant waits.
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | 0x70 | ((vm >> 4) << 14); }

// AF16: the weight tiles already hold fp16 (dequantised int4), no conversion.
template <int NB, int MB, int WGN, int WGM, int EPI, bool AF16>
__global__ __launch_bounds__(64 * WGN * WGM) __attribute__((amdgpu_waves_per_eu(
    GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU, GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU))) void
k_gemm_wf16(const uint16_t* __restrict__ Wt, const uint16_t* __restrict__ Act,
            void* __restrict__ out, int M, int N, int K, int n_begin, int n_end) {
  using C = GemmCfg<NB, MB, WGN, WGM>;
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wn = wave % C::WGN, wm = wave / C::WGN;

  // this launch covers feature rows n_begin .. n_end-1 of the N
  const int nN = (n_end - n_begin + C::BN - 1) / C::BN, nM = (M + C::BM - 1) / C::BM;
  const int T = nN * nM;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, idx = pid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + idx;
  const int tn = tile / nM, tm = tile % nM;
  const int n0 = n_begin + tn * C::BN, m0 = tm * C::BM;
  // split K: slice blockIdx.y of gridDim.y equal slices of 32-column blocks
  const int nkb = K >> 5, nrb = N >> 4;
  const int nkt = nkb / (int)gridDim.y, kbeg = (int)blockIdx.y * nkt;

  // Both operands are read through buffer descriptors based at this tile's
  // first weight row block and first token block (from its K slice start),
  // so every byte offset fits 32 bits whatever the matrix sizes; a lane's
  // offset is fixed and each K step adds one scalar offset. Reads past a
  // descriptor's extent would return zeros rather than fault (all reads
  // here are in range: row and token blocks are clamped below).
  //
  // Weight chunk i of a thread: 16-row storage tile rb = W*i + wave of the
  // tile (rows past N clamped), slot = lane; its LDS image sits at rb * 1 KB.
  const int rb0 = n0 >> 4;
  const uint16_t* wbase = Wt + ((int64_t)rb0 * nkb + kbeg) * 512;
  const int wext = buf_extent(((int64_t)nrb * nkb - ((int64_t)rb0 * nkb + kbeg)) * 1024);
  int woff[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int rb = C::W * i + wave;
    const int rbc = rb0 + rb < nrb ? rb : nrb - 1 - rb0;
    woff[i] = rbc * nkb * 1024 + lane * 16;
  }
  // Activation chunk i: fragment f = W*i + wave of the stage (token block
  // f/2 of the tile, half q = f%2), one contiguous 1 KB fragment of the tiled
  // activations (token blocks past the last one clamped to it).
  const int ntb = (M + 31) >> 5, tb0 = m0 >> 5;
  const uint16_t* abase = Act + ((int64_t)tb0 * nkb + kbeg) * 1024;
  const int aext = buf_extent(((int64_t)ntb * nkb - ((int64_t)tb0 * nkb + kbeg)) * 2048);
  int aoff[C::B_PER_T];
#pragma unroll
  for (int i = 0; i < C::B_PER_T; ++i) {
    const int f = C::W * i + wave;
    const int tb = tb0 + (f >> 1) < ntb ? (f >> 1) : ntb - 1 - tb0;
    aoff[i] = (tb * nkb * 2 + (f & 1)) * 1024 + lane * 16;
  }
  // LDS element offsets of this lane's fragment reads (within a stage): the
  // weight fragment of 32-row block b, half q gathers storage tiles 2b
  // (lanes 0-15, 32-47) and 2b+1 (lanes 16-31, 48-63), slots (2q + l/32)*16 + l%16.
  const int a_rd = (((lane >> 4) & 1) * 512) + (((lane >> 5) * 16 + (lane & 15)) * 8);
  const int b_rd = C::A_ELEMS + lane * 8;

  f32x16 acc[C::WNB][C::WMB];
#pragma unroll
  for (int i = 0; i < C::WNB; ++i)
#pragma unroll
    for (int j = 0; j < C::WMB; ++j) acc[i][j] = f32x16{};

  // the loads of step kt into stage st: weights, then activations
  auto load_a = [&](int kt, int st) __attribute__((always_inline)) {
    uint16_t* base = lds + st * C::STAGE_ELEMS;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i)
      buf_load_lds16(wbase, wext, (lptr_t)(base + (C::W * i + wave) * 512), woff[i], kt * 1024);
  };
  auto load_b = [&](int kt, int st) __attribute__((always_inline)) {
    uint16_t* base = lds + st * C::STAGE_ELEMS + C::A_ELEMS;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      buf_load_lds16(abase, aext, (lptr_t)(base + (C::W * i + wave) * 512), aoff[i], kt * 2048);
  };
  auto load_step = [&](int kt, int st) __attribute__((always_inline)) {
    load_a(kt, st);
    load_b(kt, st);
  };

  u32x4 fa[2][C::WNB], fb[2][C::WMB];
  auto frag_load_a = [&](int buf, int st, int q) __attribute__((always_inline)) {
    const uint16_t* base = lds + st * C::STAGE_ELEMS;
#pragma unroll
    for (int i = 0; i < C::WNB; ++i)
      fa[buf][i] = *reinterpret_cast<const u32x4*>(
          &base[a_rd + (wn * C::WNB + i) * 1024 + q * 256]);
  };
  auto frag_load_b = [&](int buf, int st, int q) __attribute__((always_inline)) {
    const uint16_t* base = lds + st * C::STAGE_ELEMS;
#pragma unroll
    for (int j = 0; j < C::WMB; ++j)
      fb[buf][j] = *reinterpret_cast<const u32x4*>(
          &base[b_rd + ((wm * C::WMB + j) * 2 + q) * 512]);
  };
  auto frag_load = [&](int buf, int st, int q) __attribute__((always_inline)) {
    frag_load_a(buf, st, q);
    frag_load_b(buf, st, q);
  };
  // the same reads, weights strictly first, all issued before what follows
  auto frag_load_ordered = [&](int buf, int st, int q) __attribute__((always_inline)) {
    frag_load_a(buf, st, q);
    __builtin_amdgcn_sched_barrier(0);
    frag_load_b(buf, st, q);
    __builtin_amdgcn_sched_barrier(0);
  };
  // weight fragments bf16 -> fp16 in place (after their LDS reads land)
  auto convert = [&](int buf) __attribute__((always_inline)) {
    if constexpr (!AF16) {
#pragma unroll
      for (int i = 0; i < C::WNB; ++i) fa[buf][i] = bf16x8_to_f16x8(fa[buf][i]);
    }
  };
  auto mma = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::WNB; ++i)
#pragma unroll
      for (int j = 0; j < C::WMB; ++j) acc[i][j] = mfma32_f16(fa[buf][i], fb[buf][j], acc[i][j]);
  };
  // Schedule of one sub-step: all fragment reads of the other register set
  // issue at its top (weights first, in program order), then the MFMAs, with
  // the conversions of the new weight fragments spread over the second half.
  // A conversion then waits only for its own weight read (the LDS DMA is a
  // buffer load, counted on vmcnt alone, so the LDS waits stay exact), issued
  // half a sub-step earlier. (Measured 1.5-4% faster than spreading the reads
  // over the MFMAs.)
  // kSpread: the sub-step's NL LDS-DMA loads go between its MFMAs rather
  // than in a burst at its top (8-wave tiles: gate/up 0.5-1.3% faster; the
  // 4-wave down tile measured mixed, so it keeps the burst).
  constexpr bool kSpread = C::W == 8;
  auto interleave = [&](auto nl_c) __attribute__((always_inline)) {
    constexpr int NMF = C::WNB * C::WMB;
    constexpr int NV = AF16 ? 0 : C::WNB * 12, HALF = NMF / 2;
    constexpr int NL = kSpread ? decltype(nl_c)::value : 0;
    constexpr int LS = NMF / (NL > 0 ? NL : 1) > 0 ? NMF / (NL > 0 ? NL : 1) : 1;  // MFMAs per load
#pragma unroll
    for (int g = 0; g < NMF; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);               // MFMA
      if (NL > 0 && g % LS == 0 && g / LS < NL)
        __builtin_amdgcn_sched_group_barrier(0x0020, 1, 0);             // VMEM (LDS DMA)
      if (NV > 0 && g >= HALF)
        __builtin_amdgcn_sched_group_barrier(0x0002, (NV + HALF - 1) / HALF, 0);  // VALU
    }
  };

  // prologue: steps 0..3 -> stages 0..3; wait for step 0; its first fragments
  const int npre = nkt < 4 ? nkt : 4;
  for (int s = 0; s < npre; ++s) load_step(s, s);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
  frag_load(0, 0, 0);
  convert(0);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));

  // steady state: step kt computes from stage kt % 5 while step kt+4 loads
  // into stage (kt+4) % 5, which step kt-1 released at its barrier
  // Step kt+4's weights load during the first sub-step and its activations
  // during the second, so at the barrier (between them) the loads issued
  // after step kt+1's are those of steps kt+2, kt+3 and kt+4's weights.
  int kt = 0, st = 0;
  for (; kt + 4 < nkt; ++kt) {
    const int st1 = st == 4 ? 0 : st + 1, st4 = st == 0 ? 4 : st - 1;
    if (!kSpread) load_a(kt + 4, st4);
    if (FMLP_SETPRIO) __builtin_amdgcn_s_setprio(1);
    frag_load_ordered(1, st, 1);
    if (kSpread) load_a(kt + 4, st4);
    mma(0);
    convert(1);
    interleave(std::integral_constant<int, C::A_PER_T>{});
    __builtin_amdgcn_sched_barrier(0);
    if (FMLP_SETPRIO) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * C::LD_PER_T + C::A_PER_T));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (!kSpread) load_b(kt + 4, st4);
    if (FMLP_SETPRIO) __builtin_amdgcn_s_setprio(1);
    frag_load_ordered(0, st1, 0);
    if (kSpread) load_b(kt + 4, st4);
    mma(1);
    convert(0);
    interleave(std::integral_constant<int, C::B_PER_T>{});
    __builtin_amdgcn_sched_barrier(0);
    if (FMLP_SETPRIO) __builtin_amdgcn_s_setprio(0);
    // (the activation reads were issued a whole sub-step ago: a free wait
    // that leaves the next iteration's first MFMAs nothing to wait for)
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    st = st1;
  }
  // the last (up to 4) steps: nothing left to load
  for (; kt < nkt; ++kt) {
    const int st1 = st == 4 ? 0 : st + 1;
    const int behind = nkt - 2 - kt;  // steps after kt+1 whose loads may be in flight
    frag_load(1, st, 1);
    mma(0);
    convert(1);
    if (behind >= 2)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * C::LD_PER_T));
    else if (behind == 1)
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(C::LD_PER_T));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    // (one copy of each MFMA group: accumulators that flow through
    // duplicated MFMAs in branches get split across register files)
    const bool more = kt + 1 < nkt;
    if (more) frag_load(0, st1, 0);
    mma(1);
    if (more) convert(0);
    st = st1;
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
        if (f0 >= n_end) continue;
        const float v0 = acc[i][j][4 * r], v1 = acc[i][j][4 * r + 1];
        const float v2 = acc[i][j][4 * r + 2], v3 = acc[i][j][4 * r + 3];
        if (epi_gate(EPI)) {
          const _Float16 a0 = (_Float16)act_mul(epi_act(EPI), v0, v1);
          const _Float16 a1 = (_Float16)act_mul(epi_act(EPI), v2, v3);
          const uint32_t packed = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) +
                                       act_tile_off(t, f0 / 2, N / 2)) = packed;
        } else if (EPI == EPI_STORE_BF16) {
          uint32_t* dst =
              reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + (int64_t)t * N + f0);
          dst[0] = pack_bf16_rne(v0, v1);
          dst[1] = pack_bf16_rne(v2, v3);
        } else {
          float* dst = static_cast<float*>(out) + ((int64_t)blockIdx.y * M + t) * N + f0;
          *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
        }
      }
    }
  }
}

// y = bf16(sum over the split-K partials, in slice order): deterministic.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part,
                                                       uint16_t* __restrict__ y, int64_t n4,
                                                       int splits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4 outputs per thread
  if (i >= n4) return;
  f32x4 s = reinterpret_cast<const f32x4*>(part)[i];
  for (int z = 1; z < splits; ++z) s += reinterpret_cast<const f32x4*>(part + z * n4 * 4)[i];
  uint32_t* dst = reinterpret_cast<uint32_t*>(y + i * 4);
  dst[0] = pack_bf16_rne(s[0], s[1]);
  dst[1] = pack_bf16_rne(s[2], s[3]);
}

// Launch one GEMM with a given block tile and wave grid (splits > 1 only
// with the fp32 partial epilogue).
template <int NB, int MB, int WGN, int WGM, int EPI, bool AF16>
static hipError_t launch_gemm_t(const uint16_t* W, const uint16_t* Act, void* out, int M, int N,
                                int K, int splits, hipStream_t stream, int n_begin, int n_end) {
  using C = GemmCfg<NB, MB, WGN, WGM>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_wf16<NB, MB, WGN, WGM, EPI, AF16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int tiles = ((n_end - n_begin + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
  launch_kernel(epi_gate(EPI) ? KK_GEMM_GATEUP : KK_GEMM_DOWN,
                k_gemm_wf16<NB, MB, WGN, WGM, EPI, AF16>, dim3(tiles, splits), dim3(C::THREADS),
                (uint32_t)C::LDS_BYTES, stream, W, Act, out, M, N, K, n_begin, n_end);
  return hipGetLastError();
}

#ifndef FMLP_DOWN_W4
#define FMLP_DOWN_W4 1  // down GEMM's 256 x 256 tile on 4 waves (128 x 128 each)
#endif
#ifndef FMLP_S1_WGM
#define FMLP_S1_WGM 2  // 256 x 128 tiles: 4 x FMLP_S1_WGM waves (8 measured ~0.7% faster than 4)
#endif
#ifndef FMLP_DN_WGN
#define FMLP_DN_WGN 2  // wave grid of the down GEMM's 256 x 256 tile on 4 waves
#endif
#ifndef FMLP_DN_WGM
#define FMLP_DN_WGM 2
#endif
#ifndef FMLP_S0_WGN
#define FMLP_S0_WGN 4  // wave grid of the 256 x 256 tile
#endif
#ifndef FMLP_S0_WGM
#define FMLP_S0_WGM 2
#endif

// Tile shapes: 0 = 256 x 256 (gate/up: 8 waves, 4 x 2; down: 4 waves, 2 x 2),
// 1 = 256 x 128 (8 waves, 4 x 2), 2 = 128 x 128 (4 waves, 2 x 2). tail_rows > 0: the last tail_rows feature
// rows run as a second launch of 256 x 128 tiles, so that a last round of
// 256 x 256 tiles that would leave CUs idle becomes one round of half tiles.
struct GemmPlan {
  int shape, splits, tail_rows = 0;
};

// Time model of one GEMM (microseconds): rounds of workgroups over the CUs
// times the time of one workgroup at the per-CU rate measured for its shape
// on MI355X (prefill GEMMs of Llama-8B-shaped layers), plus, for split K,
// writing and re-reading the fp32 partials and the reduction launch.
static double gemm_time_us(int M, int N, int K, int shape, int splits) {
  static const int bn[3] = {256, 256, 128}, bm[3] = {256, 128, 128}, per_cu[3] = {1, 1, 2};
  // TFLOP/s per CU with one workgroup on it, and with per_cu of them
  static const double rate1[3] = {4.3, 3.7, 2.6}, rate_full[3] = {4.3, 3.7, 3.2};
  const int64_t tiles =
      (int64_t)((N + bn[shape] - 1) / bn[shape]) * ((M + bm[shape] - 1) / bm[shape]);
  const int64_t wgs = tiles * splits, slots = 256 * per_cu[shape];
  const int64_t rounds = (wgs + slots - 1) / slots;
  const bool shared = wgs > 256 && per_cu[shape] > 1;  // several workgroups per CU
  const double wg_flops = 2.0 * bn[shape] * bm[shape] * (double)K / splits;
  double t = shared ? rounds * wg_flops * per_cu[shape] / (rate_full[shape] * 1e6)
                    : rounds * wg_flops / (rate1[shape] * 1e6);
  if (splits > 1) t += 2.0 * splits * (double)M * N * 4 / 5.0e6 + 3.0;
  return t;
}

static GemmPlan plan_gemm(int M, int N, int K, bool may_split) {
  GemmPlan best{0, 1};
  double tb = 1e300;
  for (int shape = 0; shape < 3; ++shape) {
    for (int splits = 1; splits <= (may_split ? 8 : 1); splits *= 2) {
      const int nkb = K >> 5;
      if (nkb % splits != 0 || nkb / splits < 8) continue;
      const double t = gemm_time_us(M, N, K, shape, splits);
      if (t < tb) tb = t, best = GemmPlan{shape, splits};
    }
  }
  return best;
}

template <int EPI, bool AF16>
static hipError_t launch_gemm_plan(const GemmPlan& g, const uint16_t* W, const uint16_t* Act,
                                   void* out, int M, int N, int K, hipStream_t stream) {
  const int n_main = N - g.tail_rows;
  hipError_t e = hipSuccess;
  if (n_main > 0) {
    // the down GEMM runs the 256 x 256 tile on 4 waves, the gate/up GEMM on
    // FMLP_S0_WGN x FMLP_S0_WGM (measured best for each)
    constexpr bool w4 = !epi_gate(EPI) && FMLP_DOWN_W4;
    constexpr int s0n = w4 ? FMLP_DN_WGN : FMLP_S0_WGN, s0m = w4 ? FMLP_DN_WGM : FMLP_S0_WGM;
    if (g.shape == 0)
      e = launch_gemm_t<8, 8, s0n, s0m, EPI, AF16>(W, Act, out, M, N, K, g.splits, stream, 0,
                                                  n_main);
    else if (g.shape == 1)
      e = launch_gemm_t<8, 4, 4, FMLP_S1_WGM, EPI, AF16>(W, Act, out, M, N, K, g.splits, stream, 0,
                                                        n_main);
    else
      e = launch_gemm_t<4, 4, 2, 2, EPI, AF16>(W, Act, out, M, N, K, g.splits, stream, 0, n_main);
  }
  if (e != hipSuccess || g.tail_rows == 0) return e;
  return launch_gemm_t<8, 4, 4, FMLP_S1_WGM, EPI, AF16>(W, Act, out, M, N, K, g.splits, stream,
                                                      n_main, N);
}

// Split off a tail launch when the 256 x 256 tiles fill r >= 1 whole rounds
// of the 256 CUs and then at most half a round: the leftover bands of 256
// rows run as 256 x 128 tiles, at most one round of them.
static GemmPlan with_tail(GemmPlan g, int M, int N) {
  if (g.shape != 0 || g.splits != 1 || N % 256 != 0) return g;
  const int bands = N / 256, nM = (M + 255) / 256, tiles = bands * nM;
  const int full = tiles / 256, left = tiles % 256;
  if (full < 1 || left == 0 || left > 128 || left % nM != 0) return g;
  g.tail_rows = (left / nM) * 256;
  return g;
}

#ifndef FMLP_GEMM_PLAN
#define FMLP_GEMM_PLAN 0  // 0: by the time model; s*10 + k: shape s, k-way split of the down GEMM
#endif

static GemmPlan plan_down(int64_t M, int64_t d, int64_t ff) {
  if (FMLP_GEMM_PLAN) return GemmPlan{FMLP_GEMM_PLAN / 10, FMLP_GEMM_PLAN % 10};
  return plan_gemm((int)M, (int)d, (int)ff, true);
}

// Workspace regions, in order (each 256-byte aligned): n fp16 [pad32(M), d]
// and a fp16 [pad32(M), ff], both fragment-tiled; r fp32 [M]; the down
// projection's split-K partials fp32 [splits, M, d]; for int4 weights, the
// dequantised fp16 W_gu [2ff, d] and W_down [d, ff], fragment-tiled.
struct PrefillWs {
  uint16_t *n, *a;
  float *r, *part;
  uint16_t *wgu16, *wd16;
};

static PrefillWs prefill_ws(char* base, int64_t M, int64_t d, int64_t ff, int splits, size_t* total) {
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.n = reinterpret_cast<uint16_t*>(take((size_t)pad32(M) * d * 2));
  w.a = reinterpret_cast<uint16_t*>(take((size_t)pad32(M) * ff * 2));
  w.r = reinterpret_cast<float*>(take((size_t)M * 4));
  w.part = reinterpret_cast<float*>(take(splits > 1 ? (size_t)splits * M * d * 4 : 0));
  w.wgu16 = reinterpret_cast<uint16_t*>(take((size_t)2 * ff * d * 2));
  w.wd16 = reinterpret_cast<uint16_t*>(take((size_t)d * ff * 2));
  *total = off;
  return w;
}

size_t prefill_workspace_bytes(int64_t M, int64_t d, int64_t ff, int wtype) {
  size_t total = 0;
  prefill_ws(nullptr, M, d, ff, plan_down(M, d, ff).splits, &total);
  // (the fp16 expansion of the weights: int4 only)
  if (wtype != 1) total -= align256((size_t)2 * ff * d * 2) + align256((size_t)d * ff * 2);
  return total;
}

template <bool AF16>
static hipError_t prefill_gemms(const Problem& p, const PrefillWs& w, const uint16_t* wgu,
                                const uint16_t* wd, const GemmPlan& g2, hipStream_t stream) {
  const GemmPlan g1 =
      with_tail(plan_gemm((int)p.M, (int)(2 * p.ff), (int)p.d, false), (int)p.M, (int)(2 * p.ff));
  const int N1 = (int)(2 * p.ff), M1 = (int)p.M, K1 = (int)p.d;
  hipError_t e =
      p.act == 1   ? launch_gemm_plan<EPI_GELU_TANH_MUL_F16, AF16>(g1, wgu, w.n, w.a, M1, N1, K1,
                                                                  stream)
      : p.act == 2 ? launch_gemm_plan<EPI_GELU_ERF_MUL_F16, AF16>(g1, wgu, w.n, w.a, M1, N1, K1,
                                                                 stream)
                   : launch_gemm_plan<EPI_SILU_MUL_F16, AF16>(g1, wgu, w.n, w.a, M1, N1, K1, stream);
  if (e != hipSuccess) return e;
  if (g2.splits == 1)
    return launch_gemm_plan<EPI_STORE_BF16, AF16>(g2, wd, w.a, p.y, (int)p.M, (int)p.d, (int)p.ff,
                                                  stream);
  e = launch_gemm_plan<EPI_STORE_F32, AF16>(g2, wd, w.a, w.part, (int)p.M, (int)p.d, (int)p.ff,
                                            stream);
  if (e != hipSuccess) return e;
  const int64_t n4 = p.M * p.d / 4;
  launch_kernel(KK_SPLITK_REDUCE, k_splitk_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                stream, w.part, p.y, n4, g2.splits);
  return hipGetLastError();
}

static hipError_t launch_dequant_f16(const uint8_t* q, const uint16_t* s, int64_t R, int64_t K,
                                     uint16_t* out, hipStream_t stream) {
  const int64_t chunks = (R >> 4) * (K >> 5) * 64;
  launch_kernel(KK_DEQUANT, k_dequant_f16_tiled, dim3((unsigned)((chunks + 255) / 256)), dim3(256),
                0, stream, reinterpret_cast<const uint32_t*>(q), s, R, K, out);
  return hipGetLastError();
}

hipError_t launch_prefill(const Problem& p, hipStream_t stream) {
  const GemmPlan g2 = plan_down(p.M, p.d, p.ff);
  size_t total = 0;
  const PrefillWs w = prefill_ws(p.ws, p.M, p.d, p.ff, g2.splits, &total);
  launch_kernel(KK_RMS_PREP, k_rms_scale, dim3((unsigned)((p.M + 3) / 4)), dim3(256), 0, stream,
                p.x, p.eps, w.r, (int)p.M, (int)p.d, p.res);
  const int64_t slots = pad32(p.M) * p.d / 8;
  launch_kernel(KK_RMS_TILE, k_rms_tile, dim3((unsigned)((slots + 255) / 256)), dim3(256), 0,
                stream, p.x, p.gamma, w.r, w.n, (int)p.M, (int)p.d, slots, p.res, p.hout);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.wtype == 0)
    return prefill_gemms<false>(p, w, reinterpret_cast<const uint16_t*>(p.w_gu),
                                reinterpret_cast<const uint16_t*>(p.w_down), g2, stream);
  if (p.wtype == 2)  // fp16 weights: the fp16 products read them as they are
    return prefill_gemms<true>(p, w, reinterpret_cast<const uint16_t*>(p.w_gu),
                               reinterpret_cast<const uint16_t*>(p.w_down), g2, stream);
  if ((e = launch_dequant_f16(reinterpret_cast<const uint8_t*>(p.w_gu), p.s_gu, 2 * p.ff, p.d,
                              w.wgu16, stream)) != hipSuccess)
    return e;
  if ((e = launch_dequant_f16(reinterpret_cast<const uint8_t*>(p.w_down), p.s_down, p.d, p.ff,
                              w.wd16, stream)) != hipSuccess)
    return e;
  return prefill_gemms<true>(p, w, w.wgu16, w.wd16, g2, stream);
}

}  // namespace fmlp
