// Prefill path (M > 32 tokens): the MLP is a dense contraction here, so it
// runs as two LDS-tiled MFMA GEMMs.
//
//   0. RMSNorm: n = fp16(gamma * x * r), r = 1/sqrt(mean(x^2) + eps), one
//      pass over x (FastTPS review section 3, Figure 4 part1).
//   1. C = n W_gu^T on fp16 MFMA; the epilogue pairs interleaved columns
//      (gate 2i, up 2i+1) inside each lane and writes a = SiLU(g) * u as
//      fp16 (Figure 4 part2; the [M, 2ff] gate/up product never reaches HBM).
//   2. y = a W_down^T on fp16 MFMA, stored bf16 (Figure 4 part3).
//
// int4 weights are dequantised inside the GEMMs' weight-operand path (the
// llama.cpp PR digest runs its quantized matmul and the GLU in one pass): the
// codes of each K step (a quarter of the bf16 bytes) and their group scales
// go to LDS by DMA, and each wave expands its fragments in registers to fp16
// s*q (exact product, rounded once: relative error <= 2^-11, far inside the
// accuracy bar) right before its MFMAs, as it converts bf16 fragments.
//
// Operands are fp16 rather than bf16: rounding n to bf16 alone costs about
// 2e-2 max / 3.3e-3 mean relative error on Llama-8B-shaped layers, over the
// accuracy bar, while bf16 weights convert to fp16 exactly in the fp16 normal
// range and fp16 MFMA runs at the bf16 rate. Weights are converted in
// registers after their LDS reads.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

#include <mutex>
#include <type_traits>

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
// n = fp16(gamma * x * r), r = 1/sqrt(mean(x^2) + eps), written in the
// fragment-tiled activation layout; one wave per token slot of the padded
// token range (slots past M repeat the last token: finite, never stored
// into an output). Each lane holds chunks lane, lane + 64, ... of the row
// (R of them in registers, the rest of a very long row re-read), sums
// their squares in that order, and the wave combines the lane sums; then
// every chunk is scaled and stored as one 16-byte slot of its fragment.
// With res, the row is the residual stream h = bf16_rne(x + res), stored to
// hout once per element.
// STAGE (d <= 8192): the 8 token slots of a workgroup fill whole 128-byte
// lines of each fragment (slots 8j .. 8j+7 of one column chunk), so the
// scaled chunks go through LDS first and each store instruction then writes
// 8 whole lines, rather than 64 scattered 16-byte pieces of 64 lines (one
// per token row chunk). LDS position of chunk c of the workgroup's token w:
// 8c + (w ^ c % 8), conflict-free for both the row-wise writes and the
// line-wise reads.
// R: chunks of 8 per lane kept in registers, 8 for rows up to d = 4096 and
// 16 up to 8192 (sized to the row, so that short rows leave registers for
// more waves per CU).
constexpr int kRmsStageMaxD = 8192;

template <bool STAGE, int R>
__global__ __launch_bounds__(512) void k_rms_norm_tiled(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ gamma,
                                                        float eps, uint16_t* __restrict__ n,
                                                        int M, int d,
                                                        const uint16_t* __restrict__ res,
                                                        uint16_t* __restrict__ hout) {
  extern __shared__ u32x4 rms_lds[];  // STAGE: 8 d / 8 chunks of 16 bytes
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 8 + (threadIdx.x >> 6);  // token slot (< pad32(M))
  const int ts = t < M ? t : M - 1;
  const uint16_t* xr = x + (int64_t)ts * d;
  const uint16_t* rr = res ? res + (int64_t)ts * d : nullptr;
  const int nch = d >> 3;
  auto row = [&](int c) {
    const u32x4 v = ld16(xr + c * 8);
    return rr ? add_bf16x8(v, ld16(rr + c * 8)) : v;
  };
  // the row's chunks, and for rows up to 8 chunks per lane gamma's too (in
  // flight with them rather than loaded after the row's sum is known; longer
  // rows would run out of registers)
  constexpr bool kPreGamma = R <= 8;
  u32x4 v[R], gv[kPreGamma ? R : 1];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nch ? row(c) : u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (kPreGamma) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = lane + 64 * i;
      gv[i] = c < nch ? ld16(gamma + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(v[i][j]), hi = bf16_hi(v[i][j]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  for (int c = lane + 64 * R; c < nch; c += 64) {  // only for very long rows
    const u32x4 w = row(c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float r = 1.0f / sqrtf(ss / (float)d + eps);
  // chunk c (columns 8c .. 8c+7) of token slot t: fragment (t/32, c/4, (c/2)%2),
  // slot (c%2)*32 + t%32
  const int tb = t >> 5, tl = t & 31, nkb = d >> 5;
  auto put = [&](int c, u32x4 w, u32x4 gm) {
    if (hout && t < M) st16(hout + (int64_t)t * d + c * 8, w);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(bf16_lo(w[j]) * bf16_lo(gm[j]) * r);
      const _Float16 hi = (_Float16)(bf16_hi(w[j]) * bf16_hi(gm[j]) * r);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    if constexpr (STAGE) {
      rms_lds[c * 8 + ((threadIdx.x >> 6) ^ (c & 7))] = o;
    } else {
      const int64_t frag = ((int64_t)tb * nkb + (c >> 2)) * 2 + ((c >> 1) & 1);
      st16(n + frag * 512 + ((c & 1) * 32 + tl) * 8, o);
    }
  };
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) put(c, v[i], kPreGamma ? gv[kPreGamma ? i : 0] : ld16(gamma + c * 8));
  }
  if constexpr (STAGE) {
    __syncthreads();
    // position p holds chunk c = p / 8 of token slot 8 blockIdx.x + (p % 8 ^ c % 8)
    const int tl0 = (blockIdx.x * 8) & 31;
    for (int p = threadIdx.x; p < nch * 8; p += 512) {
      const int c = p >> 3, w = (p & 7) ^ (c & 7);
      const int64_t frag = ((int64_t)tb * nkb + (c >> 2)) * 2 + ((c >> 1) & 1);
      st16(n + frag * 512 + ((c & 1) * 32 + tl0 + w) * 8, rms_lds[p]);
    }
  } else {
    for (int c = lane + 64 * R; c < nch; c += 64) put(c, row(c), ld16(gamma + c * 8));
  }
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

// Weight kinds of the prefill GEMMs: bf16 tiles (converted to fp16 in
// registers), fp16 tiles (read as they are), and int4 super-tiles with fp16
// group scales (dequantised in registers, see int4x8_to_f16x8).
enum { WF_BF16 = 0, WF_F16 = 1, WF_INT4 = 2 };

template <int NB, int MB, int WGN_, int WGM_, int WKW = WF_BF16>  // 32-row blocks; wave grid
struct GemmCfg {
  static constexpr int WGN = WGN_, WGM = WGM_, W = WGN * WGM, THREADS = 64 * W;
  static constexpr int BN = NB * 32, BM = MB * 32;
  static constexpr int WNB = NB / WGN, WMB = MB / WGM;  // 32-row blocks per wave
  static constexpr bool Q4 = WKW == WF_INT4;
  // loads per thread and step: one per 16-row weight band (a 1 KB storage
  // tile, or for int4 the band's 256 bytes of codes of the step's group),
  // int4 also one of group scales (SC_BANDS bands per wave), and one per
  // activation fragment of 1 KB
  static constexpr int A_PER_T = NB * 2 / W, SC_BANDS = NB * 2 / W;
  static constexpr int A_LD = A_PER_T + (Q4 ? 1 : 0);
  static constexpr int B_PER_T = MB * 2 / W, LD_PER_T = A_LD + B_PER_T;
  // 16-bit elements per stage: weights (tiles; or int4 codes, 128 per band,
  // then 128 per wave of scale words), activations
  static constexpr int A_CODE_ELEMS = NB * 2 * 128;
  static constexpr int A_ELEMS = Q4 ? A_CODE_ELEMS + W * 128 : NB * 1024;
  static constexpr int B_ELEMS = MB * 1024;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int STAGES = 5;
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_ELEMS * 2;
  // one wave per SIMD when the accumulators alone fill 256 registers
  static constexpr int WAVES_PER_EU = (WNB * WMB >= 16) ? 1 : 2;
  static_assert((W == 4 || W == 8) && WNB >= 1 && WMB >= 1 && A_PER_T * W == NB * 2 &&
                B_PER_T * W == MB * 2, "tile");
  static_assert(!Q4 || SC_BANDS * 16 <= 64, "int4 scale lanes");
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
// One SZ-byte-per-lane LDS DMA (SZ = 16 or 4) through a raw buffer
// descriptor over [base, base + extent): lane l's SZ bytes at byte offset
// voff + soff land at dst + SZ l. (The descriptor is built here, not in the
// kernel body: its loop-invariant scalar setup is hoisted by the compiler.)
template <int SZ>
__device__ __forceinline__ void buf_load_lds(const void* base, int extent, lptr_t dst, int voff,
                                             int soff) {
  static_assert(SZ == 4 || SZ == 16, "LDS DMA size");
  const auto rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, extent, kBufWord3);
  if constexpr (SZ == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, soff, 0, 0);
}

// Eight int4 codes (one 32-bit word, code m in bits 4m..4m+3, two's
// complement) and their fp16 group scale -> the eight weights s*q as fp16 in
// natural order, each the exact product rounded once to nearest even: the
// same value as fp16(float(s) * q). The magic-number int4 -> fp16 method
// (Kim et al., arXiv 2211.10017), with a byte permute to place the nibbles:
// with t = w ^ 0x88888888 every nibble is
// q + 8; v_perm places nibbles 2j and 2j+1 in the low bytes of the two halves
// of word j, and with 0x6400 in the high bytes the halves are the fp16
// values 1024 + q + 8 (exact); a packed fp16 add of -1032 leaves q exactly,
// and a packed fp16 multiply by s rounds s*q once.
__device__ __forceinline__ u32x4 int4x8_to_f16x8(uint32_t w, uint32_t s16) {
  const uint32_t t = w ^ 0x88888888u;
  const uint32_t ev = t & 0x0F0F0F0Fu;         // bytes: codes 0, 2, 4, 6 (+8)
  const uint32_t od = (t >> 4) & 0x0F0F0F0Fu;  // bytes: codes 1, 3, 5, 7 (+8)
  const f16x2 s2 = __builtin_bit_cast(f16x2, (s16 & 0xFFFFu) * 0x10001u);
  const f16x2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bytes (ev.j, 0, od.j, 0): selector j, 0x0C (zero), 4 + j, 0x0C
    const uint32_t sel = (uint32_t)j | 0x0C00u | ((uint32_t)(4 + j) << 16) | 0x0C000000u;
    const uint32_t h = __builtin_amdgcn_perm(od, ev, sel) | 0x64006400u;
    const f16x2 q = __builtin_bit_cast(f16x2, h) + off;
    r[j] = __builtin_bit_cast(uint32_t, q * s2);
  }
  return r;
}

// s_waitcnt immediate for vmcnt(vm) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] |
// expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]). The builtin, unlike
// inline asm, is seen by the compiler's own wait insertion, which then adds
// no redundant waits.
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | 0x70 | ((vm >> 4) << 14); }

// One workgroup's tile: the pid-th of the tiles of feature rows n_begin ..
// n_end-1 (and K slice blockIdx.y of gridDim.y). WKW: weight kind (WF_*).
// Wt: weight tiles, or int4 code super-tiles with Wsc their fp16 scales
// (unused otherwise).
template <int NB, int MB, int WGN, int WGM, int EPI, int WKW>
__device__ __forceinline__ void gemm_tile(const void* __restrict__ Wt,
                                          const uint16_t* __restrict__ Wsc,
                                          const uint16_t* __restrict__ Act,
                                          void* __restrict__ out, int M, int N, int K,
                                          int n_begin, int n_end, int pid) {
  using C = GemmCfg<NB, MB, WGN, WGM, WKW>;
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wn = wave % C::WGN, wm = wave / C::WGN;

  // this launch covers feature rows n_begin .. n_end-1 of the N
  const int nN = (n_end - n_begin + C::BN - 1) / C::BN, nM = (M + C::BM - 1) / C::BM;
  const int T = nN * nM;
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
  // Weight chunk i of a thread: 16-row band rb = W*i + wave of the tile
  // (rows past N clamped), slot = lane. bf16 / fp16: its 1 KB storage tile,
  // LDS image at rb * 1 KB. int4: word (kbeg + kt) % 4 of the lane's 16-byte
  // slot of the band's super-tile (kbeg + kt) / 4, i.e. the codes of group
  // kbeg + kt, LDS image at rb * 256 bytes in slot order; and one 4-byte
  // load per wave of group scales: lane j takes the scale pair (groups
  // 2 (g/2), +1) of row j % 16 of band wave * SC_BANDS + (j / 16) % SC_BANDS
  // (lanes past 16 SC_BANDS repeat those loads into unused LDS words).
  const int rb0 = n0 >> 4;
  const int nq = (K + 127) >> 7;  // int4 super-tiles per band
  const void* wbase;
  int wext;
  if constexpr (C::Q4) {
    wbase = static_cast<const uint8_t*>(Wt) + (int64_t)rb0 * nq * 1024;
    wext = buf_extent(((int64_t)nrb - rb0) * nq * 1024);
  } else {
    wbase = static_cast<const uint16_t*>(Wt) + ((int64_t)rb0 * nkb + kbeg) * 512;
    wext = buf_extent(((int64_t)nrb * nkb - ((int64_t)rb0 * nkb + kbeg)) * 1024);
  }
  int woff[C::A_PER_T];
#pragma unroll
  for (int i = 0; i < C::A_PER_T; ++i) {
    const int rb = C::W * i + wave;
    const int rbc = rb0 + rb < nrb ? rb : nrb - 1 - rb0;
    woff[i] = C::Q4 ? rbc * nq * 1024 + lane * 16 : rbc * nkb * 1024 + lane * 16;
  }
  const uint16_t* sbase = Wsc + (int64_t)rb0 * nq * 64;
  const int sext = C::Q4 ? buf_extent(((int64_t)nrb - rb0) * nq * 128) : 0;
  int soff_lane = 0;
  if constexpr (C::Q4) {
    const int rb = wave * C::SC_BANDS + (lane >> 4) % C::SC_BANDS;
    const int rbc = rb0 + rb < nrb ? rb : nrb - 1 - rb0;
    soff_lane = rbc * nq * 128 + (lane & 15) * 8;
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
    if constexpr (C::Q4) {
      const int g = kbeg + kt;
#pragma unroll
      for (int i = 0; i < C::A_PER_T; ++i)
        buf_load_lds<4>(wbase, wext, (lptr_t)(base + (C::W * i + wave) * 128), woff[i],
                        (g >> 2) * 1024 + (g & 3) * 4);
      buf_load_lds<4>(sbase, sext, (lptr_t)(base + C::A_CODE_ELEMS + wave * 128), soff_lane,
                      (g >> 2) * 128 + (g & 2) * 2);
    } else {
#pragma unroll
      for (int i = 0; i < C::A_PER_T; ++i)
        buf_load_lds<16>(wbase, wext, (lptr_t)(base + (C::W * i + wave) * 512), woff[i],
                         kt * 1024);
    }
  };
  auto load_b = [&](int kt, int st) __attribute__((always_inline)) {
    uint16_t* base = lds + st * C::STAGE_ELEMS + C::A_ELEMS;
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i)
      buf_load_lds<16>(abase, aext, (lptr_t)(base + (C::W * i + wave) * 512), aoff[i], kt * 2048);
  };
  auto load_step = [&](int kt, int st) __attribute__((always_inline)) {
    load_a(kt, st);
    load_b(kt, st);
  };

  // int4: lane l of the fragment of 32-row block b, half q reads the code
  // word of slot 32 q + 16 (l / 32) + l % 16 of band 2b + (l % 32) / 16, and
  // that row's fp16 scale of the step's group (half g % 2 of its pair)
  const int q4_band = (lane & 31) >> 4, q4_slot = (lane >> 5) * 16 + (lane & 15);
  u32x4 fa[2][C::WNB], fb[2][C::WMB];
  auto frag_load_a = [&](int buf, int st, int q, int kt) __attribute__((always_inline)) {
    const uint16_t* base = lds + st * C::STAGE_ELEMS;
    if constexpr (C::Q4) {
      const uint32_t* codes = reinterpret_cast<const uint32_t*>(base);
#pragma unroll
      for (int i = 0; i < C::WNB; ++i) {
        const int band = 2 * (wn * C::WNB + i) + q4_band;
        const int sw = (band / C::SC_BANDS) * 64 + (band % C::SC_BANDS) * 16 + (lane & 15);
        fa[buf][i][0] = codes[band * 64 + q * 32 + q4_slot];
        fa[buf][i][1] = base[C::A_CODE_ELEMS + sw * 2 + ((kbeg + kt) & 1)];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::WNB; ++i)
        fa[buf][i] = *reinterpret_cast<const u32x4*>(
            &base[a_rd + (wn * C::WNB + i) * 1024 + q * 256]);
    }
  };
  auto frag_load_b = [&](int buf, int st, int q) __attribute__((always_inline)) {
    const uint16_t* base = lds + st * C::STAGE_ELEMS;
#pragma unroll
    for (int j = 0; j < C::WMB; ++j)
      fb[buf][j] = *reinterpret_cast<const u32x4*>(
          &base[b_rd + ((wm * C::WMB + j) * 2 + q) * 512]);
  };
  auto frag_load = [&](int buf, int st, int q, int kt) __attribute__((always_inline)) {
    frag_load_a(buf, st, q, kt);
    frag_load_b(buf, st, q);
  };
  // the same reads, weights strictly first, all issued before what follows
  auto frag_load_ordered = [&](int buf, int st, int q, int kt) __attribute__((always_inline)) {
    frag_load_a(buf, st, q, kt);
    __builtin_amdgcn_sched_barrier(0);
    frag_load_b(buf, st, q);
    __builtin_amdgcn_sched_barrier(0);
  };
  // weight fragments to fp16 in place (after their LDS reads land): bf16
  // converted, int4 dequantised, fp16 as they are
  auto convert = [&](int buf) __attribute__((always_inline)) {
    if constexpr (WKW == WF_BF16) {
#pragma unroll
      for (int i = 0; i < C::WNB; ++i) fa[buf][i] = bf16x8_to_f16x8(fa[buf][i]);
    } else if constexpr (C::Q4) {
#pragma unroll
      for (int i = 0; i < C::WNB; ++i) fa[buf][i] = int4x8_to_f16x8(fa[buf][i][0], fa[buf][i][1]);
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
    constexpr int NV = WKW == WF_F16 ? 0 : C::WNB * (C::Q4 ? 20 : 12), HALF = NMF / 2;
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

  // prologue: steps 0..3 -> stages 0..3; wait for step 0 only (the loop's
  // waits cover steps 1..3, whose loads stay in flight: with every CU
  // starting a tile at once, waiting for all four steps held the first
  // MFMAs back by about 1 us per tile on MI355X); its first fragments
  const int npre = nkt < 4 ? nkt : 4;
  for (int s = 0; s < npre; ++s) load_step(s, s);
  if (npre == 4)
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 * C::LD_PER_T));
  else
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
  frag_load(0, 0, 0, 0);
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
    frag_load_ordered(1, st, 1, kt);
    if (kSpread) load_a(kt + 4, st4);
    mma(0);
    convert(1);
    interleave(std::integral_constant<int, C::A_LD>{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * C::LD_PER_T + C::A_LD));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (!kSpread) load_b(kt + 4, st4);
    frag_load_ordered(0, st1, 0, kt + 1);
    if (kSpread) load_b(kt + 4, st4);
    mma(1);
    convert(0);
    interleave(std::integral_constant<int, C::B_PER_T>{});
    __builtin_amdgcn_sched_barrier(0);
    // (the activation reads were issued a whole sub-step ago: a free wait
    // that leaves the next iteration's first MFMAs nothing to wait for)
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));
    st = st1;
  }
  // the last (up to 4) steps: nothing left to load
  for (; kt < nkt; ++kt) {
    const int st1 = st == 4 ? 0 : st + 1;
    const int behind = nkt - 2 - kt;  // steps after kt+1 whose loads may be in flight
    frag_load(1, st, 1, kt);
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
    if (more) frag_load(0, st1, 0, kt + 1);
    mma(1);
    if (more) convert(0);
    st = st1;
  }

  // epilogue: lane holds token t = col of block (i, j) and rows 8r + 4 grp + e
  const int col = lane & 31, grp = lane >> 5;
  if constexpr (epi_gate(EPI)) {
    // Row pair (2p, 2p+1) of a 32-row block gives product p of its 16, so
    // lane l holds products 4r + 2 grp and 4r + 2 grp + 1 (r = 0..3) of its
    // token. Lanes l and l ^ 32 swap two of their four words, leaving
    // products 0..7 in lane l < 32 and 8..15 in lane l + 32: each then
    // stores one 16-byte slot, and the wave one whole 1 KB fragment.
    // (Blocks lie wholly inside or outside n_end: both are multiples of 32.)
#pragma unroll
    for (int i = 0; i < C::WNB; ++i) {
      const int fb = n0 + (wn * C::WNB + i) * 32;
#pragma unroll
      for (int j = 0; j < C::WMB; ++j) {
        const int t = m0 + (wm * C::WMB + j) * 32 + col;
        uint32_t pk[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const _Float16 a0 =
              (_Float16)act_mul(epi_act(EPI), acc[i][j][4 * r], acc[i][j][4 * r + 1]);
          const _Float16 a1 =
              (_Float16)act_mul(epi_act(EPI), acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]);
          pk[r] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        }
        const uint32_t s0 = __shfl_xor(grp ? pk[0] : pk[2], 32);
        const uint32_t s1 = __shfl_xor(grp ? pk[1] : pk[3], 32);
        const u32x4 o = grp ? u32x4{s0, pk[2], s1, pk[3]} : u32x4{pk[0], s0, pk[1], s1};
        if (t < M && fb < n_end)
          st16(static_cast<uint16_t*>(out) + act_tile_off(t, fb / 2 + 8 * grp, N / 2), o);
      }
    }
    return;
  }
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
        if (EPI == EPI_STORE_BF16) {
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

template <int NB, int MB, int WGN, int WGM, int EPI, int WKW>
__global__ __launch_bounds__(64 * WGN * WGM) __attribute__((amdgpu_waves_per_eu(
    GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU, GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU))) void
k_gemm_wf16(const void* __restrict__ Wt, const uint16_t* __restrict__ Wsc,
            const uint16_t* __restrict__ Act, void* __restrict__ out, int M, int N, int K,
            int n_begin, int n_end) {
  gemm_tile<NB, MB, WGN, WGM, EPI, WKW>(Wt, Wsc, Act, out, M, N, K, n_begin, n_end,
                                        (int)blockIdx.x);
}

// One launch for a GEMM whose last feature rows run as lower tiles:
// workgroups below n_main_wgs take the NB x MB tiles of rows 0 .. n_main-1,
// the others the NB x MBT tiles of rows n_main .. N-1. Workgroups are
// dispatched in index order as CUs free up, so the lower tiles start while
// the last full ones drain, with no kernel boundary between them (a launch
// each measured about 4 us apart on MI355X). n_main_wgs is a multiple of 8,
// which keeps both parts' XCD-major tile order.
template <int NB, int MB, int MBT, int WGN, int WGM, int WGMT, int EPI, int WKW>
__global__ __launch_bounds__(64 * WGN * WGM) __attribute__((amdgpu_waves_per_eu(
    GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU, GemmCfg<NB, MB, WGN, WGM>::WAVES_PER_EU))) void
k_gemm_wf16_tail(const void* __restrict__ Wt, const uint16_t* __restrict__ Wsc,
                 const uint16_t* __restrict__ Act, void* __restrict__ out, int M, int N, int K,
                 int n_main, int n_main_wgs) {
  static_assert(WGN * WGM == WGN * WGMT, "both parts run on the same workgroup size");
  if ((int)blockIdx.x < n_main_wgs)
    gemm_tile<NB, MB, WGN, WGM, EPI, WKW>(Wt, Wsc, Act, out, M, N, K, 0, n_main,
                                          (int)blockIdx.x);
  else
    gemm_tile<NB, MBT, WGN, WGMT, EPI, WKW>(Wt, Wsc, Act, out, M, N, K, n_main, N,
                                            (int)blockIdx.x - n_main_wgs);
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
// The weights of one GEMM: tiles (bf16 or fp16), or int4 codes and scales.
struct GemmW {
  const void* w;
  const uint16_t* s;
};

template <int NB, int MB, int WGN, int WGM, int EPI, int WKW>
static hipError_t launch_gemm_t(GemmW W, const uint16_t* Act, void* out, int M, int N, int K,
                                int splits, hipStream_t stream, int n_begin, int n_end) {
  using C = GemmCfg<NB, MB, WGN, WGM, WKW>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_wf16<NB, MB, WGN, WGM, EPI, WKW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int tiles = ((n_end - n_begin + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
  launch_kernel(epi_gate(EPI) ? KK_GEMM_GATEUP : KK_GEMM_DOWN,
                k_gemm_wf16<NB, MB, WGN, WGM, EPI, WKW>, dim3(tiles, splits), dim3(C::THREADS),
                (uint32_t)C::LDS_BYTES, stream, W.w, W.s, Act, out, M, N, K, n_begin, n_end);
  return hipGetLastError();
}

// The 256 x 256 tiles of rows 0 .. n_main-1 and the 256 x 128 tiles of the
// rest in one launch (gate/up GEMMs: both on 8 waves, 4 x 2).
template <int EPI, int WKW>
static hipError_t launch_gemm_main_tail(GemmW W, const uint16_t* Act, void* out, int M, int N,
                                        int K, int n_main, hipStream_t stream) {
  using C0 = GemmCfg<8, 8, 4, 2, WKW>;
  using C1 = GemmCfg<8, 4, 4, 2, WKW>;
  static_assert(C0::LDS_BYTES >= C1::LDS_BYTES, "LDS");
  auto kern = k_gemm_wf16_tail<8, 8, 4, 4, 2, 2, EPI, WKW>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [kern] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)C0::LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int nM0 = (M + 255) / 256, nM1 = (M + 127) / 128;
  const int main_wgs = (n_main / 256) * nM0;
  const int tail_wgs = ((N - n_main + 255) / 256) * nM1;
  launch_kernel(KK_GEMM_GATEUP, kern, dim3(main_wgs + tail_wgs), dim3(C0::THREADS),
                (uint32_t)C0::LDS_BYTES, stream, W.w, W.s, Act, out, M, N, K, n_main, main_wgs);
  return hipGetLastError();
}

constexpr int kDownW4 = 1;  // down GEMM's 256 x 256 tile on 4 waves (128 x 128 each)
constexpr int kS1Wgm = 2;  // 256 x 128 tiles: 4 x kS1Wgm waves (8 measured ~0.7% faster than 4)
constexpr int kDnWgn = 2;  // wave grid of the down GEMM's 256 x 256 tile on 4 waves
constexpr int kDnWgm = 2;
constexpr int kS0Wgn = 4;  // wave grid of the 256 x 256 tile
constexpr int kS0Wgm = 2;

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

template <int EPI, int WKW>
static hipError_t launch_gemm_plan(const GemmPlan& g, GemmW W, const uint16_t* Act, void* out,
                                   int M, int N, int K, hipStream_t stream) {
  const int n_main = N - g.tail_rows;
  // gate/up: the 256 x 256 tiles and the 256 x 128 tail tiles share a launch
  if constexpr (epi_gate(EPI) && kS0Wgn == 4 && kS0Wgm == 2 && kS1Wgm == 2) {
    if (g.tail_rows > 0 && g.shape == 0 && g.splits == 1 && n_main > 0)
      return launch_gemm_main_tail<EPI, WKW>(W, Act, out, M, N, K, n_main, stream);
  }
  hipError_t e = hipSuccess;
  if (n_main > 0) {
    // the down GEMM runs the 256 x 256 tile on 4 waves, the gate/up GEMM on
    // kS0Wgn x kS0Wgm (measured best for each)
    constexpr bool w4 = !epi_gate(EPI) && kDownW4;
    constexpr int s0n = w4 ? kDnWgn : kS0Wgn, s0m = w4 ? kDnWgm : kS0Wgm;
    if (g.shape == 0)
      e = launch_gemm_t<8, 8, s0n, s0m, EPI, WKW>(W, Act, out, M, N, K, g.splits, stream, 0,
                                                  n_main);
    else if (g.shape == 1)
      e = launch_gemm_t<8, 4, 4, kS1Wgm, EPI, WKW>(W, Act, out, M, N, K, g.splits, stream, 0,
                                                        n_main);
    else
      e = launch_gemm_t<4, 4, 2, 2, EPI, WKW>(W, Act, out, M, N, K, g.splits, stream, 0, n_main);
  }
  if (e != hipSuccess || g.tail_rows == 0) return e;
  return launch_gemm_t<8, 4, 4, kS1Wgm, EPI, WKW>(W, Act, out, M, N, K, g.splits, stream,
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

// The down GEMM's plan depends on M only through its 128-token band (every
// tile height divides 256, so the tile counts are those of the band's top),
// and above kSplitMaxM tokens, where every shape fills the CUs many times
// over, it never splits K.
constexpr int64_t kPlanBand = 128;
constexpr int64_t kSplitMaxM = 131072;

static GemmPlan plan_down(int64_t M, int64_t d, int64_t ff) {
  const int64_t Mb = (M + kPlanBand - 1) / kPlanBand * kPlanBand;
  return plan_gemm((int)Mb, (int)d, (int)ff, M <= kSplitMaxM);
}

// Workspace regions, in order (each 256-byte aligned): n fp16 [pad32(M), d]
// and a fp16 [pad32(M), ff], both fragment-tiled; the down projection's
// split-K partials fp32 [splits, M, d]. The same for every
// weight type (int4 weights are dequantised inside the GEMMs).
struct PrefillWs {
  uint16_t *n, *a;
  float* part;
};

static PrefillWs prefill_ws(char* base, int64_t M, int64_t d, int64_t ff, size_t part_bytes,
                            size_t* total) {
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.n = reinterpret_cast<uint16_t*>(take((size_t)pad32(M) * d * 2));
  w.a = reinterpret_cast<uint16_t*>(take((size_t)pad32(M) * ff * 2));
  w.part = reinterpret_cast<float*>(take(part_bytes));
  *total = off;
  return w;
}

static size_t split_partial_bytes(int64_t M, int64_t d, int splits) {
  return splits > 1 ? (size_t)splits * M * d * 4 : 0;
}

static size_t ws_total(int64_t M, int64_t d, int64_t ff, int wtype, size_t part_bytes) {
  (void)wtype;  // the same regions for every weight type
  size_t total = 0;
  prefill_ws(nullptr, M, d, ff, part_bytes, &total);
  return total;
}

size_t prefill_workspace_bytes(int64_t M, int64_t d, int64_t ff, int wtype) {
  return ws_total(M, d, ff, wtype, split_partial_bytes(M, d, plan_down(M, d, ff).splits));
}

// The largest split-partial region over every M' <= M: the plan is constant
// on each 128-token band, so the partials of a band peak at its top (or at M
// in the last band). Every other region grows with M.
size_t prefill_workspace_envelope(int64_t M, int64_t d, int64_t ff, int wtype) {
  size_t part = 0;
  const int64_t top = M < kSplitMaxM ? M : kSplitMaxM;
  for (int64_t b = kPlanBand;; b += kPlanBand) {
    const int64_t m = b < top ? b : top;
    const size_t pb = split_partial_bytes(m, d, plan_down(m, d, ff).splits);
    part = pb > part ? pb : part;
    if (b >= top) break;
  }
  return ws_total(M, d, ff, wtype, part);
}

template <int WKW>
static hipError_t prefill_gemms(const Problem& p, const PrefillWs& w, GemmW wgu, GemmW wd,
                                const GemmPlan& g2, hipStream_t stream) {
  const GemmPlan g1 =
      with_tail(plan_gemm((int)p.M, (int)(2 * p.ff), (int)p.d, false), (int)p.M, (int)(2 * p.ff));
  const int N1 = (int)(2 * p.ff), M1 = (int)p.M, K1 = (int)p.d;
  hipError_t e =
      p.act == 1   ? launch_gemm_plan<EPI_GELU_TANH_MUL_F16, WKW>(g1, wgu, w.n, w.a, M1, N1, K1,
                                                                 stream)
      : p.act == 2 ? launch_gemm_plan<EPI_GELU_ERF_MUL_F16, WKW>(g1, wgu, w.n, w.a, M1, N1, K1,
                                                                stream)
                   : launch_gemm_plan<EPI_SILU_MUL_F16, WKW>(g1, wgu, w.n, w.a, M1, N1, K1, stream);
  if (e != hipSuccess) return e;
  if (g2.splits == 1)
    return launch_gemm_plan<EPI_STORE_BF16, WKW>(g2, wd, w.a, p.y, (int)p.M, (int)p.d, (int)p.ff,
                                                 stream);
  e = launch_gemm_plan<EPI_STORE_F32, WKW>(g2, wd, w.a, w.part, (int)p.M, (int)p.d, (int)p.ff,
                                           stream);
  if (e != hipSuccess) return e;
  const int64_t n4 = p.M * p.d / 4;
  launch_kernel(KK_SPLITK_REDUCE, k_splitk_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                stream, w.part, p.y, n4, g2.splits);
  return hipGetLastError();
}

hipError_t launch_prefill(const Problem& p, hipStream_t stream) {
  const GemmPlan g2 = plan_down(p.M, p.d, p.ff);
  size_t total = 0;
  const PrefillWs w =
      prefill_ws(p.ws, p.M, p.d, p.ff, split_partial_bytes(p.M, p.d, g2.splits), &total);
  const dim3 rgrid((unsigned)(pad32(p.M) / 8));
  if (p.d <= kRmsStageMaxD) {
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [] {
      for (const void* k : {reinterpret_cast<const void*>(&k_rms_norm_tiled<true, 8>),
                            reinterpret_cast<const void*>(&k_rms_norm_tiled<true, 16>)}) {
        const hipError_t e = hipFuncSetAttribute(
            k, hipFuncAttributeMaxDynamicSharedMemorySize, 16 * kRmsStageMaxD);
        if (e != hipSuccess) attr_err = e;
      }
    });
    if (attr_err != hipSuccess) return attr_err;
    if (p.d <= 4096)
      launch_kernel(KK_RMS_NORM, k_rms_norm_tiled<true, 8>, rgrid, dim3(512),
                    (uint32_t)(16 * p.d), stream, p.x, p.gamma, p.eps, w.n, (int)p.M, (int)p.d,
                    p.res, p.hout);
    else
      launch_kernel(KK_RMS_NORM, k_rms_norm_tiled<true, 16>, rgrid, dim3(512),
                    (uint32_t)(16 * p.d), stream, p.x, p.gamma, p.eps, w.n, (int)p.M, (int)p.d,
                    p.res, p.hout);
  } else {
    launch_kernel(KK_RMS_NORM, k_rms_norm_tiled<false, 16>, rgrid, dim3(512), 0, stream, p.x,
                  p.gamma, p.eps, w.n, (int)p.M, (int)p.d, p.res, p.hout);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const GemmW wgu{p.w_gu, p.s_gu}, wd{p.w_down, p.s_down};
  if (p.wtype == 0) return prefill_gemms<WF_BF16>(p, w, wgu, wd, g2, stream);
  if (p.wtype == 2) return prefill_gemms<WF_F16>(p, w, wgu, wd, g2, stream);
  return prefill_gemms<WF_INT4>(p, w, wgu, wd, g2, stream);
}

}  // namespace fmlp
