// Weight preparation: gate/up row interleave into the fragment-tiled layout,
// plain tiling (for W_down), int4 group-32 quantisation and its fp32
// expansion (test hook) in the row-major exchange format, and the tiling of
// row-major int4 (interleaved or plain) into the layout the kernels read.
//
// Fragment-tiled bf16 layout of a logical matrix W [R, K] (R % 16 == 0,
// K % 32 == 0): one 1024-byte tile per (16-row block rb, 32-column block kb),
// tiles in (rb, kb) row-major order; inside a tile, 16-byte slot
// L = 16*(k%32/8) + r%16 holds the 8 consecutive elements of row r starting
// at column 8*(k%32/8). Slot L is exactly what lane L supplies to an MFMA
// 16x16x32 operand, so a wave reads a whole tile as one contiguous 1 KB load.
//
// Tiled int4 (groups of 32 along K, four groups per "super-tile"): super-tile
// (rb, q) covers groups 4q .. 4q+3 of rows 16rb .. 16rb+15 in 1024 bytes;
// slot L (16 bytes) holds, in 32-bit word j, the 8 codes of row 16rb + L%16,
// group 4q + j, columns 8*(L/16) .. +7 (code m in bits 4m..4m+3, two's
// complement). Scales: fp16 element (rb*nq + q)*64 + (r%16)*4 + j. Groups
// past K/32 in the last super-tile hold zero codes and scales.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace fmlp {

// ---------------------------------------------------------------- tiling
// One thread per 16-byte output slot. With `b` non-null the logical matrix is
// the row interleave of a (even rows) and b (odd rows): FastTPS review,
// section 3 item 3 (gate and up merged into one interleaved matmul) and the
// llama.cpp PR digest (gate and up rows alternate).
__global__ __launch_bounds__(256) void k_tile_bf16(const uint16_t* __restrict__ a,
                                                   const uint16_t* __restrict__ b,
                                                   uint16_t* __restrict__ out, int64_t R,
                                                   int64_t K) {
  const int64_t nkb = K / 32, slots = R * K / 8;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < slots;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tile = c >> 6;
    const int L = (int)(c & 63);
    const int64_t rb = tile / nkb, kb = tile % nkb;
    const int64_t r = rb * 16 + (L & 15), k = kb * 32 + (L >> 4) * 8;
    const uint16_t* src = b ? ((r & 1) ? b + (r >> 1) * K : a + (r >> 1) * K) : a + r * K;
    st16(out + c * 8, ld16_stream(src + k));
  }
}

static hipError_t launch_tile(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t R,
                              int64_t K, hipStream_t stream) {
  const int64_t blocks = (R * K / 8 + 255) / 256;
  launch_kernel(KK_PACK, k_tile_bf16, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                dim3(256), 0, stream, a, b, out, R, K);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w_gate, const uint16_t* w_up, uint16_t* w_gu, int64_t ff,
                       int64_t d, hipStream_t stream) {
  return launch_tile(w_gate, w_up, w_gu, 2 * ff, d, stream);
}

hipError_t launch_tile_matrix(const uint16_t* w, uint16_t* out, int64_t R, int64_t K,
                              hipStream_t stream) {
  return launch_tile(w, nullptr, out, R, K, stream);
}

// ---------------------------------------------------------------- fp16 weights
__device__ int g_f16_range_error;

__global__ void k_f16_flag_reset() { g_f16_range_error = 0; }

// bf16 -> fp16 by truncation toward zero, 8 elements per thread: the same
// conversion the prefill GEMM applies to bf16 weight fragments in registers
// (bf16x8_to_f16x8), so a forward on the converted weights reads the values
// that one on the bf16 weights does. Non-finite values and magnitudes above
// 65504 raise the range flag (NaN fails the comparison as well).
__global__ __launch_bounds__(256) void k_convert_f16(const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n8) return;
  const u32x4 v = ld16(w + t * 8);
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ok = ok && fabsf(bf16_lo(v[j])) <= 65504.0f && fabsf(bf16_hi(v[j])) <= 65504.0f;
  if (!ok) atomicOr(&g_f16_range_error, 1);
  st16(out + t * 8, bf16x8_to_f16x8(v));
}

hipError_t launch_convert_f16(const uint16_t* w, uint16_t* out, int64_t n, hipStream_t stream,
                              int* range_error) {
  hipLaunchKernelGGL(k_f16_flag_reset, dim3(1), dim3(1), 0, stream);
  const int64_t n8 = n / 8;
  launch_kernel(KK_CONVERT_F16, k_convert_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0,
                stream, w, out, n8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int flag = 0;
  e = hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_f16_range_error), sizeof(int), 0,
                               hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  *range_error = flag;
  return e;
}

// ---------------------------------------------------------------- int4
// Exchange format (row-major, what callers hold): codes q uint8 [R, K/2],
// column k in byte k/2, even k in the low nibble, two's complement; scales
// fp16 [R, K/32], one per group of 32 consecutive columns of a row.
__device__ int g_quant_range_error;

__global__ void k_quant_flag_reset() { g_quant_range_error = 0; }

// One thread per (row, group), consecutive threads along a row's groups.
// s = fp16_rne(max|w| / 7) with IEEE fp32 division; q = clamp(rint(w / s),
// -8, 7) with rint rounding half to even; q = 0 when s == 0.
__global__ __launch_bounds__(256) void k_quantize_int4(const uint16_t* __restrict__ w, int64_t R,
                                                       int64_t K, uint8_t* __restrict__ q,
                                                       uint16_t* __restrict__ sc) {
  const int64_t ng = K / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= R * ng) return;
  const int64_t r = t / ng, g = t - r * ng;
  float f[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 v = ld16(w + r * K + g * 32 + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[c * 8 + 2 * j] = bf16_lo(v[j]);
      f[c * 8 + 2 * j + 1] = bf16_hi(v[j]);
    }
  }
  float mx = 0.0f;
  bool finite = true;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    finite = finite && __builtin_isfinite(f[k]);
    mx = fmaxf(mx, fabsf(f[k]));
  }
  const _Float16 sh = (_Float16)__fdiv_rn(mx, 7.0f);
  const float s = (float)sh;
  if (!finite || __builtin_isinf(s)) {
    atomicOr(&g_quant_range_error, 1);
    return;
  }
  sc[r * ng + g] = __builtin_bit_cast(uint16_t, sh);
  u32x4 out;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t word = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      int qi = 0;
      if (s != 0.0f) {
        const float rq = rintf(__fdiv_rn(f[c * 8 + m], s));
        qi = (int)fminf(fmaxf(rq, -8.0f), 7.0f);
      }
      word |= (uint32_t)(qi & 0xF) << (4 * m);
    }
    out[c] = word;
  }
  st16(q + r * (K / 2) + g * 16, out);
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, uint8_t* q,
                           uint16_t* scales, hipStream_t stream, int* range_error) {
  hipLaunchKernelGGL(k_quant_flag_reset, dim3(1), dim3(1), 0, stream);
  const int64_t threads = rows * (K / 32);
  launch_kernel(KK_QUANTIZE, k_quantize_int4, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                0, stream, w, rows, K, q, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int flag = 0;
  e = hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_quant_range_error), sizeof(int), 0,
                               hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  *range_error = flag;
  return e;
}

// One thread per (row, group): out[r, 32g + k] = float(s) * float(q), exact.
__global__ __launch_bounds__(256) void k_dequant_int4(const uint8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ sc, int64_t R,
                                                      int64_t K, float* __restrict__ out) {
  const int64_t ng = K / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= R * ng) return;
  const int64_t r = t / ng, g = t - r * ng;
  const float s = (float)__builtin_bit_cast(_Float16, sc[r * ng + g]);
  const u32x4 words = ld16(q + r * (K / 2) + g * 16);
  float* o = out + r * K + g * 32;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float v[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int nib = (int)((words[c] >> (4 * m)) & 0xF);
      v[m] = s * (float)(nib >= 8 ? nib - 16 : nib);
    }
    st16(o + c * 8, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3])});
    st16(o + c * 8 + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]),
                              __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
}

hipError_t launch_dequant(const uint8_t* q, const uint16_t* s, int64_t R, int64_t K, float* out,
                          hipStream_t stream) {
  const int64_t threads = R * (K / 32);
  launch_kernel(KK_DEQUANT, k_dequant_int4, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                stream, q, s, R, K, out);
  return hipGetLastError();
}

// Row-major int4 -> the tiled int4 layout (file comment). One thread per
// 16-byte slot L of super-tile (rb, sq): row r = 16 rb + L % 16, word j the 8
// codes of group 4 sq + j at columns 8 (L / 16) .. +7, i.e. the 4 bytes of
// the row-major row at byte (32 (4 sq + j) + 8 (L / 16)) / 2. Threads with
// L < 16 also write their row's 4 scales of the super-tile. Groups past K/32
// get zero codes and scales. With qb non-null the logical matrix is the row
// interleave of a (even rows) and b (odd rows), [2 Ra, K]: the gate/up
// interleave of FastTPS review section 3 item 3 and the llama.cpp PR digest,
// applied to quantised rows (quantisation groups never cross rows).
__global__ __launch_bounds__(256) void k_tile_int4(const uint8_t* __restrict__ qa,
                                                   const uint16_t* __restrict__ sa,
                                                   const uint8_t* __restrict__ qb,
                                                   const uint16_t* __restrict__ sb, int64_t R,
                                                   int64_t K, uint8_t* __restrict__ qt,
                                                   uint16_t* __restrict__ st) {
  const int64_t nq = (K + 127) / 128, ng = K / 32;
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= (R / 16) * nq * 64) return;
  const int L = (int)(c & 63);
  const int64_t tile = c >> 6, rb = tile / nq, sq = tile - rb * nq;
  const int64_t r = rb * 16 + (L & 15);
  const int64_t src_row = qb ? (r >> 1) : r;
  const uint8_t* qrow = (qb && (r & 1) ? qb : qa) + src_row * (K / 2);
  const uint16_t* srow = (qb && (r & 1) ? sb : sa) + src_row * ng;
  u32x4 o;
  uint16_t sv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t g = sq * 4 + j;
    const bool real = g < ng;
    o[j] = real ? *reinterpret_cast<const uint32_t*>(qrow + (g * 32 + (L >> 4) * 8) / 2) : 0u;
    sv[j] = real ? srow[g] : (uint16_t)0;
  }
  st16(qt + c * 16, o);
  if (L < 16) {
    uint16_t* d = st + tile * 64 + L * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = sv[j];
  }
}

hipError_t launch_tile_int4(const uint8_t* qa, const uint16_t* sa, const uint8_t* qb,
                            const uint16_t* sb, int64_t R, int64_t K, uint8_t* qt, uint16_t* st,
                            hipStream_t stream) {
  const int64_t threads = (R / 16) * ((K + 127) / 128) * 64;
  launch_kernel(KK_PACK, k_tile_int4, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                stream, qa, sa, qb, sb, R, K, qt, st);
  return hipGetLastError();
}

}  // namespace fmlp
