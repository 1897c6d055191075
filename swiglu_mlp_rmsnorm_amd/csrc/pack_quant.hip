// Weight preparation kernels: gate/up row interleave, int4 group-32
// quantisation and the int4 -> fp32 expansion test hook.
#include "device_common.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace fmlp {

// ---------------------------------------------------------------- packing
// FastTPS review, section 3 item 3 (gate/up merged into one interleaved
// matmul); llama.cpp PR digest (gate and up rows alternate).
// Thread i copies one 16-byte chunk of the output; output row 2r comes from
// gate row r, row 2r+1 from up row r.
__global__ __launch_bounds__(256) void k_pack_interleaved(const uint16_t* __restrict__ w_gate,
                                                          const uint16_t* __restrict__ w_up,
                                                          uint16_t* __restrict__ w_gu,
                                                          int64_t ff, int64_t chunks_per_row) {
  const int64_t total = 2 * ff * chunks_per_row;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t out_row = c / chunks_per_row, ch = c % chunks_per_row;
    const uint16_t* src = (out_row & 1) ? w_up : w_gate;
    const u32x4 v = ld16_stream(src + ((out_row >> 1) * chunks_per_row + ch) * 8);
    st16(w_gu + c * 8, v);
  }
}

hipError_t launch_pack(const uint16_t* w_gate, const uint16_t* w_up, uint16_t* w_gu, int64_t ff,
                       int64_t d, hipStream_t stream) {
  const int64_t chunks = 2 * ff * (d / 8);
  const int64_t blocks = (chunks + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  ProfileScope prof(KK_PACK, stream);
  hipLaunchKernelGGL(k_pack_interleaved, dim3(grid), dim3(256), 0, stream, w_gate, w_up, w_gu, ff,
                     d / 8);
  return hipGetLastError();
}

// ---------------------------------------------------------------- int4
// Set when some group has a non-finite weight or its fp16 scale overflows.
__device__ int g_quant_range_error;

__global__ void k_quant_flag_reset() { g_quant_range_error = 0; }

// One thread per (row, group of 32): s = fp16_rne(max|w| / 7) with IEEE fp32
// division, q = clamp(rint(w / s), -8, 7) (rint: half to even), q = 0 when
// s == 0. Nibble k%2==0 is the low half of byte k/2.
__global__ __launch_bounds__(256) void k_quantize_int4(const uint16_t* __restrict__ w,
                                                       int64_t groups_total,
                                                       uint8_t* __restrict__ q,
                                                       uint16_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups_total) return;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(w + g * 32 + i * 8);
  float f[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[i * 8 + 2 * j] = bf16_lo(v[i][j]);
      f[i * 8 + 2 * j + 1] = bf16_hi(v[i][j]);
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
  scales[g] = __builtin_bit_cast(uint16_t, sh);
  uint32_t packed[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int qi = 0;
      if (s != 0.0f) {
        const float r = rintf(__fdiv_rn(f[i * 8 + j], s));
        qi = (int)fminf(fmaxf(r, -8.0f), 7.0f);
      }
      word |= (uint32_t)(qi & 0xF) << (4 * j);
    }
    packed[i] = word;
  }
  u32x4 out = {packed[0], packed[1], packed[2], packed[3]};
  st16(q + g * 16, out);
}

hipError_t launch_quantize(const uint16_t* w, int64_t rows, int64_t K, uint8_t* q,
                           uint16_t* scales, hipStream_t stream, int* range_error) {
  hipLaunchKernelGGL(k_quant_flag_reset, dim3(1), dim3(1), 0, stream);
  const int64_t groups = rows * (K / 32);
  {
    ProfileScope prof(KK_QUANTIZE, stream);
    hipLaunchKernelGGL(k_quantize_int4, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                       stream, w, groups, q, scales);
  }
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

// One thread per 8 codes (one 32-bit word): out = float(s) * float(q), exact.
__global__ __launch_bounds__(256) void k_dequant_int4(const uint8_t* __restrict__ q,
                                                      const uint16_t* __restrict__ scales,
                                                      int64_t words_total, float* __restrict__ out) {
  const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= words_total) return;
  const uint32_t word = reinterpret_cast<const uint32_t*>(q)[wi];
  const float s = (float)__builtin_bit_cast(_Float16, scales[wi / 4]);  // 4 words per group
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int nib = (int)((word >> (4 * j)) & 0xF);
    r[j] = s * (float)(nib >= 8 ? nib - 16 : nib);
  }
  u32x4 a = {__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]),
             __float_as_uint(r[3])};
  u32x4 b = {__float_as_uint(r[4]), __float_as_uint(r[5]), __float_as_uint(r[6]),
             __float_as_uint(r[7])};
  st16(out + wi * 8, a);
  st16(out + wi * 8 + 4, b);
}

hipError_t launch_dequant(const uint8_t* q, const uint16_t* scales, int64_t rows, int64_t K,
                          float* out, hipStream_t stream) {
  const int64_t words = rows * (K / 8);
  ProfileScope prof(KK_DEQUANT, stream);
  hipLaunchKernelGGL(k_dequant_int4, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, q,
                     scales, words, out);
  return hipGetLastError();
}

}  // namespace fmlp
