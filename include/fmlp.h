/*
 * fmlp.h -- C ABI of libfmlp.so: the fused gated (SwiGLU) MLP with an RMSNorm
 * prologue, for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The operation (FastTPS review, xllm-io paper-review blog, section 3
 * "technical architecture", Eq(1), and the MLP-block flow / Figure 4 on the
 * same page):
 *
 *     n_m   = gamma * x_m / sqrt(mean_k(x_mk^2) + eps)          (RMSNorm, part1)
 *     z_m   = W_gu n_m        (gate and up rows interleaved, part2)
 *     a_mi  = SiLU(z_m[2i]) * z_m[2i+1],  SiLU(t) = t / (1 + e^-t)
 *     y_m   = W_down a_m                                         (part3)
 *
 * i.e. y = W_down(SiLU(W_gate n) * (W_up n)), with the gate/up matrices stored
 * as one row-interleaved matrix (llama.cpp PR digest on blog.cecily.jp: gate
 * and up rows alternate so one matmul pass produces both, and the GLU is
 * applied in that same pass).
 *
 * Conventions for every entry point:
 *   - Every buffer pointer is a caller-owned DEVICE pointer (hipMalloc'd or a
 *     torch CUDA tensor's data_ptr) on the current HIP device, 16-byte
 *     aligned. The library never allocates, frees or keeps a pointer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream). Work is enqueued asynchronously on it; only
 *     fmlp_quantize_int4 synchronises (it must report fp16 scale overflow).
 *   - Matrices are row-major, nn.Linear-shaped [out_features, in_features].
 *     bf16 / fp16 values are raw 16-bit IEEE patterns.
 *   - Return value: FMLP_OK (0) or a negative fmlp_status. Argument checks
 *     run on the host before any HIP call; a failed launch returns
 *     FMLP_ERR_HIP and records the hipError_t for fmlp_last_hip_error().
 *     Faults inside a kernel surface at the caller's next synchronisation,
 *     as for any HIP kernel. Nothing aborts, throws or prints.
 *   - Shapes: d and ff are positive multiples of 32 (the int4 group and
 *     the 16-byte load width), d <= 65536, ff <= 262144, 0 <= M <= 2^24.
 *   - Thread safety: all entry points may be called from several host
 *     threads; calls on one stream execute in order.
 */
#ifndef FMLP_H_
#define FMLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fmlp_status {
  FMLP_OK = 0,
  FMLP_ERR_INVALID_ARG = -1,       /* null pointer, bad eps, aliasing, bad enum */
  FMLP_ERR_UNSUPPORTED_SHAPE = -2, /* d/ff/M outside the limits above */
  FMLP_ERR_ALIGNMENT = -3,         /* a pointer is not 16-byte aligned */
  FMLP_ERR_WORKSPACE = -4,         /* workspace smaller than fmlp_workspace_size */
  FMLP_ERR_RANGE = -5,             /* int4 scale or fp16 weight out of fp16 range */
  FMLP_ERR_HIP = -6,               /* a HIP runtime call or launch failed */
  FMLP_ERR_DEVICE = -7             /* current device is not gfx950 */
};

enum fmlp_wtype {
  FMLP_W_BF16 = 0,     /* bf16 weights */
  FMLP_W_INT4_G32 = 1, /* int4 codes + fp16 scales, groups of 32 along K */
  FMLP_W_F16 = 2       /* fp16 weights (fmlp_convert_f16 of the bf16 tiles) */
};

enum fmlp_path {
  FMLP_PATH_AUTO = 0,    /* decode kernels for M <= 32, MFMA GEMMs above */
  FMLP_PATH_DECODE = 1,  /* force the decode (weight-streaming) kernels; M <= 32 */
  FMLP_PATH_PREFILL = 2, /* force the tiled MFMA GEMM path; any M */
  FMLP_PATH_SINGLE_PASS = 3 /* force the single-pass decode: gate/up, SiLU*mul,
                               down and the cross-workgroup sum of per-slice
                               partials in one launch (FastTPS review,
                               section 3, Fusion MLP); bf16 weights, M <= 8.
                               Its arrival counters are library-owned device
                               memory: single-pass calls must not overlap in
                               time on one GPU */
};

/*
 * Gate activations. The kernels evaluate the logistic function with the
 * hardware exponential and reciprocal (about 1 ulp each; the tanh form
 * through 0.5 (1 + tanh y) = sigma(2 y)) and erf by Abramowitz and Stegun's
 * formula 7.1.26 (absolute error below 1.5e-7), in fp32; each product a is
 * then rounded to fp16 (or kept as a bf16 hi + lo pair on the bf16 decode
 * path at M <= 16).
 */
enum fmlp_activation {
  FMLP_ACT_SILU = 0,      /* SiLU(t) = t / (1 + e^-t): Eq(1), the default */
  FMLP_ACT_GELU_TANH = 1, /* 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))) */
  FMLP_ACT_GELU_ERF = 2   /* 0.5 t (1 + erf(t / sqrt 2)) = t Phi(t) */
};

/*
 * Weight storage. The library keeps every weight matrix in a
 * "fragment-tiled" layout: a storage permutation of the logical row-major
 * nn.Linear matrix, chosen so each 16-row x 32-column block is one
 * contiguous 1024-byte tile that a wave64 reads with one 16-byte load per
 * lane straight into the MFMA 16x16x32 operand layout.
 *
 * Tiled bf16, logical W [R, K], R % 16 == 0, K % 32 == 0: element (r, k) is
 * stored at element index
 *     ((r/16)*(K/32) + k/32)*512 + (((k%32)/8)*16 + r%16)*8 + k%8.
 *
 * Tiled int4, logical codes q [R, K] (two's complement, -8..7) and fp16
 * scales s [R, K/32] (one per group of 32 consecutive columns), with
 * nq = ceil(K/128): code (r, k) of group g = k/32 is nibble k%8 (bits
 * 4*(k%8) .. +3) of 32-bit word ((r/16)*nq + g/4)*256 + (((k%32)/8)*16 +
 * r%16)*4 + g%4; scale (r, g) is fp16 element ((r/16)*nq + g/4)*64 +
 * (r%16)*4 + g%4. Groups past K/32 in the last super-tile of 4 groups hold
 * zero codes and zero scales. Buffer sizes: fmlp_int4_sizes.
 */

/*
 * Interleave gate and up weights into one matrix (the "one big matmul" of
 * FastTPS Fusion MLP, FastTPS review section 3 item 3; row interleave as in
 * the llama.cpp PR digest) and store it tiled.
 *   w_gate, w_up : bf16 [ff, d] row-major, read only.
 *   w_gu         : tiled bf16 of the logical [2ff, d] matrix whose row 2i is
 *                  w_gate row i and row 2i+1 is w_up row i. Bit copies.
 *   w_gu must not overlap either input (FMLP_ERR_INVALID_ARG).
 */
int fmlp_pack_interleaved(const void* w_gate, const void* w_up, void* w_gu,
                          int64_t ff, int64_t d, void* stream);

/*
 * Store a bf16 row-major matrix [rows, K] tiled (used for W_down [d, ff]).
 * rows % 16 == 0, K % 32 == 0; w_tiled (rows*K bf16) must not overlap w.
 */
int fmlp_pack_matrix(const void* w, void* w_tiled, int64_t rows, int64_t K,
                     void* stream);

/*
 * int4 exchange format (row-major, what a caller holds or receives from
 * fmlp_quantize_int4): for a logical matrix [rows, K], K % 32 == 0,
 *   q      : uint8 [rows, K/2]; column k is nibble k%2 of byte k/2 (even k
 *            in the low nibble, odd k in the high one), two's complement,
 *            values -8..7;
 *   scales : fp16 [rows, K/32]; scale (r, g) applies to columns 32g..32g+31
 *            of row r, so w[r, k] = scales[r, k/32] * q[r, k].
 * The pages only name Q4_K / Q4_K_M (llama.cpp PR digest, blog.cecily.jp);
 * this is the plainest symmetric group format. fmlp_forward reads int4 in
 * the tiled layout above, written from this format by fmlp_pack_int4_*.
 */

/* Byte sizes of the tiled int4 code and scale buffers of a [rows, K] matrix. */
int fmlp_int4_sizes(int64_t rows, int64_t K, size_t* code_bytes,
                    size_t* scale_bytes);

/*
 * Quantise a bf16 row-major matrix [rows, K] to the int4 exchange format,
 * one fp16 scale per group of 32 consecutive elements of a row:
 *   s = fp16_rne( fp32(max_group |w|) / 7 )      (IEEE fp32 division)
 *   q = clamp( round_half_even( fp32(w) / fp32(s) ), -8, 7 ),  q = 0 if s == 0
 *   w      : bf16 [rows, K] row-major, read only.
 *   q      : uint8 [rows, K/2], scales : fp16 [rows, K/32] (exchange format).
 *   rows >= 1 (no row blocking), K % 32 == 0; buffers must not overlap.
 * Synchronises `stream`. Returns FMLP_ERR_RANGE if some group holds a
 * non-finite weight or its scale overflows fp16 (outputs then undefined).
 * Groups never cross rows, so quantising the row-interleaved gate/up matrix
 * equals interleaving the quantised gate and up matrices.
 */
int fmlp_quantize_int4(const void* w, int64_t rows, int64_t K, void* q,
                       void* scales, void* stream);

/*
 * Interleave quantised gate and up weights into one matrix and store it in
 * the tiled int4 layout (the int4 counterpart of fmlp_pack_interleaved:
 * FastTPS review section 3 item 3, one matmul over interleaved gate/up rows;
 * llama.cpp PR digest, gate and up rows alternate).
 *   q_gate, q_up : uint8 [ff, d/2];  s_gate, s_up : fp16 [ff, d/32]
 *                  (exchange format), read only.
 *   q_gu, s_gu   : tiled codes and scales of the logical [2ff, d] matrix
 *                  whose row 2i is gate row i and row 2i+1 is up row i;
 *                  sizes from fmlp_int4_sizes(2ff, d). Bit copies.
 * d, ff as for fmlp_forward. Outputs must not overlap any input or each
 * other (FMLP_ERR_INVALID_ARG). Asynchronous.
 */
int fmlp_pack_int4_interleaved(const void* q_gate, const void* s_gate,
                               const void* q_up, const void* s_up, int64_t ff,
                               int64_t d, void* q_gu, void* s_gu, void* stream);

/*
 * Store an int4 matrix given in the exchange format [rows, K] (used for
 * W_down [d, ff]) in the tiled int4 layout. rows % 16 == 0, K % 32 == 0;
 * q_tiled / s_tiled sized by fmlp_int4_sizes(rows, K), not overlapping the
 * inputs or each other. Asynchronous.
 */
int fmlp_pack_int4_matrix(const void* q, const void* scales, int64_t rows,
                          int64_t K, void* q_tiled, void* s_tiled,
                          void* stream);

/*
 * Convert bf16 weights to fp16 for the FMLP_W_F16 weight type: element i of
 * out is the fp16 value of largest magnitude not above that of w[i], with its
 * sign (truncation toward zero). Every bf16 value in the fp16 normal range
 * [2^-14, 65504] is exact in fp16, so only magnitudes below 2^-14 round,
 * exactly as the MFMA prefill path rounds bf16 weights before its fp16
 * products; a forward on the converted weights therefore takes the same
 * values as one on the bf16 weights there. Element-wise, so it applies to
 * the tiled matrices (fmlp_pack_interleaved, fmlp_pack_matrix) as to any
 * other layout. A storage option: the prefill GEMMs' fp16 products then
 * read the weights as they are, with no conversion in the inner loop.
 *   w    : bf16 [n], read only.     out : fp16 [n]; must not overlap w.
 *   n    : element count, a positive multiple of 8, at most (2^31 - 1) * 2048
 *          (FMLP_ERR_UNSUPPORTED_SHAPE above).
 * Synchronises `stream`. Returns FMLP_ERR_RANGE if some w[i] is not finite
 * or exceeds 65504 in magnitude (out then undefined).
 */
int fmlp_convert_f16(const void* w, void* out, int64_t n, void* stream);

/*
 * Expand int4 in the exchange format to row-major fp32 [rows, K]:
 * out[r,k] = float(scales[r,k/32]) * q[r,k], exact in fp32. A test hook for
 * the expansion the int4 forward kernels perform in registers; not used by
 * fmlp_forward. rows >= 1, K % 32 == 0; out must not overlap the inputs.
 */
int fmlp_dequant_int4(const void* q, const void* scales, int64_t rows,
                      int64_t K, float* out, void* stream);

/*
 * Bytes of scratch fmlp_forward needs for this problem (for any path it may
 * take, fmlp_forward_path's forced ones included), or 0 when the shape is
 * unsupported. Depends only on the arguments, and never decreases as M grows
 * with d, ff and wtype fixed, so a buffer sized for the largest M serves
 * every smaller one.
 */
size_t fmlp_workspace_size(int64_t M, int64_t d, int64_t ff, int32_t wtype);

/*
 * y = W_down( SiLU(W_gate n) * (W_up n) ),  n = RMSNorm(x; gamma, eps),
 * computed row by row of x (rows are independent).
 *   x          : bf16 [M, d]          gamma : bf16 [d]
 *   eps        : finite, >= 0 (added to mean(x^2) inside the square root)
 *   wtype      : FMLP_W_BF16: w_gu tiled bf16 [2ff, d] (fmlp_pack_interleaved),
 *                             w_down tiled bf16 [d, ff] (fmlp_pack_matrix);
 *                             gu_scales and down_scales ignored (may be NULL)
 *                FMLP_W_INT4_G32: tiled int4 codes + scales of the same two
 *                             logical matrices (fmlp_quantize_int4, then
 *                             fmlp_pack_int4_interleaved for W_gu and
 *                             fmlp_pack_int4_matrix for W_down). Decode
 *                             (M <= 32) dequantises in registers, exactly;
 *                             prefill dequantises inside its GEMMs, each
 *                             weight fp16(s*q) (the exact product rounded
 *                             once to nearest even) right before its MFMAs,
 *                             with no expanded copy and no extra workspace
 *                FMLP_W_F16: w_gu and w_down as for FMLP_W_BF16, converted
 *                             by fmlp_convert_f16; scales ignored. Decode
 *                             takes fp16 n and a at every M (one RMSNorm
 *                             launch before gate/up); prefill runs its fp16
 *                             products on them directly
 *   y          : bf16 [M, d], written (round to nearest even); must not
 *                overlap any other buffer.
 *   workspace  : device scratch of at least fmlp_workspace_size(M,d,ff,wtype)
 *                bytes; contents on entry are ignored, on exit undefined.
 *   M == 0 is a no-op returning FMLP_OK (x and y may then be NULL).
 * Accumulation is fp32. The normalised input and the SiLU*mul intermediate
 * are kept as bf16 hi + lo pairs (about 2^-17 relative, the range of fp32)
 * on the bf16 decode path up to 16 tokens, and as fp16 on every other path
 * (the prefill path also converts bf16 weights to fp16 the way
 * fmlp_convert_f16 does, and int4 weights to fp16(s*q) as above). On those paths an intermediate beyond +-65504
 * becomes +-inf, so that row of y comes out non-finite (inf or NaN), never
 * a finite wrong value; magnitudes below 2^-14 lose relative precision
 * gradually (fp16 subnormals).
 * Not bitwise identical across paths; deterministic for a given path and
 * shape. Concurrent calls must not share a workspace.
 */
int fmlp_forward(const void* x, const void* gamma, float eps, int32_t wtype,
                 const void* w_gu, const void* gu_scales, const void* w_down,
                 const void* down_scales, void* y, int64_t M, int64_t d,
                 int64_t ff, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * fmlp_forward with the kernel path chosen by the caller (enum fmlp_path);
 * used to test both paths at the same shapes, for either weight type.
 * FMLP_PATH_DECODE with M > 32, and FMLP_PATH_SINGLE_PASS with M > 8 or
 * weights other than bf16, return FMLP_ERR_UNSUPPORTED_SHAPE.
 */
int fmlp_forward_path(const void* x, const void* gamma, float eps,
                      int32_t wtype, const void* w_gu, const void* gu_scales,
                      const void* w_down, const void* down_scales, void* y,
                      int64_t M, int64_t d, int64_t ff, void* workspace,
                      size_t workspace_bytes, void* stream, int32_t path);

/*
 * fmlp_forward_path with two variants of the layer around Eq(1), both from
 * the Together AI fusion post (blog.hotdry.top), which fuses a GELU MLP and
 * fuses the residual add into the next normalisation:
 *   activation : gate activation, enum fmlp_activation (FMLP_ACT_SILU is
 *                Eq(1) of the FastTPS review; the GELU forms make the GeGLU
 *                variant: a = GELU(W_gate n) * (W_up n)).
 *   residual   : NULL, or bf16 [M, d], the previous sublayer's output r.
 *                Then the row normalised is the residual stream
 *                h = bf16_rne(x + r) (correctly rounded), and
 *   h_out      : bf16 [M, d] receives h; NULL exactly when residual is NULL.
 *                It must not overlap x, residual, gamma, the weights, y or
 *                the workspace (it is written while they are read).
 * Other arguments, errors and paths as fmlp_forward_path; an unknown
 * activation, or only one of residual / h_out given, is
 * FMLP_ERR_INVALID_ARG. The workspace size does not depend on either.
 */
int fmlp_forward_ex(const void* x, const void* residual, void* h_out, const void* gamma,
                    float eps, int32_t activation, int32_t wtype, const void* w_gu,
                    const void* gu_scales, const void* w_down, const void* down_scales, void* y,
                    int64_t M, int64_t d, int64_t ff, void* workspace, size_t workspace_bytes,
                    void* stream, int32_t path);

/*
 * fmlp_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Arguments, path choice, results and errors are those of
 * fmlp_forward (the same kernels on the same path, so y is bitwise the
 * same), except that the scratch is a fixed device array inside the library,
 * FMLP_NOALLOC_SCRATCH_BYTES long, that each GPU the library runs on holds
 * until the process ends. A problem whose automatic path needs more scratch
 * returns FMLP_ERR_WORKSPACE; fmlp_workspace_size(M, d, ff, wtype) <=
 * FMLP_NOALLOC_SCRATCH_BYTES guarantees it fits (every decode problem of up
 * to 32 tokens with d <= 8192 and ff <= 28672 does). The call allocates and
 * frees nothing. Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents (each call clears what it needs cleared), so calls
 * that overlap in time on one GPU (several host threads, or several streams
 * without ordering between them) race and must not be made.
 */
#define FMLP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fmlp_forward_noalloc(const void* x, const void* gamma, float eps,
                         int32_t wtype, const void* w_gu, const void* gu_scales,
                         const void* w_down, const void* down_scales, void* y,
                         int64_t M, int64_t d, int64_t ff, void* stream);

/*
 * Per-kernel timing (measurement support, not needed for computing).
 * fmlp_profile_enable(1) discards earlier records and starts launching every
 * kernel of the library with a pair of HIP events that the runtime stamps at
 * the dispatch's start and end on its stream; fmlp_profile_enable(0) stops recording (records are
 * kept until the next enable). fmlp_profile_read synchronises the recorded
 * events of one kernel kind and returns how many launches were recorded and
 * their summed GPU time in milliseconds. Kinds are 0 .. n-1 in the order of
 * fmlp_kernel_name, which returns NULL past the last kind. Events add a
 * little GPU time per launch, so timing runs should be separate from
 * throughput runs.
 */
int fmlp_profile_enable(int32_t on);

/*
 * Streaming-read probe (measurement support, not part of the computation):
 * reads `bytes` of device memory at src once, with 16-byte nontemporal loads
 * in a grid-stride loop over `workgroups` workgroups of 256 threads, and
 * stores one 32-bit XOR of its reads per thread to sink (workgroups*256
 * words, caller-owned). It gives the HBM read rate that a kernel reading the
 * same number of bytes per launch can reach, the yardstick for the weight
 * streams of the decode kernels. Timed like the other kernels while
 * profiling is enabled (kind "read_probe"). src 16-byte aligned, bytes a
 * multiple of 16, sink 4-byte aligned; else FMLP_ERR_ALIGNMENT. Asynchronous.
 */
int fmlp_read_probe(const void* src, int64_t bytes, void* sink, int32_t workgroups,
                    void* stream);
int fmlp_profile_read(int32_t kind, int64_t* launches, double* total_ms);
const char* fmlp_kernel_name(int32_t kind);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fmlp_status_string(int status);

/* hipError_t of this thread's most recent FMLP_ERR_HIP (0 if none). */
int fmlp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FMLP_H_ */
