/*
 * qlq.h - C ABI of libqlq, a weight-quantized linear layer for AMD MI355X
 * (gfx950):  y = x . dequant(W)^T + b  computed from packed low-bit codes.
 *
 * Three weight formats are supported:
 *   - group-wise affine n-bit weights ("Struct QuantizedLinear", nuvec-nn
 *     docs: packed uint32 weight [N, K*bits/32], per-group scales and biases
 *     [N, K/group_size], w = scale*q + bias as in the MLX affine format quoted
 *     in the pergroup_linear docstring of "cider/ops.py");
 *   - ternary BitLinear ("mlx-lm/mlx_lm/models/bitlinear_layers.py": uint8
 *     [N/4, K], four 2-bit codes per byte across output rows, code c meaning
 *     c - 1, one per-tensor weight scale);
 *   - per-channel symmetric W8A8 ("cider/ops.py", perchannel_linear and
 *     int8_matmul_int32).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns an int status (QLQ_OK == 0) and never throws.
 *    qlq_last_error() returns a thread-local message about the last failure.
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, to a
 *    contiguous row-major array.  The library never allocates, frees or keeps
 *    these pointers.  Forward calls allocate no device memory at all; where
 *    temporary device memory is needed the caller passes a workspace whose
 *    size a *_workspace_size() function returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous: they validate their arguments on the host,
 *    enqueue kernels on `stream` and return.  Device faults surface at the
 *    caller's next synchronisation.  The exceptions are qlq_pack and
 *    bitlinear_pack, which synchronise `stream` to report data errors.
 *  - Argument validation (null pointers, sizes, supported bit widths, group
 *    sizes and dtypes, 16-byte alignment of tensor pointers) happens before
 *    any HIP call, so an invalid call has no device side effect.
 *  - An empty batch (M == 0 rows of x, R == 0 rows to quantize) is a valid
 *    call that does nothing; the pointers of the empty tensors (x and y, or
 *    the rows and their outputs) may then be NULL.
 *  - Dtype codes: QLQ_F32, QLQ_F16, QLQ_BF16 (IEEE binary32, binary16, and
 *    bfloat16 = the top half of a binary32).  Narrowing to a storage dtype is
 *    round-to-nearest-even.
 */
#ifndef QLQ_H
#define QLQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QLQ_API __attribute__((visibility("default")))
#else
#define QLQ_API
#endif

enum qlq_status {
  QLQ_OK = 0,
  QLQ_ERR_INVALID_ARG = 1, /* null pointer, non-positive or inconsistent size */
  QLQ_ERR_UNSUPPORTED = 2, /* bits / group size / dtype combination not built  */
  QLQ_ERR_DTYPE = 3,       /* dtype mismatch between related tensors          */
  QLQ_ERR_ALIGNMENT = 4,   /* a tensor pointer is not 16-byte aligned         */
  QLQ_ERR_WORKSPACE = 5,   /* workspace missing or too small                  */
  QLQ_ERR_DATA = 6,        /* non-finite weight / parameter, value out of set */
  QLQ_ERR_DEVICE = 7,      /* current device is not gfx950                    */
  QLQ_ERR_HIP = 8          /* HIP runtime or launch error                     */
};

enum qlq_dtype { QLQ_F32 = 0, QLQ_F16 = 1, QLQ_BF16 = 2 };

/* ------------------------------------------------------------------------
 * Group-wise affine n-bit weights
 * ------------------------------------------------------------------------ */

/*
 * qlq_pack - quantize fp32 weights group-wise and pack the codes.
 * ("Struct QuantizedLinear", from_linear and Fields; affine formula of the
 *  pergroup_linear docstring in "cider/ops.py".)
 *
 *   w       [N, K] fp32, finite.
 *   packed  [N, K*bits/32] uint32 (out).  A row's codes form one bit stream,
 *           least significant bit first: code k fills stream bits
 *           bits*k .. bits*k + bits - 1, and stream bit i is bit i mod 32 of
 *           word i / 32.  For bits in {1, 2, 4, 8} this puts code k at bit
 *           offset bits*(k mod (32/bits)) of word k / (32/bits); 3-, 5- and
 *           6-bit codes may straddle two words.
 *   scales, biases  [N, K/group_size] of sb_dtype (out).
 *
 * Per group of group_size consecutive K values: mn, mx = fp32 min and max;
 * scale = (mx - mn) / (2^bits - 1) and bias = mn, both in fp32 and rounded to
 * sb_dtype; a zero stored scale becomes 1; q = clamp(rint((w - bias)/scale),
 * 0, 2^bits - 1) with the subtraction and the division in fp32 against the
 * stored scale and bias (rint rounds half to even).
 *
 * bits in {1, ..., 6, 8}; group_size in {32, 64, 128}; K % group_size == 0.
 * Synchronises `stream`.  Returns QLQ_ERR_DATA (outputs unspecified) if a
 * weight is not finite or a stored scale/bias overflows sb_dtype.
 */
QLQ_API int qlq_pack(const float* w, int64_t N, int64_t K, int bits, int group_size,
                     uint32_t* packed, void* scales, void* biases, int sb_dtype,
                     void* stream);

/*
 * qlq_unpack - packed [N, K*bits/32] uint32 -> codes [N, K] uint8 (one code
 * per byte).  Bit-exact inverse of the packing described under qlq_pack.
 * bits in {1, ..., 6, 8}; K*bits % 32 == 0 (QLQ_ERR_INVALID_ARG otherwise).
 */
QLQ_API int qlq_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits,
                       uint8_t* codes, void* stream);

/*
 * qlq_dequantize - w[n, k] = scale[n, g]*q[n, k] + bias[n, g] with
 * g = k / group_size, computed as one fp32 fused multiply-add (single
 * rounding), out [N, K] fp32.  ("Struct QuantizedLinear", dequantized_weight.)
 * bits, group_size and the shape limits as for qlq_pack.
 */
QLQ_API int qlq_dequantize(const uint32_t* packed, const void* scales, const void* biases,
                           int sb_dtype, int64_t N, int64_t K, int bits, int group_size,
                           float* w, void* stream);

/*
 * qlq_linear_workspace_size - bytes of device workspace qlq_linear_forward
 * needs for these arguments (0 when the call takes the skinny path, or the
 * arguments are invalid).  GEMM path: x rescaled to fp16 [M, K], per-row and
 * per-column exponents, and the per-group fp16 (scale, bias) pairs
 * [K/group_size, round_up(N, 4)]; for 1-, 2-, 3-, 5- and 6-bit codes also
 * the codes rewritten for the GEMM (N*K/2 bytes as nibbles for 1, 2 and 3
 * bits, N*K bytes for 5 and 6).
 */
QLQ_API size_t qlq_linear_workspace_size(int64_t M, int64_t K, int64_t N, int bits,
                                         int group_size, int x_dtype);

/*
 * qlq_linear_forward - y = x . dequant(W)^T (+ bias) over the last axis of x.
 * ("Struct QuantizedLinear", forward: x W^T + b computed from the packed
 *  weight, its scales and biases.)
 *
 *   x       [M, K] of x_dtype.
 *   packed  [N, K*bits/32] uint32; scales, biases [N, K/group_size] of
 *           sb_dtype (== x_dtype), as written by qlq_pack.
 *   bias    [N] of x_dtype, or NULL.
 *   y       [M, N] of x_dtype (out).  Accumulation is fp32; y is rounded once.
 *   workspace  device memory of at least qlq_linear_workspace_size() bytes,
 *           256-byte aligned (QLQ_ERR_ALIGNMENT otherwise); may be NULL when
 *           that size is 0.  The call overwrites it; it holds no state
 *           between calls, and calls sharing one workspace must be ordered
 *           on one stream.
 *
 * M <= qlq_get_skinny_max_m() (and every fp32 x) takes the GEMV-shaped skinny
 * kernel.  Larger M takes the MFMA GEMM when K % 64 == 0, 512*K < 2^31 (a
 * 256-row tile of fp16 x) and 4*(K/group_size)*round_up(N, 4) < 2^31 (its
 * operands are addressed with 32-bit buffer offsets); other shapes take the
 * skinny kernel, and qlq_linear_workspace_size() returns 0 for them.  bits in
 * {1, ..., 6, 8} (the GEMM runs 1-, 2- and 3-bit codes as 4-bit ones, 5- and
 * 6-bit codes as 8-bit ones, transcoded in the workspace); group_size in
 * {32, 64, 128};
 * x_dtype == sb_dtype in {F32, F16, BF16}.
 */
QLQ_API int qlq_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                               const uint32_t* packed, const void* scales,
                               const void* biases, int sb_dtype, int64_t N, int bits,
                               int group_size, const void* bias, void* y,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dispatch threshold: calls with M <= this value take the skinny kernel.
 * Process-wide.  A call reads it once, so a call that overlaps a change takes
 * one path, with the workspace that path needs, and
 * qlq_linear_workspace_size answers for the value it reads.  Values < 0 are
 * rejected.  Used by the tests to force either path.
 */
QLQ_API int qlq_set_skinny_max_m(int m);
QLQ_API int qlq_get_skinny_max_m(void);

/* ------------------------------------------------------------------------
 * Ternary BitLinear ("mlx-lm/mlx_lm/models/bitlinear_layers.py")
 * ------------------------------------------------------------------------ */

/*
 * bitlinear_pack - ternary values t [N, K] int8 in {-1, 0, 1} -> packed
 * [N/4, K] uint8 with byte[r, k] = sum_j (t[r + j*N/4, k] + 1) << 2j
 * (the layout make_bitlinear_kernel decodes).  N % 4 == 0.
 * Synchronises `stream`; QLQ_ERR_DATA if a value lies outside {-1, 0, 1}.
 */
QLQ_API int bitlinear_pack(const int8_t* t, int64_t N, int64_t K, uint8_t* packed,
                           void* stream);

/*
 * bitlinear_forward - y[m, r + j*N/4] = sigma * sum_k x[m, k]*(c - 1) (+ bias)
 * where c is field j (bits 2j..2j+1) of packed[r, k] and sigma is
 * weight_scale[0], or 1/weight_scale[0] when invert_weight_scale != 0.
 * (make_bitlinear_kernel; BitLinear.execute_matmul_kernel and __call__.)
 *
 *   x [M, K] of x_dtype (BF16, F16 or F32); packed [N/4, K] uint8;
 *   weight_scale: one element of x_dtype (the page requires the input dtype
 *   to equal the weight-scale dtype); bias [N] of x_dtype or NULL;
 *   y [M, N] of x_dtype (out), fp32 accumulation, bias added after scaling,
 *   one final rounding.  N % 4 == 0, K % 32 == 0, M >= 1; with 16-bit x
 *   K < 2^26 (QLQ_ERR_UNSUPPORTED otherwise).
 */
QLQ_API int bitlinear_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                              const uint8_t* packed, int64_t N, const void* weight_scale,
                              int invert_weight_scale, const void* bias, void* y,
                              void* stream);

/* ------------------------------------------------------------------------
 * Per-channel symmetric W8A8 ("cider/ops.py")
 * ------------------------------------------------------------------------ */

/*
 * qlq_quantize_rows_int8 - per-row symmetric int8 quantization of v [R, K]
 * (quantize_weight_int8, absmax branch; the same rule quantizes activations):
 * a = max |v[r, :]|, s = a/127 in fp32 (1 if 0), q = clamp(rint(v/s), -128,
 * 127).  v of v_dtype (F32, F16 or BF16); q [R, K] int8 and scale [R] fp32
 * (out).  K % 16 == 0.
 */
QLQ_API int qlq_quantize_rows_int8(const void* v, int v_dtype, int64_t R, int64_t K,
                                   int8_t* q, float* scale, void* stream);

/*
 * qlq_quantize_rows_int8_clip - quantize_weight_int8 with clip_percentile:
 * per row, clip = the clip_percentile-th percentile of |v[r, :]| (NumPy's
 * linear method, every step in fp32: q = p/100, index (K-1) q, the sorted
 * neighbours a, b and weight t combined as a + (b-a) t for t < 0.5, else
 * b - (b-a)(1-t)); a zero clip becomes max |v[r, :]|; s = clip/127 (1 if 0);
 * q = clamp(rint(clamp(v, -clip, clip) / s), -128, 127).  v of v_dtype (F32,
 * F16 or BF16); q [R, K] int8 and scale [R] fp32 (out).  1 <= K <= 16384
 * (each row is sorted on chip), 0 <= clip_percentile <= 100.  Non-finite
 * values give unspecified output.
 */
QLQ_API int qlq_quantize_rows_int8_clip(const void* v, int v_dtype, int64_t R, int64_t K,
                                        float clip_percentile, int8_t* q, float* scale, void* stream);

/*
 * qlq_int8_matmul_int32 - c = a . b^T exactly: a [M, K] int8, b [N, K] int8
 * (the transposed weight layout of int8_matmul_int32), c [M, N] int32 (out).
 * K % 16 == 0 and K <= 131071 (so |c| <= 128*128*K < 2^31).
 */
QLQ_API int qlq_int8_matmul_int32(const int8_t* a, const int8_t* b, int64_t M, int64_t N,
                                  int64_t K, int32_t* c, void* stream);

/* Bytes of workspace w8a8_linear_forward needs: M*K int8 + M fp32, aligned. */
QLQ_API size_t w8a8_workspace_size(int64_t M, int64_t K);

/*
 * w8a8_linear_forward - y = dequant(quant_a(x) . w^T) (+ bias)
 * (perchannel_linear).  quant_a is per-row symmetric int8 as in
 * qlq_quantize_rows_int8; the int32 accumulator is scaled as
 * acc * sx[m] * scale_w[n] (+ bias[n]) in fp32 and rounded once to x_dtype.
 *
 *   x [M, K] of x_dtype (F16 or BF16); w [N, K] int8; scale_w [N] fp32;
 *   bias [N] of x_dtype or NULL; y [M, N] of x_dtype (out);
 *   workspace >= w8a8_workspace_size(M, K) bytes, 16-byte aligned (holds
 *   quant_a(x) and sx; overwritten, no state kept between calls).
 *   K % 16 == 0, K <= 131071.
 */
QLQ_API int w8a8_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                                const int8_t* w, const float* scale_w, int64_t N,
                                const void* bias, void* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Where the activation quantizer runs ("cider/ops.py", perchannel_linear:
 * y = dequant(quant_a(x) @ w_int8) + bias).  0 (default): quant_a writes
 * xq [M, K] int8 and sx [M] to the workspace, then the int8 GEMM reads xq.
 * 1: a pre-pass writes sx only and the GEMM quantizes each x tile itself
 * (fp16/bf16 tiles into registers, the same quotient, rounding and clamp, so
 * the codes, the int32 sums and y are bit-identical to mode 0); every
 * column block of the GEMM then quantizes its rows again, which costs more
 * than the xq round trip it saves.  Process-wide, read once at each call of
 * w8a8_linear_forward and w8a8_linear_forward_noalloc (both modes use the
 * same workspace), so a call that overlaps a change runs one mode or the
 * other.  Values other than 0 and 1 are rejected (QLQ_ERR_INVALID_ARG).
 */
QLQ_API int qlq_set_w8a8_fused_quant(int on);
QLQ_API int qlq_get_w8a8_fused_quant(void);

/*
 * w8a8_linear_forward_noalloc - w8a8_linear_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and
 * result, with no workspace argument.  quant_a(x) and sx go to a static
 * device array of QLQ_W8A8_NOALLOC_SCRATCH_BYTES bytes that each GPU the
 * library runs on holds until the process ends; its address is looked up
 * once per device, on the first call there.  The call allocates nothing.
 *
 *   Arguments as w8a8_linear_forward without workspace / workspace_bytes.
 *   w8a8_workspace_size(M, K) must not exceed QLQ_W8A8_NOALLOC_SCRATCH_BYTES
 *   (else QLQ_ERR_WORKSPACE, checked before any HIP call): M*K up to about
 *   16 million int8 values, e.g. up to 4092 rows at K = 4096.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents: two calls that overlap on one GPU (different streams without an
 * ordering between them, or different host threads) race on it and give
 * undefined results.  Calls ordered on one stream are safe; nothing in the
 * array needs to start at zero (the quantizer writes every byte the GEMM
 * reads).
 */
#define QLQ_W8A8_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
QLQ_API int w8a8_linear_forward_noalloc(const void* x, int x_dtype, int64_t M, int64_t K,
                                        const int8_t* w, const float* scale_w, int64_t N,
                                        const void* bias, void* y, void* stream);

/* ------------------------------------------------------------------------
 * Per-group int8 weights ("cider/ops.py": pergroup_linear)
 * ------------------------------------------------------------------------ */

/*
 * qlq_quantize_groups_int8 - per-group symmetric int8 quantization of
 * w [N, K] (w_dtype F32, F16 or BF16): every group of group_size consecutive
 * input values of a row follows the rule of qlq_quantize_rows_int8 (fp32
 * absmax/127, 1 if 0, q = clamp(rint(w/s), -128, 127)).  q [N, K] int8 and
 * scale [K/group_size, N] fp32 (out; group-major, the transposed layout of
 * pergroup_linear).  group_size in {64, 128, 256}, K % group_size == 0.
 */
QLQ_API int qlq_quantize_groups_int8(const void* w, int w_dtype, int64_t N, int64_t K,
                                     int group_size, int8_t* q, float* scale, void* stream);

/* Bytes of workspace pergroup_linear_forward needs: 0 for M == 1, else as
 * w8a8_workspace_size (quant_a(x) and its row scales). */
QLQ_API size_t pergroup_workspace_size(int64_t M, int64_t K);

/*
 * pergroup_linear_forward - per-group int8 linear (pergroup_linear).
 *   M > 1:  y = sx[m] * sum_g scale_w[g, n] * (sum_{k in g} xq[m, k] w[n, k])
 *           (+ bias[n]) with xq, sx = quant_a(x) as in w8a8_linear_forward;
 *           int32 per group, rescaled in fp32, rounded once to x_dtype.
 *   M == 1: y = sum_k x[k] * w[n, k] * scale_w[g(k), n] (+ bias[n]) with x as
 *           stored (no activation quantization), fp32 accumulation.
 *
 *   x [M, K] of x_dtype (F16 or BF16); w [N, K] int8; scale_w [K/group_size,
 *   N] fp32; bias [N] of x_dtype or NULL; y [M, N] of x_dtype (out);
 *   workspace >= pergroup_workspace_size(M, K) bytes, 16-byte aligned, may be
 *   NULL when that is 0 (overwritten, no state kept between calls).
 *   group_size in {64, 128, 256}; K % group_size == 0; K <= 131071, and
 *   K <= 16384 when M == 1 (x is staged whole on chip): else
 *   QLQ_ERR_UNSUPPORTED.
 */
QLQ_API int pergroup_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                                    const int8_t* w, const float* scale_w, int64_t N,
                                    int group_size, const void* bias, void* y, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Per-column int4 weights, int8 activations ("cider/ops.py":
 * pack_weight_int4, w4a8_linear)
 * ------------------------------------------------------------------------ */

/*
 * w4a8_pack_weight_int4 - per-column symmetric int4 quantization of
 * w [K, N] (row-major, N contiguous; w_dtype F32, F16 or BF16):
 * s = max |w[:, n]| / 7 in fp32 (1 if 0), code = clamp(rint(w/s) + 8, 0, 15)
 * with the quotient correctly rounded.  packed [K/2, N] uint8 (out): byte
 * (j, n) holds the code of k = 2j in its high nibble and of k = 2j + 1 in its
 * low nibble; scale [N] fp32 (out).  K even.  Non-finite weights give
 * unspecified codes (no check on the device).
 */
QLQ_API int w4a8_pack_weight_int4(const void* w, int w_dtype, int64_t K, int64_t N,
                                  uint8_t* packed, float* scale, void* stream);

/* Bytes of workspace w4a8_linear_forward needs: quant_a(x) and its row
 * scales for the GEMM; for M <= 8 at least the skinny path's exact int32
 * partial sums (one per 128 input values, row and column) and row scales. */
QLQ_API size_t w4a8_workspace_size(int64_t M, int64_t K, int64_t N);

/*
 * w4a8_linear_forward - y = dequant(quant_a(x) . unpack4(packed_w)) (+ bias)
 * (w4a8_linear).  unpack4 gives the value code - 8 of each nibble; quant_a
 * is per-row symmetric int8 as in qlq_quantize_rows_int8; the exact int32
 * sum is scaled as acc * sx[m] * scale_w[n] (+ bias[n]) in fp32 and rounded
 * once to x_dtype.  The pages' function has no bias: pass NULL for it.
 * M <= min(8, qlq_get_skinny_max_m()) takes a kernel split over K (exact
 * int32 partials, then a kernel that adds them and scales); larger M the
 * GEMM.  Both give identical outputs (the sums are exact integers).
 *
 *   x [M, K] of x_dtype (F16 or BF16); packed_w [K/2, N] uint8 as written by
 *   w4a8_pack_weight_int4 (4-byte aligned); scale_w [N] fp32; bias [N] of
 *   x_dtype or NULL; y [M, N] of x_dtype (out); workspace >=
 *   w4a8_workspace_size(M, K, N) bytes, 16-byte aligned (overwritten, no state
 *   kept between calls).  K % 16 == 0, K <= 131071, (K/2)*N < 2^31.
 */
QLQ_API int w4a8_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                                const uint8_t* packed_w, const float* scale_w, int64_t N,
                                const void* bias, void* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Device and error reporting
 * ------------------------------------------------------------------------ */

/* QLQ_OK iff `device` exists and is a gfx950; QLQ_ERR_DEVICE otherwise. */
QLQ_API int qlq_device_check(int device);

/* Thread-local text of the last error ("" if none). Valid until the next call. */
QLQ_API const char* qlq_last_error(void);

/* Library version string. */
QLQ_API const char* qlq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLQ_H */
