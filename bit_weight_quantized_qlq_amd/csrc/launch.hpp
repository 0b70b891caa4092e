// Host-side launchers of the qlq kernels.  Each returns the hipError_t of its
// launch; the C ABI layer (api.cpp) validates arguments before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlq {

// pack.hip
hipError_t launch_affine_pack(const float* w, int64_t N, int64_t K, int bits, int G,
                              uint32_t* packed, void* scales, void* biases, int sb_dtype,
                              int* err_flag, hipStream_t s);
hipError_t launch_affine_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits,
                                uint8_t* codes, hipStream_t s);
// 1- or 3-bit codes rewritten in the 4-bit packed layout (N*K % 32 == 0)
hipError_t launch_affine_to_nibbles(const uint32_t* packed, int64_t N, int64_t K, int bits,
                                    uint32_t* out, hipStream_t s);
hipError_t launch_affine_dequant(const uint32_t* packed, const void* scales, const void* biases,
                                 int sb_dtype, int64_t N, int64_t K, int bits, int G, float* w,
                                 hipStream_t s);
hipError_t launch_ternary_pack(const int8_t* t, int64_t N, int64_t K, uint8_t* packed,
                               int* err_flag, hipStream_t s);
// nibble_order: each 16-byte chunk of q in the order eight packed int4 bytes
// unpack to (high nibbles then low nibbles, four bytes at a time)
hipError_t launch_quantize_rows_int8(const void* v, int v_dtype, int64_t R, int64_t K,
                                     int8_t* q, float* scale, hipStream_t s, bool nibble_order = false);
// per-row int8 with the clip at a percentile of |v| (K <= kClipMaxK)
// the row scales of launch_quantize_rows_int8 alone (K % 16 == 0)
hipError_t launch_row_scales_int8(const void* v, int v_dtype, int64_t R, int64_t K, float* scale, hipStream_t s);
constexpr int64_t kClipMaxKHost = 16384;
hipError_t launch_quantize_rows_int8_clip(const void* v, int v_dtype, int64_t R, int64_t K, float pct, int8_t* q,
                                          float* scale, hipStream_t s);
hipError_t launch_pack_int4_cols(const void* w, int w_dtype, int64_t K, int64_t N, uint8_t* packed,
                                 float* scale, hipStream_t s);

// gemv.hip: skinny affine forward (small M)
hipError_t launch_affine_gemv(const void* x, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, const void* scales, const void* biases,
                              int64_t N, int bits, int G, const void* bias, void* y,
                              hipStream_t s);

// gemm.hip: affine prefill GEMM (bf16 / f16 x) on 4- or 8-bit packed codes
// bits: the width the GEMM runs on (4 or 8)
size_t affine_gemm_workspace(int64_t M, int64_t K, int64_t N, int group_size, int bits);
hipError_t launch_affine_gemm(const void* x, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, const void* scales, const void* biases,
                              int64_t N, int bits, int G, const void* bias, void* y,
                              void* workspace, hipStream_t s);

// ternary.hip
hipError_t launch_ternary_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const uint8_t* packed, int64_t N, const void* weight_scale,
                                  int invert, const void* bias, void* y, hipStream_t s);

// int8.hip
// the W8A8 product with the activation quantizer in the GEMM: x [M, K] fp16 /
// bf16 and its row scales sx (launch_row_scales_int8); out of x's dtype
hipError_t launch_int8_gemm_quant_a(const void* x, int x_dtype, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                    const float* sx, const float* sb, const void* bias, void* out, hipStream_t s);
hipError_t launch_int8_gemm(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, const void* bias, int out_dtype,
                            void* out, hipStream_t s);
// b: packed int4 [K/2, N] (even k in the high nibble, value = code - 8);
// a: int8 [M, K] in nibble order; y = fp32(a . b) * sa[m] * sb[n] (+ bias)
hipError_t launch_w4a8_gemm(const int8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, const void* bias, int out_dtype, void* out,
                            hipStream_t s);
// w4a8.hip: a few rows (M <= kW4a8SkinnyMaxM), split over K; workspace of
// w4a8_skinny_workspace bytes (int32 partials, then the row scales)
constexpr int64_t kW4a8SkinnyMaxM = 8;
size_t w4a8_skinny_workspace(int64_t M, int64_t K, int64_t N);
hipError_t launch_w4a8_skinny(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* b, int64_t N,
                              const float* sw, const void* bias, void* y, void* workspace, hipStream_t s);
hipError_t launch_int8_gemm_pergroup(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                     const float* sa, const float* scale_w, int group_size,
                                     const void* bias, int out_dtype, void* out, hipStream_t s);

// pack.hip (per-group weights)
hipError_t launch_quantize_groups_int8(const void* w, int w_dtype, int64_t N, int64_t K, int group_size,
                                       int8_t* q, float* scale, hipStream_t s);

// pergroup.hip
constexpr int64_t kPergroupMvMaxK = 16384;
hipError_t launch_pergroup_mv(const void* x, int x_dtype, int64_t K, const int8_t* w, const float* scale,
                              int64_t N, int group_size, const void* bias, void* y, hipStream_t s);

}  // namespace qlq
