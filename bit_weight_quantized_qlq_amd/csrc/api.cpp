// C ABI of libqlq: argument validation, device check, dispatch, launches.
// Every entry point validates on the host before its first HIP call, so an
// invalid call returns an error without touching the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/qlq.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;
// process-wide switches; each call reads a switch once, so a call that
// overlaps a change takes one setting or the other throughout
std::atomic<int> g_skinny_max_m{8};
std::atomic<int> g_w8a8_fused_quant{0};  // W8A8: activation quantizer inside the GEMM (1) or before it (0)

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return QLQ_OK;
}
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool dtype_ok(int d) { return d == QLQ_F32 || d == QLQ_F16 || d == QLQ_BF16; }
size_t dtype_size(int d) { return d == QLQ_F32 ? 4 : 2; }
constexpr int64_t kMaxDim = (int64_t)1 << 31;

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QLQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// gfx950 check, cached per device.
std::mutex g_dev_mu;
signed char g_dev_state[64];  // 0 unknown, 1 gfx950, -1 other

int device_status(int dev) {
  if (dev < 0 || dev >= 64) return fail(QLQ_ERR_DEVICE, "device %d out of range", dev);
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 1) return QLQ_OK;
    if (g_dev_state[dev] == -1) return fail(QLQ_ERR_DEVICE, "device %d is not a gfx950", dev);
  }
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || dev >= count)
    return fail(QLQ_ERR_DEVICE, "no HIP device %d", dev);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(QLQ_ERR_DEVICE, "cannot query HIP device %d", dev);
  const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_state[dev] = is950 ? 1 : -1;
  }
  if (!is950) return fail(QLQ_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return QLQ_OK;
}

int current_device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(QLQ_ERR_DEVICE, "no current HIP device");
  }
  return device_status(dev);
}

#define QLQ_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

bool affine_bits_ok(int bits) { return (bits >= 1 && bits <= 6) || bits == 8; }
// the packed width the GEMM runs on: 1-, 2- and 3-bit codes are transcoded
// to the 4-bit layout, 5- and 6-bit codes to the 8-bit one
int gemm_bits(int bits) { return bits <= 3 ? 4 : bits == 5 || bits == 6 ? 8 : bits; }
bool transcoded_gemm(int bits) { return gemm_bits(bits) != bits; }

int check_affine_shape(int64_t N, int64_t K, int bits, int G) {
  QLQ_REQUIRE(N >= 1 && K >= 1 && N < kMaxDim && K < kMaxDim, QLQ_ERR_INVALID_ARG,
              "invalid shape N=%lld K=%lld", (long long)N, (long long)K);
  QLQ_REQUIRE(affine_bits_ok(bits), QLQ_ERR_UNSUPPORTED, "bits=%d not supported (1-6, 8)", bits);
  QLQ_REQUIRE(G == 32 || G == 64 || G == 128, QLQ_ERR_UNSUPPORTED,
              "group_size=%d not built (32, 64, 128)", G);
  QLQ_REQUIRE(K % G == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of group_size=%d", (long long)K, G);
  return QLQ_OK;
}

// The GEMM path takes 16-bit x with K a multiple of its 64-wide k-iteration.
// The prefill GEMM addresses its operands through 32-bit buffer offsets: the
// tallest x16 tile the launcher can pick (256 rows of 2 K bytes, chosen at
// launch from the tile count), a 128-row tile of 8-bit codes (128 K bytes)
// and the (s', b') table (4 (K/G) N bytes) must stay below 2^31 bytes; other
// shapes take the skinny kernel.
constexpr int64_t kGemmTallestTileRows = 256;
bool takes_gemm(int64_t M, int64_t K, int64_t N, int G, int x_dtype, int skinny_max_m) {
  return x_dtype != QLQ_F32 && M > skinny_max_m && K % 64 == 0 && K * 2 * kGemmTallestTileRows < kMaxDim &&
         (K / G) * ((N + 3) & ~(int64_t)3) * 4 < kMaxDim;
}

// one-shot device int flag for the synchronising pack calls
struct DevFlag {
  int* p = nullptr;
  ~DevFlag() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

extern "C" {

QLQ_API const char* qlq_last_error(void) { return g_err.c_str(); }
QLQ_API const char* qlq_version(void) { return "qlq 0.1.0 (gfx950)"; }

QLQ_API int qlq_device_check(int device) {
  const int st = device_status(device);
  return st == QLQ_OK ? ok() : st;
}

QLQ_API int qlq_set_skinny_max_m(int m) {
  QLQ_REQUIRE(m >= 0, QLQ_ERR_INVALID_ARG, "skinny max M must be >= 0 (got %d)", m);
  g_skinny_max_m.store(m, std::memory_order_relaxed);
  return ok();
}
QLQ_API int qlq_get_skinny_max_m(void) { return g_skinny_max_m.load(std::memory_order_relaxed); }

QLQ_API int qlq_set_w8a8_fused_quant(int on) {
  QLQ_REQUIRE(on == 0 || on == 1, QLQ_ERR_INVALID_ARG, "fused activation quant must be 0 or 1 (got %d)", on);
  g_w8a8_fused_quant.store(on, std::memory_order_relaxed);
  return ok();
}
QLQ_API int qlq_get_w8a8_fused_quant(void) { return g_w8a8_fused_quant.load(std::memory_order_relaxed); }

// ----------------------------------------------------------------- affine
QLQ_API int qlq_pack(const float* w, int64_t N, int64_t K, int bits, int group_size, uint32_t* packed,
                     void* scales, void* biases, int sb_dtype, void* stream) {
  QLQ_REQUIRE(w && packed && scales && biases, QLQ_ERR_INVALID_ARG, "null pointer");
  if (int st = check_affine_shape(N, K, bits, group_size)) return st;
  QLQ_REQUIRE(dtype_ok(sb_dtype), QLQ_ERR_UNSUPPORTED, "sb_dtype %d", sb_dtype);
  QLQ_REQUIRE(aligned(w, 16), QLQ_ERR_ALIGNMENT, "w not 16-byte aligned");
  QLQ_REQUIRE(aligned(packed, 4) && aligned(scales, dtype_size(sb_dtype)) &&
                  aligned(biases, dtype_size(sb_dtype)),
              QLQ_ERR_ALIGNMENT, "misaligned output");
  if (int st = current_device_status()) return st;
  hipStream_t s = (hipStream_t)stream;
  DevFlag flag;
  if (int st = hip_status(hipMalloc((void**)&flag.p, sizeof(int)), "hipMalloc(flag)")) return st;
  if (int st = hip_status(hipMemsetAsync(flag.p, 0, sizeof(int), s), "hipMemsetAsync")) return st;
  if (int st = hip_status(qlq::launch_affine_pack(w, N, K, bits, group_size, packed, scales, biases,
                                                  sb_dtype, flag.p, s),
                          "affine_pack launch"))
    return st;
  int host_flag = 0;
  if (int st = hip_status(hipMemcpyAsync(&host_flag, flag.p, sizeof(int), hipMemcpyDeviceToHost, s),
                          "hipMemcpyAsync(flag)"))
    return st;
  if (int st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize")) return st;
  QLQ_REQUIRE(host_flag == 0, QLQ_ERR_DATA, "non-finite weight, or scale/bias overflows the storage dtype");
  return ok();
}

QLQ_API int qlq_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits, uint8_t* codes,
                       void* stream) {
  QLQ_REQUIRE(packed && codes, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(N >= 1 && K >= 1 && N < kMaxDim && K < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(affine_bits_ok(bits), QLQ_ERR_UNSUPPORTED, "bits=%d not supported (1-6, 8)", bits);
  QLQ_REQUIRE((K * bits) % 32 == 0, QLQ_ERR_INVALID_ARG, "K must fill whole words");
  QLQ_REQUIRE(aligned(packed, 4), QLQ_ERR_ALIGNMENT, "packed not 4-byte aligned");
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_affine_unpack(packed, N, K, bits, codes, (hipStream_t)stream), "unpack");
}

QLQ_API int qlq_dequantize(const uint32_t* packed, const void* scales, const void* biases, int sb_dtype,
                           int64_t N, int64_t K, int bits, int group_size, float* w, void* stream) {
  QLQ_REQUIRE(packed && scales && biases && w, QLQ_ERR_INVALID_ARG, "null pointer");
  if (int st = check_affine_shape(N, K, bits, group_size)) return st;
  QLQ_REQUIRE(dtype_ok(sb_dtype), QLQ_ERR_UNSUPPORTED, "sb_dtype %d", sb_dtype);
  QLQ_REQUIRE(aligned(packed, 4) && aligned(w, 4) && aligned(scales, dtype_size(sb_dtype)) &&
                  aligned(biases, dtype_size(sb_dtype)),
              QLQ_ERR_ALIGNMENT, "misaligned pointer");
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_affine_dequant(packed, scales, biases, sb_dtype, N, K, bits, group_size, w,
                                               (hipStream_t)stream),
                    "dequantize");
}

namespace {
// workspace of the GEMM path: pre-pass outputs and partials, then the
// transcoded codes for 1-, 2-, 3-, 5- and 6-bit codes
size_t affine_gemm_ws_bytes(int64_t M, int64_t K, int64_t N, int bits, int G) {
  size_t need = (qlq::affine_gemm_workspace(M, K, N, G, gemm_bits(bits)) + 255) & ~(size_t)255;
  if (transcoded_gemm(bits)) need += (size_t)N * (size_t)K * gemm_bits(bits) / 8;
  return need;
}
}  // namespace

QLQ_API size_t qlq_linear_workspace_size(int64_t M, int64_t K, int64_t N, int bits, int group_size,
                                         int x_dtype) {
  if (M <= 0 || K <= 0 || N <= 0 || group_size <= 0 || K % group_size) return 0;
  if (!takes_gemm(M, K, N, group_size, x_dtype, g_skinny_max_m.load(std::memory_order_relaxed))) return 0;
  return affine_gemm_ws_bytes(M, K, N, bits, group_size);
}

QLQ_API int qlq_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* packed,
                               const void* scales, const void* biases, int sb_dtype, int64_t N, int bits,
                               int group_size, const void* bias, void* y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  // x and y may be NULL for an empty batch (M == 0)
  QLQ_REQUIRE(((x && y) || M == 0) && packed && scales && biases, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid M=%lld", (long long)M);
  if (int st = check_affine_shape(N, K, bits, group_size)) return st;
  QLQ_REQUIRE(dtype_ok(x_dtype), QLQ_ERR_UNSUPPORTED, "x_dtype %d", x_dtype);
  QLQ_REQUIRE(sb_dtype == x_dtype, QLQ_ERR_DTYPE, "scales/biases dtype %d != x dtype %d", sb_dtype, x_dtype);
  const size_t es = dtype_size(x_dtype);
  QLQ_REQUIRE(aligned(x, 16) && aligned(packed, 16), QLQ_ERR_ALIGNMENT, "x / packed not 16-byte aligned");
  QLQ_REQUIRE(aligned(scales, es) && aligned(biases, es) && aligned(y, es) && (!bias || aligned(bias, es)),
              QLQ_ERR_ALIGNMENT, "misaligned scales / biases / bias / y");
  // one read of the threshold decides the path and the workspace it needs
  const bool gemm = takes_gemm(M, K, N, group_size, x_dtype, g_skinny_max_m.load(std::memory_order_relaxed));
  if (gemm) {
    const size_t need = affine_gemm_ws_bytes(M, K, N, bits, group_size);
    QLQ_REQUIRE(workspace && workspace_bytes >= need, QLQ_ERR_WORKSPACE,
                "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    QLQ_REQUIRE(aligned(workspace, 256), QLQ_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  } else {
    QLQ_REQUIRE((M + 7) / 8 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for the skinny kernel");
  }
  if (M == 0) return ok();
  if (int st = current_device_status()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (gemm && transcoded_gemm(bits)) {
    // 1, 2, 3, 5, 6 bits: the codes are rewritten in the 4-bit (1, 2, 3) or
    // 8-bit (5, 6: one byte per code) packed layout, and that width's GEMM
    // runs on them with the same scales and biases
    uint32_t* codes = (uint32_t*)((char*)workspace +
                                  ((qlq::affine_gemm_workspace(M, K, N, group_size, gemm_bits(bits)) + 255) & ~(size_t)255));
    const int wb = gemm_bits(bits);
    const hipError_t e = wb == 4 ? qlq::launch_affine_to_nibbles(packed, N, K, bits, codes, s)
                                 : qlq::launch_affine_unpack(packed, N, K, bits, (uint8_t*)codes, s);
    if (int st = hip_status(e, "transcode")) return st;
    return hip_status(qlq::launch_affine_gemm(x, x_dtype, M, K, codes, scales, biases, N, wb, group_size, bias,
                                              y, workspace, s),
                      "affine gemm");
  }
  if (gemm)
    return hip_status(qlq::launch_affine_gemm(x, x_dtype, M, K, packed, scales, biases, N, bits, group_size,
                                              bias, y, workspace, s),
                      "affine gemm");
  return hip_status(qlq::launch_affine_gemv(x, x_dtype, M, K, packed, scales, biases, N, bits, group_size,
                                            bias, y, s),
                    "affine gemv");
}

// ---------------------------------------------------------------- ternary
QLQ_API int bitlinear_pack(const int8_t* t, int64_t N, int64_t K, uint8_t* packed, void* stream) {
  QLQ_REQUIRE(t && packed, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(N >= 4 && K >= 1 && N < kMaxDim && K < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(N % 4 == 0, QLQ_ERR_INVALID_ARG, "N=%lld is not a multiple of 4", (long long)N);
  if (int st = current_device_status()) return st;
  hipStream_t s = (hipStream_t)stream;
  DevFlag flag;
  if (int st = hip_status(hipMalloc((void**)&flag.p, sizeof(int)), "hipMalloc(flag)")) return st;
  if (int st = hip_status(hipMemsetAsync(flag.p, 0, sizeof(int), s), "hipMemsetAsync")) return st;
  if (int st = hip_status(qlq::launch_ternary_pack(t, N, K, packed, flag.p, s), "ternary_pack launch"))
    return st;
  int host_flag = 0;
  if (int st = hip_status(hipMemcpyAsync(&host_flag, flag.p, sizeof(int), hipMemcpyDeviceToHost, s),
                          "hipMemcpyAsync(flag)"))
    return st;
  if (int st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize")) return st;
  QLQ_REQUIRE(host_flag == 0, QLQ_ERR_DATA, "ternary value outside {-1, 0, 1}");
  return ok();
}

QLQ_API int bitlinear_forward(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* packed,
                              int64_t N, const void* weight_scale, int invert_weight_scale, const void* bias,
                              void* y, void* stream) {
  QLQ_REQUIRE(((x && y) || M == 0) && packed && weight_scale, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim && N >= 4 && N < kMaxDim && K >= 1 && K < kMaxDim, QLQ_ERR_INVALID_ARG,
              "invalid shape");
  QLQ_REQUIRE(N % 4 == 0, QLQ_ERR_INVALID_ARG, "N=%lld is not a multiple of 4", (long long)N);
  QLQ_REQUIRE(K % 32 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 32", (long long)K);
  QLQ_REQUIRE(dtype_ok(x_dtype), QLQ_ERR_UNSUPPORTED, "x_dtype %d", x_dtype);
  const size_t es = dtype_size(x_dtype);
  QLQ_REQUIRE(aligned(x, 16) && aligned(packed, 16), QLQ_ERR_ALIGNMENT, "x / packed not 16-byte aligned");
  QLQ_REQUIRE(aligned(weight_scale, es) && aligned(y, es) && (!bias || aligned(bias, es)),
              QLQ_ERR_ALIGNMENT, "misaligned weight_scale / bias / y");
  QLQ_REQUIRE((M + 15) / 16 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for one launch");
  // 16-bit x: a block's 16 x rows (and 8 packed rows) sit behind 32-bit buffer ranges
  QLQ_REQUIRE(x_dtype == QLQ_F32 || K < ((int64_t)1 << 26), QLQ_ERR_UNSUPPORTED,
              "K=%lld not below 2^26 with 16-bit x", (long long)K);
  if (M == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_ternary_forward(x, x_dtype, M, K, packed, N, weight_scale,
                                                invert_weight_scale, bias, y, (hipStream_t)stream),
                    "ternary forward");
}

// ------------------------------------------------------------------- W8A8
QLQ_API int qlq_quantize_rows_int8(const void* v, int v_dtype, int64_t R, int64_t K, int8_t* q, float* scale,
                                   void* stream) {
  QLQ_REQUIRE((v && q && scale) || R == 0, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(R >= 0 && R < kMaxDim && K >= 16 && K < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K % 16 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  QLQ_REQUIRE(dtype_ok(v_dtype), QLQ_ERR_UNSUPPORTED, "v_dtype %d", v_dtype);
  QLQ_REQUIRE(aligned(v, 16) && aligned(q, 16) && aligned(scale, 4), QLQ_ERR_ALIGNMENT, "misaligned pointer");
  if (R == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_quantize_rows_int8(v, v_dtype, R, K, q, scale, (hipStream_t)stream),
                    "quantize rows");
}

QLQ_API int qlq_quantize_rows_int8_clip(const void* v, int v_dtype, int64_t R, int64_t K, float clip_percentile,
                                        int8_t* q, float* scale, void* stream) {
  QLQ_REQUIRE((v && q && scale) || R == 0, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(R >= 0 && R < kMaxDim && K >= 1, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K <= qlq::kClipMaxKHost, QLQ_ERR_UNSUPPORTED, "K=%lld above %lld (rows are sorted on chip)",
              (long long)K, (long long)qlq::kClipMaxKHost);
  QLQ_REQUIRE(clip_percentile >= 0.0f && clip_percentile <= 100.0f, QLQ_ERR_INVALID_ARG,
              "clip_percentile outside [0, 100]");
  QLQ_REQUIRE(dtype_ok(v_dtype), QLQ_ERR_UNSUPPORTED, "v_dtype %d", v_dtype);
  QLQ_REQUIRE(aligned(v, dtype_size(v_dtype)) && aligned(scale, 4), QLQ_ERR_ALIGNMENT, "misaligned pointer");
  if (R == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_quantize_rows_int8_clip(v, v_dtype, R, K, clip_percentile, q, scale,
                                                        (hipStream_t)stream),
                    "quantize rows (percentile clip)");
}

QLQ_API int qlq_int8_matmul_int32(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K, int32_t* c,
                                  void* stream) {
  QLQ_REQUIRE(((a && c) || M == 0) && b, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim && N >= 1 && N < kMaxDim && K >= 16, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K % 16 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  QLQ_REQUIRE(K <= 131071, QLQ_ERR_UNSUPPORTED, "K=%lld could overflow int32", (long long)K);
  QLQ_REQUIRE(aligned(a, 16) && aligned(b, 16) && aligned(c, 4), QLQ_ERR_ALIGNMENT, "misaligned pointer");
  QLQ_REQUIRE((M + 127) / 128 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for one launch");
  if (M == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_int8_gemm(a, b, M, N, K, nullptr, nullptr, nullptr, -1, c, (hipStream_t)stream),
                    "int8 gemm");
}

QLQ_API size_t w8a8_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || M >= kMaxDim || K >= kMaxDim) return 0;  // shapes no forward call accepts
  const size_t q = ((size_t)M * (size_t)K + 255) & ~(size_t)255;
  return q + (size_t)M * sizeof(float);
}

}  // extern "C"

namespace {

// Arguments of w8a8_linear_forward and its allocation-free variant, apart
// from where the quantized activations go.
int check_w8a8_args(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* w, const float* scale_w,
                    int64_t N, const void* bias, const void* y) {
  QLQ_REQUIRE(((x && y) || M == 0) && w && scale_w, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim && N >= 1 && N < kMaxDim && K >= 16, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K % 16 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  QLQ_REQUIRE(K <= 131071, QLQ_ERR_UNSUPPORTED, "K=%lld could overflow int32", (long long)K);
  QLQ_REQUIRE(x_dtype == QLQ_F16 || x_dtype == QLQ_BF16, QLQ_ERR_UNSUPPORTED, "x_dtype must be F16 or BF16");
  QLQ_REQUIRE(aligned(x, 16) && aligned(w, 16) && aligned(scale_w, 4) && aligned(y, 2) &&
                  (!bias || aligned(bias, 2)),
              QLQ_ERR_ALIGNMENT, "misaligned pointer");
  QLQ_REQUIRE((M + 127) / 128 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for one launch");
  return QLQ_OK;
}

// quant_a(x) into xq [M, K] and sx [M] at the aligned offset of
// w8a8_workspace_size, then the int8 GEMM with the scale epilogue; or, with
// the fused quantizer selected, only sx (a pre-pass) and the GEMM quantizing
// x itself (the same codes, sums and epilogue).
int run_w8a8(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* w, const float* scale_w, int64_t N,
             const void* bias, void* y, void* buf, hipStream_t s) {
  int8_t* xq = (int8_t*)buf;
  float* sx = (float*)((char*)buf + (((size_t)M * (size_t)K + 255) & ~(size_t)255));
  if (g_w8a8_fused_quant.load(std::memory_order_relaxed)) {
    if (int st = hip_status(qlq::launch_row_scales_int8(x, x_dtype, M, K, sx, s), "activation row scales"))
      return st;
    return hip_status(qlq::launch_int8_gemm_quant_a(x, x_dtype, w, M, N, K, sx, scale_w, bias, y, s),
                      "int8 gemm (quantized A)");
  }
  if (int st = hip_status(qlq::launch_quantize_rows_int8(x, x_dtype, M, K, xq, sx, s), "activation quant"))
    return st;
  return hip_status(qlq::launch_int8_gemm(xq, w, M, N, K, sx, scale_w, bias, x_dtype, y, s), "int8 gemm");
}

}  // namespace

// Scratch of w8a8_linear_forward_noalloc: quant_a(x) and its row scales live
// in this file-scope device array instead of a caller workspace.  Every GPU
// the library runs on holds its own copy, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: host code uses only the per-device address taken below.
constexpr size_t kNoAllocScratchBytes = QLQ_W8A8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch`, per device; taken once

// The current device's copy of `scratch`: its address is looked up the first
// time a call runs on that device, with that device current.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fail(QLQ_ERR_DEVICE, "no current HIP device");
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(QLQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLQ_OK;
}

}  // namespace

extern "C" {

QLQ_API int w8a8_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* w,
                                const float* scale_w, int64_t N, const void* bias, void* y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (int st = check_w8a8_args(x, x_dtype, M, K, w, scale_w, N, bias, y)) return st;
  if (M == 0) return ok();
  const size_t need = w8a8_workspace_size(M, K);
  QLQ_REQUIRE(workspace && workspace_bytes >= need, QLQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  QLQ_REQUIRE(aligned(workspace, 16), QLQ_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  if (int st = current_device_status()) return st;
  return run_w8a8(x, x_dtype, M, K, w, scale_w, N, bias, y, workspace, (hipStream_t)stream);
}

QLQ_API int w8a8_linear_forward_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* w,
                                        const float* scale_w, int64_t N, const void* bias, void* y, void* stream) {
  if (int st = check_w8a8_args(x, x_dtype, M, K, w, scale_w, N, bias, y)) return st;
  if (M == 0) return ok();
  const size_t need = w8a8_workspace_size(M, K);
  QLQ_REQUIRE(need <= kNoAllocScratchBytes, QLQ_ERR_WORKSPACE,
              "M=%lld, K=%lld need %zu bytes of scratch; the allocation-free call holds at most %zu "
              "(use w8a8_linear_forward with a workspace)",
              (long long)M, (long long)K, need, kNoAllocScratchBytes);
  if (int st = current_device_status()) return st;
  void* buf = nullptr;
  if (int st = scratch_on_current_device(&buf)) return st;
  // every byte of the scratch that the GEMM reads (xq and sx) is written by
  // the quantizer first in the same stream, so nothing needs clearing
  return run_w8a8(x, x_dtype, M, K, w, scale_w, N, bias, y, buf, (hipStream_t)stream);
}

QLQ_API int qlq_quantize_groups_int8(const void* w, int w_dtype, int64_t N, int64_t K, int group_size,
                                     int8_t* q, float* scale, void* stream) {
  QLQ_REQUIRE(w && q && scale, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(N >= 0 && N < kMaxDim && K >= 1 && K < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(group_size == 64 || group_size == 128 || group_size == 256, QLQ_ERR_UNSUPPORTED,
              "group_size=%d not built (64, 128, 256)", group_size);
  QLQ_REQUIRE(K % group_size == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of group_size=%d",
              (long long)K, group_size);
  QLQ_REQUIRE(dtype_ok(w_dtype), QLQ_ERR_UNSUPPORTED, "w_dtype %d", w_dtype);
  QLQ_REQUIRE(aligned(w, 16) && aligned(q, 16) && aligned(scale, 4), QLQ_ERR_ALIGNMENT, "misaligned pointer");
  if (N == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_quantize_groups_int8(w, w_dtype, N, K, group_size, q, scale, (hipStream_t)stream),
                    "quantize groups");
}

QLQ_API size_t pergroup_workspace_size(int64_t M, int64_t K) {
  if (M <= 1 || K <= 0) return 0;  // M == 1 keeps x in floating point (larger shapes: w8a8_workspace_size gives 0)
  return w8a8_workspace_size(M, K);
}

QLQ_API int pergroup_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* w,
                                    const float* scale_w, int64_t N, int group_size, const void* bias, void* y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  QLQ_REQUIRE(((x && y) || M == 0) && w && scale_w, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim && N >= 1 && N < kMaxDim && K >= 1, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(group_size == 64 || group_size == 128 || group_size == 256, QLQ_ERR_UNSUPPORTED,
              "group_size=%d not built (64, 128, 256)", group_size);
  QLQ_REQUIRE(K % group_size == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of group_size=%d",
              (long long)K, group_size);
  QLQ_REQUIRE(x_dtype == QLQ_F16 || x_dtype == QLQ_BF16, QLQ_ERR_UNSUPPORTED, "x_dtype must be F16 or BF16");
  QLQ_REQUIRE(K <= 131071, QLQ_ERR_UNSUPPORTED, "K=%lld could overflow int32", (long long)K);
  QLQ_REQUIRE(M != 1 || K <= qlq::kPergroupMvMaxK, QLQ_ERR_UNSUPPORTED,
              "K=%lld above %lld for the M == 1 product", (long long)K, (long long)qlq::kPergroupMvMaxK);
  QLQ_REQUIRE(aligned(x, 16) && aligned(w, 16) && aligned(scale_w, 4) && aligned(y, 2) &&
                  (!bias || aligned(bias, 2)),
              QLQ_ERR_ALIGNMENT, "misaligned pointer");
  QLQ_REQUIRE((M + 127) / 128 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for one launch");
  if (M == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  if (M == 1) {
    if (int st = current_device_status()) return st;
    return hip_status(qlq::launch_pergroup_mv(x, x_dtype, K, w, scale_w, N, group_size, bias, y, s),
                      "per-group matrix-vector product");
  }
  const size_t need = pergroup_workspace_size(M, K);
  QLQ_REQUIRE(workspace && workspace_bytes >= need, QLQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  QLQ_REQUIRE(aligned(workspace, 16), QLQ_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  if (int st = current_device_status()) return st;
  int8_t* xq = (int8_t*)workspace;
  float* sx = (float*)((char*)workspace + (((size_t)M * (size_t)K + 255) & ~(size_t)255));
  if (int st = hip_status(qlq::launch_quantize_rows_int8(x, x_dtype, M, K, xq, sx, s), "activation quant"))
    return st;
  return hip_status(qlq::launch_int8_gemm_pergroup(xq, w, M, N, K, sx, scale_w, group_size, bias, x_dtype, y, s),
                    "per-group int8 gemm");
}

QLQ_API int w4a8_pack_weight_int4(const void* w, int w_dtype, int64_t K, int64_t N, uint8_t* packed, float* scale,
                                  void* stream) {
  QLQ_REQUIRE(w && packed && scale, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(K >= 2 && K < kMaxDim && N >= 0 && N < kMaxDim, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K % 2 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is odd", (long long)K);
  QLQ_REQUIRE(dtype_ok(w_dtype), QLQ_ERR_UNSUPPORTED, "w_dtype %d", w_dtype);
  QLQ_REQUIRE(aligned(w, dtype_size(w_dtype)) && aligned(scale, 4), QLQ_ERR_ALIGNMENT, "misaligned pointer");
  if (N == 0) return ok();
  if (int st = current_device_status()) return st;
  return hip_status(qlq::launch_pack_int4_cols(w, w_dtype, K, N, packed, scale, (hipStream_t)stream),
                    "pack int4");
}

QLQ_API size_t w4a8_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || N <= 0 || M >= kMaxDim || K >= kMaxDim || N >= kMaxDim) return 0;
  const size_t gemm = w8a8_workspace_size(M, K);
  if (M > qlq::kW4a8SkinnyMaxM) return gemm;
  const size_t skinny = qlq::w4a8_skinny_workspace(M, K, N);
  return skinny > gemm ? skinny : gemm;
}

QLQ_API int w4a8_linear_forward(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* packed_w,
                                const float* scale_w, int64_t N, const void* bias, void* y, void* workspace,
                                size_t workspace_bytes, void* stream) {
  QLQ_REQUIRE(((x && y) || M == 0) && packed_w && scale_w, QLQ_ERR_INVALID_ARG, "null pointer");
  QLQ_REQUIRE(M >= 0 && M < kMaxDim && N >= 1 && N < kMaxDim && K >= 16, QLQ_ERR_INVALID_ARG, "invalid shape");
  QLQ_REQUIRE(K % 16 == 0, QLQ_ERR_INVALID_ARG, "K=%lld is not a multiple of 16", (long long)K);
  QLQ_REQUIRE(K <= 131071, QLQ_ERR_UNSUPPORTED, "K=%lld could overflow int32", (long long)K);
  QLQ_REQUIRE((K / 2) * N < kMaxDim, QLQ_ERR_UNSUPPORTED, "packed weight of %lld bytes above 2^31",
              (long long)((K / 2) * N));
  QLQ_REQUIRE(x_dtype == QLQ_F16 || x_dtype == QLQ_BF16, QLQ_ERR_UNSUPPORTED, "x_dtype must be F16 or BF16");
  QLQ_REQUIRE(aligned(x, 16) && aligned(packed_w, 4) && aligned(scale_w, 4) && aligned(y, 2) &&
                  (!bias || aligned(bias, 2)),
              QLQ_ERR_ALIGNMENT, "misaligned pointer");
  QLQ_REQUIRE((M + 127) / 128 <= 65535, QLQ_ERR_UNSUPPORTED, "M too large for one launch");
  if (M == 0) return ok();
  const size_t need = w4a8_workspace_size(M, K, N);
  QLQ_REQUIRE(workspace && workspace_bytes >= need, QLQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  QLQ_REQUIRE(aligned(workspace, 16), QLQ_ERR_ALIGNMENT, "workspace not 16-byte aligned");
  if (int st = current_device_status()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (M <= qlq::kW4a8SkinnyMaxM && M <= g_skinny_max_m.load(std::memory_order_relaxed))
    return hip_status(qlq::launch_w4a8_skinny(x, x_dtype, M, K, packed_w, N, scale_w, bias, y, workspace, s),
                      "w4a8 skinny");
  int8_t* xq = (int8_t*)workspace;
  float* sx = (float*)((char*)workspace + (((size_t)M * (size_t)K + 255) & ~(size_t)255));
  if (int st = hip_status(qlq::launch_quantize_rows_int8(x, x_dtype, M, K, xq, sx, s, true), "activation quant"))
    return st;
  return hip_status(qlq::launch_w4a8_gemm(xq, packed_w, M, N, K, sx, scale_w, bias, x_dtype, y, s), "w4a8 gemm");
}

}  // extern "C"
