// Host-side driver for the sanitized build of the C ABI (address and
// undefined-behaviour sanitizers on the host code of api.cpp): every entry
// point is called with arguments that its host validation must reject, with
// extreme sizes whose byte counts overflow 32 and 64 bits, and with empty
// batches, and the status codes are checked.  Pointers are fake, aligned,
// non-null addresses; no call may reach the device (on a machine without a
// GPU the fully valid calls at the end return QLQ_ERR_DEVICE).  Prints
// "PASS <n>" and exits 0, or names the first failing check and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/qlq.h"

namespace {

int g_checks = 0;

#define EXPECT(call, want)                                                                              \
  do {                                                                                                  \
    const int got_ = (call);                                                                            \
    ++g_checks;                                                                                         \
    if (got_ != (want)) {                                                                               \
      std::printf("FAIL line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_, (int)(want), \
                  qlq_last_error());                                                                     \
      return 1;                                                                                         \
    }                                                                                                   \
    if ((want) != QLQ_OK && std::strlen(qlq_last_error()) == 0) {                                        \
      std::printf("FAIL line %d: %s set no error text\n", __LINE__, #call);                              \
      return 1;                                                                                         \
    }                                                                                                   \
  } while (0)

#define EXPECT_SIZE(expr, cond)                                              \
  do {                                                                       \
    const size_t v_ = (expr);                                                \
    ++g_checks;                                                              \
    if (!(cond)) {                                                           \
      std::printf("FAIL line %d: %s = %zu\n", __LINE__, #expr, v_);          \
      return 1;                                                              \
    }                                                                        \
  } while (0)

void* const A = reinterpret_cast<void*>(0x100000);  // 16-byte aligned fake device addresses
void* const B = reinterpret_cast<void*>(0x200000);
void* const ODD = reinterpret_cast<void*>(0x100002);
const int64_t BIG = (int64_t)1 << 40;

int affine() {
  const uint32_t* P = static_cast<const uint32_t*>(A);
  EXPECT(qlq_linear_forward(nullptr, QLQ_BF16, 4, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, -1, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, BIG, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, BIG, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, 250, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, 256, P, A, A, QLQ_BF16, 64, 7, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, 256, P, A, A, QLQ_BF16, 64, 4, 48, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(qlq_linear_forward(A, 9, 4, 256, P, A, A, 9, 64, 4, 64, nullptr, A, nullptr, 0, nullptr), QLQ_ERR_UNSUPPORTED);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, 256, P, A, A, QLQ_F32, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_DTYPE);
  EXPECT(qlq_linear_forward(ODD, QLQ_BF16, 4, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_ALIGNMENT);
  EXPECT(qlq_linear_forward(A, QLQ_BF16, 4096, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, A, nullptr, 0, nullptr),
         QLQ_ERR_WORKSPACE);
  EXPECT(qlq_linear_forward(nullptr, QLQ_BF16, 0, 256, P, A, A, QLQ_BF16, 64, 4, 64, nullptr, nullptr, nullptr, 0,
                            nullptr),
         QLQ_OK);
  // workspace sizes: extreme and invalid arguments give 0 and never overflow
  EXPECT_SIZE(qlq_linear_workspace_size(BIG, BIG, BIG, 4, 64, QLQ_BF16), v_ == 0);
  EXPECT_SIZE(qlq_linear_workspace_size(-5, 4096, 4096, 4, 64, QLQ_BF16), v_ == 0);
  EXPECT_SIZE(qlq_linear_workspace_size(2048, 4096, 11008, 4, 0, QLQ_BF16), v_ == 0);
  EXPECT_SIZE(qlq_linear_workspace_size(2048, (1 << 22) + 128, 16256, 4, 128, QLQ_BF16), v_ == 0);
  EXPECT_SIZE(qlq_linear_workspace_size(2048, 4096, 11008, 3, 128, QLQ_BF16), v_ > (size_t)11008 * 4096 / 2);
  EXPECT(qlq_pack(nullptr, 8, 64, 4, 64, static_cast<uint32_t*>(A), A, A, QLQ_BF16, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_pack(static_cast<const float*>(A), 8, BIG, 4, 64, static_cast<uint32_t*>(A), A, A, QLQ_BF16, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_pack(static_cast<const float*>(ODD), 8, 64, 4, 64, static_cast<uint32_t*>(A), A, A, QLQ_BF16, nullptr),
         QLQ_ERR_ALIGNMENT);
  EXPECT(qlq_unpack(P, 4, 40, 3, static_cast<uint8_t*>(A), nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_unpack(P, 4, BIG, 4, static_cast<uint8_t*>(A), nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_dequantize(P, A, A, QLQ_BF16, 4, 64, 4, 48, static_cast<float*>(A), nullptr), QLQ_ERR_UNSUPPORTED);
  return 0;
}

int ternary() {
  const uint8_t* P = static_cast<const uint8_t*>(A);
  EXPECT(bitlinear_forward(A, QLQ_BF16, 8, 64, P, 6, B, 0, nullptr, A, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward(A, QLQ_BF16, 8, 48, P, 16, B, 0, nullptr, A, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward(A, QLQ_BF16, 8, 1 << 26, P, 16, B, 0, nullptr, A, nullptr), QLQ_ERR_UNSUPPORTED);
  EXPECT(bitlinear_forward(A, QLQ_BF16, BIG, 64, P, 16, B, 0, nullptr, A, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward(A, QLQ_BF16, 8, 64, P, 16, nullptr, 0, nullptr, A, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(bitlinear_forward(ODD, QLQ_BF16, 8, 64, P, 16, B, 0, nullptr, A, nullptr), QLQ_ERR_ALIGNMENT);
  EXPECT(bitlinear_forward(nullptr, QLQ_BF16, 0, 256, P, 64, A, 0, nullptr, nullptr, nullptr), QLQ_OK);
  EXPECT(bitlinear_pack(static_cast<const int8_t*>(A), 6, 8, static_cast<uint8_t*>(A), nullptr), QLQ_ERR_INVALID_ARG);
  return 0;
}

int int8_paths() {
  const int8_t* W = static_cast<const int8_t*>(B);
  const float* S = static_cast<const float*>(A);
  EXPECT(w8a8_linear_forward(A, QLQ_F16, 16, 40, W, S, 32, nullptr, A, B, 1 << 20, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(w8a8_linear_forward(A, QLQ_F16, 16, 131072, W, S, 32, nullptr, A, B, 1 << 20, nullptr), QLQ_ERR_UNSUPPORTED);
  EXPECT(w8a8_linear_forward(A, QLQ_F32, 16, 64, W, S, 32, nullptr, A, B, 1 << 20, nullptr), QLQ_ERR_UNSUPPORTED);
  EXPECT(w8a8_linear_forward(A, QLQ_F16, 16, 64, W, S, 32, nullptr, A, nullptr, 0, nullptr), QLQ_ERR_WORKSPACE);
  EXPECT(w8a8_linear_forward(A, QLQ_F16, 16, 64, W, S, 32, nullptr, A, B, 100, nullptr), QLQ_ERR_WORKSPACE);
  EXPECT(w8a8_linear_forward(A, QLQ_F16, BIG, 64, W, S, 32, nullptr, A, B, 1 << 20, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(w8a8_linear_forward(nullptr, QLQ_F16, 0, 64, W, S, 32, nullptr, nullptr, nullptr, 0, nullptr), QLQ_OK);
  EXPECT_SIZE(w8a8_workspace_size(BIG, BIG), v_ == 0);  // shapes no forward call accepts: 0, no wrap-around
  EXPECT_SIZE(w4a8_workspace_size(1, 4096, BIG), v_ == 0);
  EXPECT_SIZE(w8a8_workspace_size(0, 4096), v_ == 0);
  EXPECT(w8a8_linear_forward_noalloc(A, QLQ_F16, 4093, 4096, W, S, 32, nullptr, A, nullptr), QLQ_ERR_WORKSPACE);
  EXPECT(w8a8_linear_forward_noalloc(A, QLQ_F16, 16, 40, W, S, 32, nullptr, A, nullptr), QLQ_ERR_INVALID_ARG);
  EXPECT(w8a8_linear_forward_noalloc(nullptr, QLQ_F16, 0, 64, W, S, 32, nullptr, nullptr, nullptr), QLQ_OK);
  EXPECT(qlq_int8_matmul_int32(static_cast<const int8_t*>(A), W, 4, 4, 131088, static_cast<int32_t*>(A), nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(qlq_quantize_rows_int8(A, QLQ_F16, 4, 40, static_cast<int8_t*>(A), static_cast<float*>(A), nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_quantize_rows_int8_clip(A, QLQ_F32, 4, 16385, 99.9f, static_cast<int8_t*>(A), static_cast<float*>(B),
                                     nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(qlq_quantize_rows_int8_clip(A, QLQ_F32, 4, 64, 100.5f, static_cast<int8_t*>(A), static_cast<float*>(B),
                                     nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_quantize_groups_int8(A, QLQ_F32, 8, 128, 32, static_cast<int8_t*>(A), static_cast<float*>(B), nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(pergroup_linear_forward(A, QLQ_F16, 1, 32768, W, S, 32, 64, nullptr, A, B, 1 << 20, nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(pergroup_linear_forward(A, QLQ_F16, 4, 320, W, S, 32, 128, nullptr, A, B, 1 << 20, nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT_SIZE(pergroup_workspace_size(1, 4096), v_ == 0);
  EXPECT(w4a8_linear_forward(A, QLQ_F16, 16, 65536, static_cast<const uint8_t*>(B), S, 65536, nullptr, A, B, 1 << 20,
                             nullptr),
         QLQ_ERR_UNSUPPORTED);
  EXPECT(w4a8_pack_weight_int4(A, QLQ_F32, 63, 32, static_cast<uint8_t*>(A), static_cast<float*>(B), nullptr),
         QLQ_ERR_INVALID_ARG);
  EXPECT_SIZE(w4a8_workspace_size(1, 4096, 4096), v_ >= (size_t)32 * 4096 * 4);
  return 0;
}

int plumbing(bool no_device) {
  EXPECT(qlq_set_skinny_max_m(-1), QLQ_ERR_INVALID_ARG);
  const int old = qlq_get_skinny_max_m();
  EXPECT(qlq_set_skinny_max_m(3), QLQ_OK);
  EXPECT(qlq_set_skinny_max_m(old), QLQ_OK);
  EXPECT(qlq_set_w8a8_fused_quant(7), QLQ_ERR_INVALID_ARG);
  EXPECT(qlq_device_check(-1), QLQ_ERR_DEVICE);
  EXPECT(qlq_device_check(64), QLQ_ERR_DEVICE);
  if (no_device) {
    // fully valid arguments: validation passes, then the device check fails
    EXPECT(qlq_linear_forward(A, QLQ_BF16, 4, 256, static_cast<const uint32_t*>(A), A, A, QLQ_BF16, 64, 4, 64,
                              nullptr, A, nullptr, 0, nullptr),
           QLQ_ERR_DEVICE);
    EXPECT(w8a8_linear_forward_noalloc(A, QLQ_F16, 16, 64, static_cast<const int8_t*>(B),
                                       static_cast<const float*>(A), 32, nullptr, A, nullptr),
           QLQ_ERR_DEVICE);
  }
  if (std::strstr(qlq_version(), "gfx950") == nullptr) {
    std::printf("FAIL: version string %s\n", qlq_version());
    return 1;
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  if (affine() || ternary() || int8_paths() || plumbing(no_device)) return 1;
  std::printf("PASS %d\n", g_checks);
  return 0;
}
