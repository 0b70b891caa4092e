// int8 x int8 -> int32 GEMM on the int8 matrix cores, with either a raw
// int32 output or the W8A8 scale epilogue.
//
// "cider/ops.py": int8_matmul_int32 (a [M,K] int8 times b [N,K] int8, the
// transposed weight layout, to int32 [M,N], bit-exact) and perchannel_linear
// (y = dequant(quant_a(x) @ w_int8) + bias with per-row weight scales).
//
// c[m,n] = sum_k a[m,k] * b[n,k] accumulates exactly in int32 (|c| <= 2^14 K).
// Epilogue: y = fp32(c) * sa[m] * sb[n] (+ bias[n]), rounded once to the
// output dtype.
//
// Tiling: block tile 128x128, k-iteration 128, 8 waves: 4 sub-tiles of 64x64
// (2x2 MFMA 32x32x32 tiles) times 2 halves of each k-iteration's k-steps, so
// two waves share each SIMD while one block covers a CU; the halves are summed
// through LDS at the end.  LDS double buffer fed from two register stages,
// XCD-aware tile order.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace qlq {

namespace i8 {
constexpr int BM = 128, BN = 128, BK = 128, KS = 32;  // KS: MFMA k-step
constexpr int WAVES = 8;   // 4 sub-tiles x 2 halves of each k-iteration
constexpr int THREADS = 64 * WAVES;
constexpr int LDS_STRIDE = BK + 16;  // bytes per LDS row (16-byte pad)
constexpr int U4_T = BM * BK / 16 / THREADS;  // 16-byte loads per thread per operand
}  // namespace i8

typedef __attribute__((ext_vector_type(16))) int i32x16_v;
// 32x32x32 int8 MFMA.  Operands: lane l holds 16 consecutive k (bytes) of row
// (A) or column (B) l % 32, k offset 16 * (l / 32).  Result: lane l, element e
// is row 8*(e/4) + 4*(l/32) + e%4, column l % 32.
__device__ __forceinline__ i32x16_v mma_i8(u32x4_v a, u32x4_v b, i32x16_v c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_v, a), __builtin_bit_cast(i32x4_v, b),
                                                c, 0, 0, 0);
}

// Pipeline (one barrier per k-iteration): register stage (it+1)%2 holds the
// tile of iteration it+1, loaded two iterations earlier.  Step `it`:
//   barrier; store regs[(it+1)%2] -> LDS[(it+1)%2]; load tile it+3 into the
//   freed registers; compute tile it from LDS[it%2].
// Two tiles stay in flight while a third is computed.  Rows past M / N and
// k past K are read from clamped addresses and zeroed with a select, so the
// loop has no branches.
template <int OUT>
__global__ void __launch_bounds__(i8::THREADS, 1)
int8_gemm_kernel(const int8_t* __restrict__ a, const int8_t* __restrict__ b, int M, int N, int K,
                 const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
                 void* __restrict__ out) {
  using namespace i8;
  // one LDS allocation: two A and two B tile buffers during the K loop, then
  // the 64 KiB of int32 partial sums that join the two k-halves
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * (BM + BN) * LDS_STRIDE];
  static_assert(2 * (BM + BN) * LDS_STRIDE >= 4 * 64 * 64 * 4, "reduction area fits");
  int8_t (*As)[BM * LDS_STRIDE] = reinterpret_cast<int8_t (*)[BM * LDS_STRIDE]>(smem);
  int8_t (*Bs)[BN * LDS_STRIDE] = reinterpret_cast<int8_t (*)[BN * LDS_STRIDE]>(smem + 2 * BM * LDS_STRIDE);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wq = wid & 3, kh = wid >> 2;  // 64x64 sub-tile, half of the k-steps
  const int wm = wq >> 1, wn = wq & 1;
  int tm, tn;
  tile_coords<8>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m_blk = tm * BM, n_blk = tn * BN;
  const int nk = (K + BK - 1) / BK;

  // per-thread load coordinates (fixed across k-iterations)
  const int8_t* ap[U4_T];
  const int8_t* bp[U4_T];
  int lofs[U4_T], kc[U4_T];
#pragma unroll
  for (int i = 0; i < U4_T; ++i) {
    const int idx = tid + THREADS * i, r = idx / (BK / 16), c = idx % (BK / 16);
    const int gm = min(m_blk + r, M - 1), gn = min(n_blk + r, N - 1);
    ap[i] = a + (int64_t)gm * K + c * 16;
    bp[i] = b + (int64_t)gn * K + c * 16;
    lofs[i] = r * LDS_STRIDE + c * 16;
    kc[i] = c * 16;
  }
  u32x4_v ra0[U4_T], ra1[U4_T], rb0[U4_T], rb1[U4_T];
  // Stage operations as macros: literal register-array indices only.
  int k0s0 = 0, k0s1 = 0;  // k offset of the tile each register stage holds
  // Stage operations as macros: literal register-array indices only.  The
  // load stage only issues loads (any use of the loaded registers would make
  // the compiler wait for them right there); the K-tail zeroing happens when
  // the stage is written to LDS.
#define QLQ_LOAD(ST, IT)                                                   \
  do {                                                                     \
    k0s##ST = (IT) * BK;                                                   \
    _Pragma("unroll") for (int i = 0; i < U4_T; ++i) {                     \
      const int kk_ = k0s##ST + kc[i] < K ? k0s##ST : 0;                   \
      ra##ST[i] = *reinterpret_cast<const u32x4_v*>(ap[i] + kk_);          \
      rb##ST[i] = *reinterpret_cast<const u32x4_v*>(bp[i] + kk_);          \
    }                                                                      \
  } while (0)
#define QLQ_STORE(ST, BUF)                                                 \
  do {                                                                     \
    _Pragma("unroll") for (int i = 0; i < U4_T; ++i) {                     \
      const bool in_ = k0s##ST + kc[i] < K;                                \
      *reinterpret_cast<u32x4_v*>(&As[BUF][lofs[i]]) = in_ ? ra##ST[i] : u32x4_v{0, 0, 0, 0}; \
      *reinterpret_cast<u32x4_v*>(&Bs[BUF][lofs[i]]) = in_ ? rb##ST[i] : u32x4_v{0, 0, 0, 0}; \
    }                                                                      \
  } while (0)

  i32x16_v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = i32x16_v{};

  const int a_row = wm * 64 + (lane & 31), b_row = wn * 64 + (lane & 31);
  const int kofs = (lane >> 5) * 16;
#define QLQ_COMPUTE(BUF)                                                                               \
  do {                                                                                                 \
    _Pragma("unroll") for (int ks = kh * (BK / 2); ks < kh * (BK / 2) + BK / 2; ks += KS) {            \
      u32x4_v af_[2], bf_[2];                                                                          \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                    \
          af_[i] = *reinterpret_cast<const u32x4_v*>(&As[BUF][(a_row + 32 * i) * LDS_STRIDE + ks + kofs]); \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                    \
          bf_[j] = *reinterpret_cast<const u32x4_v*>(&Bs[BUF][(b_row + 32 * j) * LDS_STRIDE + ks + kofs]); \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                    \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] = mma_i8(af_[i], bf_[j], acc[i][j]);   \
    }                                                                                                  \
  } while (0)

  // Loads past the last tile re-read the last tile (clamped index) and the
  // matching stores fill the idle buffer: both are harmless and keep the loop
  // body free of conditional register writes.
  const int last = nk - 1;
  QLQ_LOAD(0, 0);
  QLQ_LOAD(1, min(1, last));
  QLQ_STORE(0, 0);
  QLQ_LOAD(0, min(2, last));
  for (int it = 0; it < nk; it += 2) {
    // even step: compute buffer 0; stage 1 (tile it+1) -> buffer 1
    __syncthreads();
    QLQ_STORE(1, 1);
    QLQ_LOAD(1, min(it + 3, last));
    QLQ_COMPUTE(0);
    if (it + 1 >= nk) break;
    // odd step: compute buffer 1; stage 0 (tile it+2) -> buffer 0
    __syncthreads();
    QLQ_STORE(0, 0);
    QLQ_LOAD(0, min(it + 4, last));
    QLQ_COMPUTE(1);
  }
#undef QLQ_LOAD
#undef QLQ_STORE
#undef QLQ_COMPUTE

  // ---- join the two k-halves: waves 4-7 park their sums in LDS (the tile
  // buffers are free now), waves 0-3 add them and run the epilogue
  int32_t* red = reinterpret_cast<int32_t*>(smem);  // 4 sub-tiles x 64 values x 64 lanes
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[(wq * 64 + (i * 2 + j) * 16 + e) * 64 + lane] = acc[i][j][e];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] += red[(wq * 64 + (i * 2 + j) * 16 + e) * 64 + lane];

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m_blk + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= M) continue;
      const float sam = OUT ? sa[m] : 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n_blk + wn * 64 + 32 * j + (lane & 31);
        if (n >= N) continue;
        if constexpr (OUT == 0) {
          reinterpret_cast<int32_t*>(out)[(int64_t)m * N + n] = acc[i][j][e];
        } else {
          float v = ((float)acc[i][j][e] * sam) * sb[n];
          if constexpr (OUT == 1) {
            if (bias) v = v + Elem<f16_t>::load((const f16_t*)bias, n);
            Elem<f16_t>::store((f16_t*)out, (int64_t)m * N + n, v);
          } else {
            if (bias) v = v + Elem<bf16_t>::load((const bf16_t*)bias, n);
            Elem<bf16_t>::store((bf16_t*)out, (int64_t)m * N + n, v);
          }
        }
      }
    }
  }
}

hipError_t launch_int8_gemm(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, const void* bias, int out_dtype,
                            void* out, hipStream_t s) {
  const int64_t tiles = cdiv(M, i8::BM) * cdiv(N, i8::BN);
  dim3 grid((unsigned)tiles), block(i8::THREADS);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (out_dtype < 0)
    hipLaunchKernelGGL(int8_gemm_kernel<0>, grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  else if (out_dtype == F16)
    hipLaunchKernelGGL(int8_gemm_kernel<1>, grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  else
    hipLaunchKernelGGL(int8_gemm_kernel<2>, grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  return hipGetLastError();
}

}  // namespace qlq
