// Ternary BitLinear forward: y[m, r + j*R] = sigma * sum_k x[m,k] * (c - 1)
// (+ bias) with c = bits 2j..2j+1 of packed[r, k] and R = N/4.
//
// "mlx-lm/mlx_lm/models/bitlinear_layers.py": make_bitlinear_kernel (layout,
// decode c - 1, multiply by weight_scale or by its reciprocal) and
// BitLinear.__call__ (bias added after the scaled product).
//
// The prior-art Metal kernel re-reads every packed row once per batch row and
// accumulates on the vector ALU.  Here each packed byte is read once for all
// batch rows and the contraction runs on the matrix cores:
//  * one block (16 waves) owns 16 packed rows = 64 output rows (4 fields);
//    the waves split K, issue all their loads before computing, and an
//    LDS reduction joins their partial sums;
//  * per 32-k step a lane loads 8 bytes (packed row l%16, 8 consecutive k) and
//    turns field j of each 4-byte dword into two 16-bit float pairs with one
//    shift and one and-or:  ((d >> 2j) & 0x00030003) | MAGIC = (OFF + c_k,
//    OFF + c_k+2)  (OFF = 128 for bf16, 1024 for f16, exact), giving the B
//    operand of one MFMA 16x16x32 per field; the four fields share one A
//    operand (x, rows padded to 16 with zeros, k permuted to match);
//  * sum x*(OFF + c) - (OFF + 1) * sum x = sum x*(c - 1); products are exact
//    and accumulate in fp32.
// fp32 x takes a plain vector-ALU kernel.
#include "common.hpp"
#include "launch.hpp"

namespace qlq {

namespace tern {
constexpr int ROWS = 16;     // packed rows per block
constexpr int WAVES = 16;    // waves per block; they split K
constexpr int THREADS = 64 * WAVES;
constexpr int KS = 32;       // MFMA k-step
constexpr int BATCH = 8;     // k-steps a wave loads before computing
}  // namespace tern

template <typename XT> struct TernT;
template <> struct TernT<bf16_t> {
  static constexpr uint32_t MAGIC = 0x43004300u;
  static constexpr uint32_t ONES = 0x3F803F80u;
  static constexpr float OFF = 128.0f;
  static __device__ __forceinline__ f32x4_v mma(u32x4_v a, u32x4_v b, f32x4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                   __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                           __builtin_bit_cast(bf16x2_v, b), c, false);
  }
};
template <> struct TernT<f16_t> {
  static constexpr uint32_t MAGIC = 0x64006400u;
  static constexpr uint32_t ONES = 0x3C003C00u;
  static constexpr float OFF = 1024.0f;
  static __device__ __forceinline__ f32x4_v mma(u32x4_v a, u32x4_v b, f32x4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a),
                                                  __builtin_bit_cast(f16x8_v, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_v, a), __builtin_bit_cast(f16x2_v, b), c,
                                  false);
  }
};

// One block: 16 packed rows x 16 rows of x.  Wave w takes k-steps w, w+16, ...
// in batches of BATCH: every load of a batch is issued before its MFMAs, so a
// wave makes one memory round trip per batch (one in total for K <= 4096).
template <typename XT>
__global__ void __launch_bounds__(tern::THREADS)
ternary_mfma_kernel(const XT* __restrict__ x, int M, int K, const uint8_t* __restrict__ packed,
                    int R, const XT* __restrict__ wscale, int invert,
                    const XT* __restrict__ bias, XT* __restrict__ y) {
  using namespace tern;
  using TT = TernT<XT>;
  __shared__ float red[WAVES][4][4][64];  // [wave][field][elem][lane]
  __shared__ float xsum_sh[WAVES][16];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r0 = blockIdx.x * ROWS;
  const int m0 = blockIdx.y * 16;
  const int N = 4 * R;
  const int prow = min(r0 + (lane & 15), R - 1);
  const int mrow = m0 + (lane & 15);
  const bool mvalid = mrow < M;
  const int kofs = (lane >> 4) * 8;
  const uint8_t* wp = packed + (int64_t)prow * K + kofs;
  const XT* xp = x + (int64_t)(mvalid ? mrow : 0) * K + kofs;

  f32x4_v P[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) P[j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  float xs = 0.0f;

  const int nsteps = K / KS;
  for (int base = wid; base < nsteps; base += WAVES * BATCH) {
    uint2 wb[BATCH];
    u32x4_v xv[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int st = min(base + b * WAVES, nsteps - 1);  // clamped: extra steps are dropped below
      wb[b] = *reinterpret_cast<const uint2*>(wp + st * KS);
      xv[b] = *reinterpret_cast<const u32x4_v*>(xp + st * KS);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (base + b * WAVES >= nsteps) break;
      const u32x4_v v = mvalid ? xv[b] : u32x4_v{0, 0, 0, 0};
      // x pairs in the code order of a dword: (k0,k2), (k1,k3) per 4 k
      u32x4_v a;
      a[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
      a[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
      a[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
      a[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
      xs = TT::dot2(v[3], TT::ONES, TT::dot2(v[2], TT::ONES, TT::dot2(v[1], TT::ONES, TT::dot2(v[0], TT::ONES, xs))));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_v bq;
        bq[0] = ((wb[b].x >> (2 * j)) & 0x00030003u) | TT::MAGIC;
        bq[1] = ((wb[b].x >> (2 * j + 8)) & 0x00030003u) | TT::MAGIC;
        bq[2] = ((wb[b].y >> (2 * j)) & 0x00030003u) | TT::MAGIC;
        bq[3] = ((wb[b].y >> (2 * j + 8)) & 0x00030003u) | TT::MAGIC;
        P[j] = TT::mma(a, bq, P[j]);
      }
    }
  }
  // X[m] partial: lanes l, l+16, l+32, l+48 hold the same row
  xs += __shfl_xor(xs, 16, kWave);
  xs += __shfl_xor(xs, 32, kWave);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wid][j][e][lane] = P[j][e];
  if (lane < 16) xsum_sh[wid][lane] = xs;
  __syncthreads();

  const float ws = Elem<XT>::load(wscale, 0);
  const float sigma = invert ? __fdiv_rn(1.0f, ws) : ws;
  // block outputs: 16 m x 4 fields x 16 packed rows = 1024, one per thread
  for (int o = tid; o < 1024; o += THREADS) {
    const int ri = o & 15, mi = (o >> 4) & 15, j = o >> 8;
    // D layout: lane = (mi / 4) * 16 + ri holds row mi at element mi % 4
    const int src_lane = (mi >> 2) * 16 + ri, e = mi & 3;
    float p = 0.0f, X = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      p += red[w][j][e][src_lane];
      X += xsum_sh[w][mi];
    }
    const int m = m0 + mi, r = r0 + ri;
    if (m < M && r < R) {
      const int n = r + j * R;
      float v = sigma * __fmaf_rn(-(TT::OFF + 1.0f), X, p);
      if (bias) v = v + Elem<XT>::load(bias, n);
      Elem<XT>::store(y, (int64_t)m * N + n, v);
    }
  }
}

// fp32 x: one wave per (m, packed row), lanes stride over K.
__global__ void __launch_bounds__(256)
ternary_f32_kernel(const float* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
                   int64_t R, const float* __restrict__ wscale, int invert,
                   const float* __restrict__ bias, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= M * R) return;
  const int64_t m = wv / R, r = wv % R;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k = lane; k < K; k += 64) {
    const float xv = x[m * K + k];
    const uint32_t b = packed[r * K + k];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __fmaf_rn(xv, (float)((int)((b >> (2 * j)) & 3u) - 1), acc[j]);
  }
  const float ws = wscale[0];
  const float sigma = invert ? __fdiv_rn(1.0f, ws) : ws;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v = wave_sum(acc[j]);
    if (lane == 0) {
      const int64_t n = r + j * R;
      v = sigma * v;
      if (bias) v = v + bias[n];
      y[m * 4 * R + n] = v;
    }
  }
}

hipError_t launch_ternary_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const uint8_t* packed, int64_t N, const void* weight_scale,
                                  int invert, const void* bias, void* y, hipStream_t s) {
  const int64_t R = N / 4;
  if (x_dtype == F32) {
    dim3 grid((unsigned)cdiv(M * R, 4)), block(256);
    hipLaunchKernelGGL(ternary_f32_kernel, grid, block, 0, s, (const float*)x, M, K, packed, R,
                       (const float*)weight_scale, invert, (const float*)bias, (float*)y);
    return hipGetLastError();
  }
  dim3 grid((unsigned)cdiv(R, tern::ROWS), (unsigned)cdiv(M, 16)), block(tern::THREADS);
  const int m = (int)M, k = (int)K, r = (int)R;
  if (x_dtype == BF16)
    hipLaunchKernelGGL(ternary_mfma_kernel<bf16_t>, grid, block, 0, s, (const bf16_t*)x, m, k, packed, r,
                       (const bf16_t*)weight_scale, invert, (const bf16_t*)bias, (bf16_t*)y);
  else
    hipLaunchKernelGGL(ternary_mfma_kernel<f16_t>, grid, block, 0, s, (const f16_t*)x, m, k, packed, r,
                       (const f16_t*)weight_scale, invert, (const f16_t*)bias, (f16_t*)y);
  return hipGetLastError();
}

}  // namespace qlq
