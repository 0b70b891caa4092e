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
//  * one block (4 waves) owns 8 packed rows = 32 output rows (4 fields);
//    the waves split K, issue their loads before computing, and an LDS
//    reduction joins their partial sums;
//  * a field's 2-bit codes become 16-bit floats in place: masking bits
//    2f, 2f+1 of a dword shifted by 4t and or-ing MAGIC gives the pair
//    (OFF + 4^f c_k, OFF + 4^f c_k+2) exactly (OFF = 128 for bf16, 1024 for
//    f16), the B operand of an MFMA 16x16x32; x is the A operand (16 rows,
//    k permuted to match);
//  * sum x*(OFF + 4^f c) = OFF sum x + 4^f sum x*c, so
//    sum x*(c - 1) = (P - OFF X) / 4^f - X; products are exact and
//    accumulate in fp32.
// fp32 x takes a plain vector-ALU kernel.
#include "common.hpp"
#include "launch.hpp"

namespace qlq {

namespace tern {
constexpr int ROWS = 8;      // packed rows per block (32 outputs)
constexpr int WAVES = 4;     // waves per block; they split K
constexpr int KW = 128;      // k window: a lane loads 32 consecutive k of it
constexpr int NB = 5;        // windows a wave loads before computing
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

// One block: 8 packed rows x 16 rows of x; its waves split K in windows of
// 128 k.
//  * MFMA column n (= lane % 16) is packed row n % 8; MFMA t covers field
//    2t + n / 8 of it, so two MFMAs per k-step cover the 4 fields.  The
//    field's two code bits are masked where they sit, after a shift by 4t
//    shared by the lanes: (w >> 4t) & (0x00030003 << 2f) | MAGIC is the pair
//    (OFF + 4^f c, OFF + 4^f c') with f = n / 8, exact; the epilogue divides
//    by 4^f.
//  * In a window, lane group q (= lane / 16) owns the 32 consecutive k
//    32q .. 32q + 31 of its packed row (32 bytes, two 16-byte loads) and of
//    its x row (64 bytes, four loads), so one wave reads whole 128-byte
//    lines; MFMA k-step s (0..3) of the window takes k = 32q + 8s .. + 7 from
//    lane group q for both operands (the same k reach A and B, in an order
//    the sum does not see).
//  * A wave issues the loads of NB windows (indexes clamped, no branch), then
//    computes them in issue order with no branch, so each window waits only
//    for its own loads.  MASK: K is not a multiple of 128 or the windows do
//    not split evenly; a lane's k past K (or a window past the end) then
//    reads zeros for x.  Rows of x past M read zeros through the buffer
//    range check (no memory traffic); their outputs are never stored.
template <typename XT, bool MASK>
__global__ void __launch_bounds__(64 * tern::WAVES)
ternary_mfma_kernel(const XT* __restrict__ x, int M, int K, const uint8_t* __restrict__ packed,
                    int R, const XT* __restrict__ wscale, int invert,
                    const XT* __restrict__ bias, XT* __restrict__ y) {
  using namespace tern;
  using TT = TernT<XT>;
  __shared__ float red[WAVES][2][4][64];  // [wave][mfma][elem][lane]
  __shared__ float xsum_sh[WAVES][16];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r0 = blockIdx.x * ROWS;
  const int m0 = blockIdx.y * 16;
  const int N = 4 * R;
  const int n = lane & 15;
  const int prow = min(r0 + (n & 7), R - 1);
  const uint32_t fmask = 0x00030003u << (2 * (n >> 3));
  const int q = lane >> 4;
  // the block's packed rows through one buffer descriptor; this lane's row
  // in the offset
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed + (int64_t)r0 * K, (min(R, r0 + ROWS) - r0) * K);
  const int wrow = (prow - r0) * K;
  // the block's 16 x rows through one descriptor as well (cached: every block reads them)
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)m0 * K, (min(M, m0 + 16) - m0) * K * 2);
  // row m0 + n; rows past M lie past the descriptor's range and load zeros
  // without touching memory
  const int xrow = n * K * 2;

  f32x4_v P[2];
  P[0] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  P[1] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  float xs = 0.0f;

  const int nwin = (K + KW - 1) / KW;
  for (int base = wid; base < nwin; base += WAVES * NB) {
    uint4 wb[NB][2];
    u32x4_v xv[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int win = min(base + b * WAVES, nwin - 1);
      const int kc = min(win * KW + 32 * q, K - 32);
      // each packed byte is read once: streaming loads
      const u32x4_v w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow + kc, 0, kStreamAux);
      const u32x4_v w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow + kc + 16, 0, kStreamAux);
      wb[b][0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
      wb[b][1] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[b][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xrow + 2 * (kc + 8 * j), 0, 0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // K % 32 == 0: a lane's 32 k of the window are all inside K or all past it
      const bool use = !MASK || (base + b * WAVES < nwin && (base + b * WAVES) * KW + 32 * q < K);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_v v = use ? xv[b][st] : u32x4_v{0, 0, 0, 0};
        // x pairs in the code order of a dword: (k0,k2), (k1,k3) per 4 k
        u32x4_v a;
        a[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
        a[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
        a[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
        a[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
        xs = TT::dot2(v[3], TT::ONES, TT::dot2(v[2], TT::ONES, TT::dot2(v[1], TT::ONES, TT::dot2(v[0], TT::ONES, xs))));
        const uint4 h = wb[b][st >> 1];
        const uint32_t w0 = (st & 1) ? h.z : h.x, w1 = (st & 1) ? h.w : h.y;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4_v bq;
          bq[0] = ((w0 >> (4 * t)) & fmask) | TT::MAGIC;
          bq[1] = ((w0 >> (4 * t + 8)) & fmask) | TT::MAGIC;
          bq[2] = ((w1 >> (4 * t)) & fmask) | TT::MAGIC;
          bq[3] = ((w1 >> (4 * t + 8)) & fmask) | TT::MAGIC;
          P[t] = TT::mma(a, bq, P[t]);
        }
      }
    }
  }
  // X[m] partial: lanes l, l+16, l+32, l+48 hold the same row
  xs += __shfl_xor(xs, 16, kWave);
  xs += __shfl_xor(xs, 32, kWave);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wid][t][e][lane] = P[t][e];
  if (lane < 16) xsum_sh[wid][lane] = xs;
  __syncthreads();

  const float ws = Elem<XT>::load(wscale, 0);
  const float sigma = invert ? __fdiv_rn(1.0f, ws) : ws;
  // block outputs: 16 m x 4 fields x 8 packed rows = 512
  for (int o = tid; o < 512; o += 64 * WAVES) {
    const int ri = o & 7, mi = (o >> 3) & 15, j = o >> 7;
    // D layout: lane (mi / 4) * 16 + column holds row mi at element mi % 4;
    // field j is MFMA j / 2, column ri + 8 (j % 2), scaled by 4^(j % 2)
    const int t = j >> 1, src_lane = (mi >> 2) * 16 + ri + 8 * (j & 1), e = mi & 3;
    float p = 0.0f, X = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      p += red[w][t][e][src_lane];
      X += xsum_sh[w][mi];
    }
    const int m = m0 + mi, r = r0 + ri;
    if (m < M && r < R) {
      const int nn = r + j * R;
      // sum x (c - 1) = (P - OFF X) / 4^f - X
      const float c = __fmaf_rn(-TT::OFF, X, p) * ((j & 1) ? 0.25f : 1.0f);
      float v = sigma * (c - X);
      if (bias) v = v + Elem<XT>::load(bias, nn);
      Elem<XT>::store(y, (int64_t)m * N + nn, v);
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
  using namespace tern;
  dim3 grid((unsigned)cdiv(R, ROWS), (unsigned)cdiv(M, 16)), block(64 * WAVES);
  const int m = (int)M, k = (int)K, r = (int)R;
  const int64_t nwin = cdiv(K, KW);
  const bool mask = K % KW != 0 || nwin % (WAVES * NB) != 0;
#define QLQ_TERN(XT_, MASK_)                                                                               \
  hipLaunchKernelGGL((ternary_mfma_kernel<XT_, MASK_>), grid, block, 0, s, (const XT_*)x, m, k, packed, r, \
                     (const XT_*)weight_scale, invert, (const XT_*)bias, (XT_*)y)
  if (x_dtype == BF16) {
    if (mask) QLQ_TERN(bf16_t, true); else QLQ_TERN(bf16_t, false);
  } else {
    if (mask) QLQ_TERN(f16_t, true); else QLQ_TERN(f16_t, false);
  }
#undef QLQ_TERN
  return hipGetLastError();
}

}  // namespace qlq
