// Prefill-shaped affine forward (large M): y = x . dequant(W)^T (+ bias) on
// the fp16 matrix cores, dequantizing the packed codes in registers.
//
// "Struct QuantizedLinear" (nuvec-nn docs), forward: x W^T + b computed from
// the packed weight, its scales and biases; dequantization w = scale*q + bias
// (MLX affine docstring of pergroup_linear, "cider/ops.py", whose M > 1
// branch runs a GEMM on the matrix units).
//
// Arithmetic.  With per-row powers of two 2^e_m (x) and per-column 2^f_n (w):
//   y[m,n] = 2^(e_m + f_n) * sum_k x16[m,k] * w16[n,k]  (+ bias[n])
//   x16 = fp16(x * 2^-e_m)                  (exact: a bf16 or fp16 value
//                                            rescaled into fp16 range)
//   w16 = fp16((s*q + b) * 2^-f_n)           (one rounding, 2^-11 relative)
// Products of two fp16 values are exact in fp32; the MFMA accumulates in
// fp32.  The dequantization costs one packed fp16 FMA per two codes:
// (w >> bits*j) & mask leaves two codes in the low bits of two 16-bit lanes,
// which as fp16 bit patterns are the exact subnormals q*2^-24; with
// s' = fp16(s * 2^(24 - f_n)) and b' = fp16(b * 2^-f_n) (exact for bf16/fp16
// scales in range), v_pk_fma_f16(s', q*2^-24, b') = w16 for both lanes.
// Such a pair holds codes (j, j + 16/bits) of a word, so the pre-pass writes
// x16 in that k-order and the two operands stay aligned.
//
// f_n is the smallest exponent keeping s' below 2^15 and |s*q + b|*2^-f_n
// below 2^15 for every group of column n; e_m puts max|x[m,:]| in
// [2^14, 2^15).
//
// Tiling: 256 threads (2x2 waves), block tile 128x128, k-iteration 64, wave
// tile 64x64 = 2x2 MFMA 32x32x16 tiles, LDS double buffer fed from two
// register stages (one barrier per k-iteration), XCD-aware tile order.  Codes
// are dequantized once per block, while written to LDS.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace qlq {

namespace gemm {
constexpr int BM = 128, BN = 128, BK = 64, KS = 16;  // KS: MFMA k-step
constexpr int THREADS = 256;
constexpr int LDS_STRIDE = BK + 8;  // fp16 elements per LDS row (16-byte pad)
constexpr int A_U4 = BM * BK / 8 / THREADS;  // 4 uint4 of x16 per thread per k-iteration
}  // namespace gemm

__device__ __forceinline__ int floor_log2(float v) {  // v > 0, finite
  int e;
  frexpf(v, &e);  // v = f * 2^e, f in [0.5, 1)
  return e - 1;
}

// ------------------------------------------------------------------ pre-pass
// Column exponents f_n: one thread per column n.
template <int BITS, typename XT>
__device__ __forceinline__ void column_exponent(const XT* __restrict__ scales, const XT* __restrict__ biases,
                                                int n, int ng, int* __restrict__ wexp) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  int f = -1000;
  for (int g = 0; g < ng; ++g) {
    const float s = Elem<XT>::load(scales, (int64_t)n * ng + g);
    const float b = Elem<XT>::load(biases, (int64_t)n * ng + g);
    const float top = fabsf(b) + qmax * fabsf(s);
    if (s != 0.0f) f = max(f, floor_log2(fabsf(s)) + 10);
    if (top != 0.0f) f = max(f, floor_log2(top) - 14);
  }
  wexp[n] = f == -1000 ? 0 : f;
}

// x16[m, k] for one row held by one wave: element k of block b (PER codes)
// goes to position 2j or 2j+1 of the pair order (j, j + PER/2).  Lanes own
// groups of 16 consecutive elements, interleaved across the wave (16-byte
// coalesced loads and stores).  Blocks [0, ceil(M/4)) do rows (4 per block),
// the remaining blocks do the column exponents.
template <int BITS, typename XT, int EPT>
__global__ void __launch_bounds__(256)
gemm_prep_wave_kernel(const XT* __restrict__ x, int M, int K, const XT* __restrict__ scales,
                      const XT* __restrict__ biases, int N, int G, f16_t* __restrict__ x16,
                      int* __restrict__ xexp, int* __restrict__ wexp) {
  constexpr int PER = 32 / BITS;
  constexpr int HALF = PER / 2;
  constexpr int G16 = EPT / 16;
  const int row_blocks = (M + 3) / 4;
  if ((int)blockIdx.x >= row_blocks) {
    const int n = ((int)blockIdx.x - row_blocks) * 256 + threadIdx.x;
    if (n < N) column_exponent<BITS, XT>(scales, biases, n, K / G, wexp);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const XT* xr = x + (int64_t)m * K;
  float e[EPT];
  bool in[G16];
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    const int k = (g * 64 + lane) * 16;
    in[g] = k < K;
    float t[16];
    load16<XT>(xr + (in[g] ? k : 0), t);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[g * 16 + i] = in[g] ? t[i] : 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) amax = fmaxf(amax, fabsf(e[i]));
  amax = wave_max_dpp(amax);
  const int ex = amax > 0.0f ? floor_log2(amax) - 14 : 0;
  if (lane == 0) xexp[m] = ex;
  f16_t* out = x16 + (int64_t)m * K;
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    if (!in[g]) continue;
    uint32_t w[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {  // output pair p = positions 2p, 2p+1 of the 16
      const int lo = (2 * p) / PER * PER + p % HALF;  // (j, j + PER/2) within block
      const int i0 = PER >= 16 ? p : lo, i1 = PER >= 16 ? p + HALF : lo + HALF;
      const f16x2_v h = {(f16_t)ldexpf(e[g * 16 + i0], -ex), (f16_t)ldexpf(e[g * 16 + i1], -ex)};
      w[p] = __builtin_bit_cast(uint32_t, h);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + (g * 64 + lane) * 16);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// General K: one block per row (rows), then the column exponents.
template <int BITS, typename XT>
__global__ void __launch_bounds__(256)
gemm_prep_kernel(const XT* __restrict__ x, int M, int K, const XT* __restrict__ scales,
                 const XT* __restrict__ biases, int N, int G, f16_t* __restrict__ x16,
                 int* __restrict__ xexp, int* __restrict__ wexp) {
  constexpr int PER = 32 / BITS;  // codes per word = x block permuted together
  constexpr int HALF = PER / 2;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= M) {
    const int n = ((int)blockIdx.x - M) * 256 + tid;
    if (n < N) column_exponent<BITS, XT>(scales, biases, n, K / G, wexp);
    return;
  }
  __shared__ float red[4];
  const int m = blockIdx.x;
  const XT* xr = x + (int64_t)m * K;
  float amax = 0.0f;
  for (int k = tid * 8; k < K; k += 256 * 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(Elem<XT>::load(xr, k + i)));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = amax > 0.0f ? floor_log2(amax) - 14 : 0;
  if (tid == 0) xexp[m] = e;
  f16_t* out = x16 + (int64_t)m * K;
  // blocks of PER elements: out[2j] = x[j], out[2j+1] = x[j + PER/2]
  for (int k = tid * 8; k < K; k += 256 * 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = k + i, blk = kk / PER * PER, j = kk - blk;
      const int src = blk + (j >> 1) + ((j & 1) ? HALF : 0);
      out[kk] = (f16_t)ldexpf(Elem<XT>::load(xr, src), -e);
    }
  }
}

// ------------------------------------------------------------------- GEMM
template <int BITS, typename XT>
__global__ void __launch_bounds__(gemm::THREADS, 1)
affine_gemm_kernel(const f16_t* __restrict__ x16, const int* __restrict__ xexp, int M, int K,
                   const uint32_t* __restrict__ packed, const XT* __restrict__ scales,
                   const XT* __restrict__ biases, const int* __restrict__ wexp, int N, int G,
                   const XT* __restrict__ bias, XT* __restrict__ y) {
  using namespace gemm;
  constexpr int PER = 32 / BITS;                     // codes per word
  constexpr int WROW = BK / PER;                     // words per B row per k-iteration
  constexpr int B_U4 = BN * WROW / 4;                // uint4 of codes per k-iteration
  constexpr int B_U4_T = (B_U4 + THREADS - 1) / THREADS;
  constexpr int U4_PER_ROW = WROW / 4;               // 1 (2-bit), 2 (4-bit), 4 (8-bit)
  constexpr uint32_t MASK = ((1u << BITS) - 1u) * 0x00010001u;

  __shared__ __attribute__((aligned(16))) f16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) f16_t Bs[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  int tm, tn;
  tile_coords<8>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m_blk = tm * BM, n_blk = tn * BN;
  const int nk = K / BK;        // K % BK == 0 on this path
  const int ng = K / G;
  const int wpr = K / PER;      // words per packed row

  // A: rows of x16
  const f16_t* ap[A_U4];
  int a_lofs[A_U4];
#pragma unroll
  for (int i = 0; i < A_U4; ++i) {
    const int idx = tid + THREADS * i, r = idx / (BK / 8), c = idx % (BK / 8);
    ap[i] = x16 + (int64_t)min(m_blk + r, M - 1) * K + c * 8;
    a_lofs[i] = r * LDS_STRIDE + c * 8;
  }
  // B: this thread's packed-code uint4 (fixed row, fixed k offset in the tile)
  const uint32_t* bp[B_U4_T];
  int b_lofs[B_U4_T], b_kofs[B_U4_T];
  int64_t b_gbase[B_U4_T];
  int b_fexp[B_U4_T];  // f_n of this thread's row
  bool b_on[B_U4_T];
  // 2-bit codes: one uint4 holds 64 codes, which may span two groups of 32
  constexpr int SBN = BITS == 2 ? 2 : 1;
#pragma unroll
  for (int i = 0; i < B_U4_T; ++i) {
    const int idx = tid + THREADS * i;
    b_on[i] = idx < B_U4;
    const int r = b_on[i] ? idx / U4_PER_ROW : 0, c = idx % U4_PER_ROW;
    const int n = min(n_blk + r, N - 1);
    bp[i] = packed + (int64_t)n * wpr + c * 4;
    b_lofs[i] = r * LDS_STRIDE + c * 4 * PER;
    b_kofs[i] = c * 4 * PER;
    b_gbase[i] = (int64_t)n * ng;
    b_fexp[i] = wexp[n];
  }

  u32x4_v ra0[A_U4], ra1[A_U4], rb0[B_U4_T], rb1[B_U4_T];
  uint32_t rs0[B_U4_T][SBN], rs1[B_U4_T][SBN], rbi0[B_U4_T][SBN], rbi1[B_U4_T][SBN];  // raw 16-bit scale, bias

  // Stage operations, written as macros so that every register-array index is
  // a literal and the arrays stay in registers.  The load stage only issues
  // loads: any use of a loaded register there would make the compiler wait
  // for it at once and serialise the prefetch.
#define QLQ_LOAD(ST, IT)                                                                 \
  do {                                                                                   \
    const int k0_ = (IT) * BK;                                                           \
    _Pragma("unroll") for (int i = 0; i < A_U4; ++i)                                     \
        ra##ST[i] = *reinterpret_cast<const u32x4_v*>(ap[i] + k0_);                        \
    _Pragma("unroll") for (int i = 0; i < B_U4_T; ++i) {                                 \
      if (B_U4 % THREADS == 0 || b_on[i]) {                                              \
        rb##ST[i] = *reinterpret_cast<const u32x4_v*>(bp[i] + k0_ / PER);                  \
        _Pragma("unroll") for (int h = 0; h < SBN; ++h) {                                \
          const int64_t g_ = b_gbase[i] + (k0_ + b_kofs[i] + 32 * h) / G;               \
          rs##ST[i][h] = reinterpret_cast<const uint16_t*>(scales)[g_];                  \
          rbi##ST[i][h] = reinterpret_cast<const uint16_t*>(biases)[g_];                 \
        }                                                                                \
      }                                                                                  \
    }                                                                                    \
  } while (0)

#define QLQ_STORE(ST, BUF)                                                               \
  do {                                                                                   \
    _Pragma("unroll") for (int i = 0; i < A_U4; ++i)                                     \
        *reinterpret_cast<u32x4_v*>(&As[BUF][a_lofs[i]]) = ra##ST[i];                      \
    _Pragma("unroll") for (int i = 0; i < B_U4_T; ++i) {                                 \
      if (B_U4 % THREADS == 0 || b_on[i]) {                                              \
        f16x2_v s2_[SBN], b2_[SBN];                                                      \
        _Pragma("unroll") for (int h = 0; h < SBN; ++h) {                                \
          const float s_ = bits16_to_f32<XT>((uint16_t)rs##ST[i][h]);                    \
          const float bb_ = bits16_to_f32<XT>((uint16_t)rbi##ST[i][h]);                  \
          const f16_t s16_ = (f16_t)ldexpf(s_, 24 - b_fexp[i]);                          \
          const f16_t b16_ = (f16_t)ldexpf(bb_, -b_fexp[i]);                             \
          s2_[h] = f16x2_v{s16_, s16_};                                                  \
          b2_[h] = f16x2_v{b16_, b16_};                                                  \
        }                                                                                \
        const uint32_t w4_[4] = {rb##ST[i][0], rb##ST[i][1], rb##ST[i][2], rb##ST[i][3]};    \
        uint32_t d_[2 * PER];                                                            \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                  \
          const int h_ = SBN == 2 ? t / 2 : 0;                                           \
          _Pragma("unroll") for (int j = 0; j < PER / 2; ++j) {                          \
            const uint32_t qd_ = (w4_[t] >> (BITS * j)) & MASK;                          \
            const f16x2_v wv_ =                                                          \
                __builtin_elementwise_fma(s2_[h_], __builtin_bit_cast(f16x2_v, qd_), b2_[h_]); \
            d_[t * (PER / 2) + j] = __builtin_bit_cast(uint32_t, wv_);                   \
          }                                                                              \
        }                                                                                \
        f16_t* dst_ = &Bs[BUF][b_lofs[i]];                                               \
        _Pragma("unroll") for (int q = 0; q < PER / 2; ++q)                              \
            *reinterpret_cast<u32x4_v*>(dst_ + 8 * q) =                                  \
                u32x4_v{d_[4 * q], d_[4 * q + 1], d_[4 * q + 2], d_[4 * q + 3]};         \
      }                                                                                  \
    }                                                                                    \
  } while (0)

  // 32x32x16 fp16 MFMA: lane l holds 8 consecutive k of row (A) / column (B)
  // l % 32 at k offset 8 * (l / 32); result element e of lane l is row
  // 8*(e/4) + 4*(l/32) + e%4, column l % 32.
  f32x16_v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_v{};

  const int a_row = wm * 64 + (lane & 31), b_row = wn * 64 + (lane & 31);
  const int kofs = (lane >> 5) * 8;
#define QLQ_COMPUTE(BUF)                                                                             \
  do {                                                                                               \
    _Pragma("unroll") for (int ks = 0; ks < BK; ks += KS) {                                          \
      u32x4_v af_[2], bf_[2];                                                                        \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                  \
          af_[i] = *reinterpret_cast<const u32x4_v*>(&As[BUF][(a_row + 32 * i) * LDS_STRIDE + ks + kofs]); \
      _Pragma("unroll") for (int j = 0; j < 2; ++j)                                                  \
          bf_[j] = *reinterpret_cast<const u32x4_v*>(&Bs[BUF][(b_row + 32 * j) * LDS_STRIDE + ks + kofs]); \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                                  \
          _Pragma("unroll") for (int j = 0; j < 2; ++j) acc[i][j] =                                  \
              __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_v, af_[i]),            \
                                                     __builtin_bit_cast(f16x8_v, bf_[j]), acc[i][j], 0, 0, 0); \
    }                                                                                                \
  } while (0)

  // Loads past the last tile re-read the last tile (clamped index) and the
  // matching stores fill the idle buffer: both are harmless and keep the loop
  // body free of conditional register writes.
  const int last = nk - 1;
  QLQ_LOAD(0, 0);
  QLQ_LOAD(1, min(1, last));
  QLQ_STORE(0, 0);
  QLQ_LOAD(0, min(2, last));
  // The loop body holds a whole even/odd pair with no exit in between: an
  // exit there lets the compiler sink one stage's loads down to their first
  // use, which removes the prefetch.  An odd last tile is finished after it.
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    // even step: compute buffer 0; stage 1 (tile it+1) -> buffer 1
    __syncthreads();
    QLQ_STORE(1, 1);
    QLQ_LOAD(1, min(it + 3, last));
    QLQ_COMPUTE(0);
    // odd step: compute buffer 1; stage 0 (tile it+2) -> buffer 0
    __syncthreads();
    QLQ_STORE(0, 0);
    QLQ_LOAD(0, min(it + 4, last));
    QLQ_COMPUTE(1);
  }
  if (it < nk) {  // odd nk: buffer 0 holds the last tile
    __syncthreads();
    QLQ_COMPUTE(0);
  }
#undef QLQ_LOAD
#undef QLQ_STORE
#undef QLQ_COMPUTE

  // ---- epilogue: y = 2^(e_m + f_n) * acc + bias, one rounding
  int fcol[2];
  float bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = min(n_blk + wn * 64 + 32 * j + (lane & 31), N - 1);
    fcol[j] = wexp[n];
    bcol[j] = bias ? Elem<XT>::load(bias, n) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m_blk + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m >= M) continue;
      const int em = xexp[m];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n_blk + wn * 64 + 32 * j + (lane & 31);
        if (n >= N) continue;
        float v = ldexpf(acc[i][j][e], em + fcol[j]);
        if (bias) v = v + bcol[j];
        Elem<XT>::store(y, (int64_t)m * N + n, v);
      }
    }
  }
}

size_t affine_gemm_workspace(int64_t M, int64_t K, int64_t N) {
  size_t x16 = ((size_t)M * (size_t)K * 2 + 255) & ~(size_t)255;
  size_t xe = ((size_t)M * 4 + 255) & ~(size_t)255;
  return x16 + xe + (size_t)N * 4;
}

template <int BITS, typename XT>
static hipError_t gemm_launch(const void* x, int64_t M, int64_t K, const uint32_t* packed,
                              const void* scales, const void* biases, int64_t N, int G,
                              const void* bias, void* y, void* ws, hipStream_t s) {
  f16_t* x16 = (f16_t*)ws;
  const size_t x16b = ((size_t)M * (size_t)K * 2 + 255) & ~(size_t)255;
  int* xexp = (int*)((char*)ws + x16b);
  int* wexp = (int*)((char*)ws + x16b + (((size_t)M * 4 + 255) & ~(size_t)255));
  const int m = (int)M, n = (int)N, k = (int)K;
  if (K <= 64 * 64) {
    const unsigned blocks = (unsigned)(cdiv(M, 4) + cdiv(N, 256));
#define QLQ_PREP(EPT_)                                                                                  \
  hipLaunchKernelGGL((gemm_prep_wave_kernel<BITS, XT, EPT_>), dim3(blocks), dim3(256), 0, s, (const XT*)x, m, \
                     k, (const XT*)scales, (const XT*)biases, n, G, x16, xexp, wexp)
    if (K <= 64 * 16) QLQ_PREP(16);
    else if (K <= 64 * 32) QLQ_PREP(32);
    else QLQ_PREP(64);
#undef QLQ_PREP
  } else {
    hipLaunchKernelGGL((gemm_prep_kernel<BITS, XT>), dim3((unsigned)(M + cdiv(N, 256))), dim3(256), 0, s,
                       (const XT*)x, m, k, (const XT*)scales, (const XT*)biases, n, G, x16, xexp, wexp);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = cdiv(M, gemm::BM) * cdiv(N, gemm::BN);
  hipLaunchKernelGGL((affine_gemm_kernel<BITS, XT>), dim3((unsigned)tiles), dim3(gemm::THREADS), 0, s,
                     (const f16_t*)x16, (const int*)xexp, m, k, packed, (const XT*)scales, (const XT*)biases,
                     (const int*)wexp, n, G, (const XT*)bias, (XT*)y);
  return hipGetLastError();
}

template <int BITS>
static hipError_t gemm_dispatch_x(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const uint32_t* packed, const void* scales, const void* biases,
                                  int64_t N, int G, const void* bias, void* y, void* ws,
                                  hipStream_t s) {
  if (x_dtype == BF16) return gemm_launch<BITS, bf16_t>(x, M, K, packed, scales, biases, N, G, bias, y, ws, s);
  return gemm_launch<BITS, f16_t>(x, M, K, packed, scales, biases, N, G, bias, y, ws, s);
}

hipError_t launch_affine_gemm(const void* x, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, const void* scales, const void* biases,
                              int64_t N, int bits, int G, const void* bias, void* y,
                              void* workspace, hipStream_t s) {
  switch (bits) {
    case 2: return gemm_dispatch_x<2>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, workspace, s);
    case 4: return gemm_dispatch_x<4>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, workspace, s);
    default: return gemm_dispatch_x<8>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, workspace, s);
  }
}

}  // namespace qlq
