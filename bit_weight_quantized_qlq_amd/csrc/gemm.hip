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
//   x16 = fp16(x * 2^-e_m)                  (exact for every element within
//                                            2^24 of the row maximum; smaller
//                                            ones fall into fp16 subnormals
//                                            and round, far below the bound)
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
// Tiling: 256 threads, block tile 256x128 (128x128 for few tiles), k-iteration
// 64; x16, packed codes
// and the pre-scaled (s', b') pairs go straight from global memory into a
// ring of LDS stages (one barrier per k-iteration); each wave dequantizes the
// codes of its own B fragments after reading them from LDS, so codes cross
// LDS at BITS/16 of the bytes of fp16 weights.  XCD-aware tile order.  A
// short tail of tiles past the last whole round of resident blocks runs as
// k-halves with fp32 partial sums, joined by a small second kernel.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace qlq {

#ifndef QLQ_PREP_ROWS_PER_WAVE
#define QLQ_PREP_ROWS_PER_WAVE 2  // pre-pass: x rows per wave (their loads all issued first)
#endif

namespace gemm {
constexpr int BN = 128;  // block columns
constexpr int WAVES = 4;     // waves per block (two blocks per compute unit)
constexpr int KB = 64;       // k-iteration
constexpr int NSTAGES = 2;   // LDS ring depth (double buffer: small enough for three blocks per CU)
// block rows: 256 (wave tile 128x64, half the dequantization per MFMA of
// 128-row blocks) when that still gives two blocks per compute unit
constexpr int TILE_M_TALL = 256, TILE_M = 128;
}  // namespace gemm

__device__ __forceinline__ int floor_log2(float v) {  // v > 0, finite
  int e;
  frexpf(v, &e);  // v = f * 2^e, f in [0.5, 1)
  return e - 1;
}

// ------------------------------------------------------------------ pre-pass
// Columns n0 .. n0+63 (one 256-thread block): exponent f_n (four threads per
// column, groups interleaved), then the fp16 pair (s', b') of every group,
// stored group-major (sbt[g * NP + n], NP = N rounded up to 4) so that a
// k-range's entries for a block of columns are contiguous; consecutive
// threads write consecutive columns.
template <int BITS, typename XT>
__device__ __forceinline__ void column_block(const XT* __restrict__ scales, const XT* __restrict__ biases,
                                             int n0, int N, int ng, int* __restrict__ wexp,
                                             uint32_t* __restrict__ sbt) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  __shared__ int fsh[64];
  const int tid = threadIdx.x, NP = (N + 3) & ~3;
  {
    const int c = tid >> 2, n = n0 + c;
    int f = -1000;
    if (n < N) {
#pragma unroll 4
      for (int g = tid & 3; g < ng; g += 4) {
        const float sv = Elem<XT>::load(scales, (int64_t)n * ng + g);
        const float bv = Elem<XT>::load(biases, (int64_t)n * ng + g);
        const float top = fabsf(bv) + qmax * fabsf(sv);
        if (sv != 0.0f) f = max(f, floor_log2(fabsf(sv)) + 10);
        if (top != 0.0f) f = max(f, floor_log2(top) - 14);
      }
    }
    f = max(f, __shfl_xor(f, 1, kWave));
    f = max(f, __shfl_xor(f, 2, kWave));
    f = f == -1000 ? 0 : f;
    if ((tid & 3) == 0) {
      fsh[c] = f;
      if (n < N) wexp[n] = f;
    }
  }
  __syncthreads();
  const int c = tid & 63, n = n0 + c;
  if (n >= N) return;
  const int f = fsh[c];
#pragma unroll 4
  for (int g = tid >> 6; g < ng; g += 4) {
    const float sv = Elem<XT>::load(scales, (int64_t)n * ng + g);
    const float bv = Elem<XT>::load(biases, (int64_t)n * ng + g);
    const f16_t s16 = (f16_t)ldexpf(sv, 24 - f), b16 = (f16_t)ldexpf(bv, -f);
    sbt[(int64_t)g * NP + n] = (uint32_t)__builtin_bit_cast(uint16_t, s16) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, b16) << 16);
  }
}

// x16[m, k] for RPW rows held by one wave, one after another: element k of
// block b (PER codes) goes to position 2j or 2j+1 of the pair order
// (j, j + PER/2).  Lanes own groups of 16 consecutive elements, interleaved
// across the wave (16-byte coalesced loads and stores).  Blocks
// [0, ceil(N/64)) do the column exponents, whose chains of dependent loads
// start first that way; the remaining blocks do rows (4 waves per block).
template <int BITS, typename XT, int EPT, int RPW>
__global__ void __launch_bounds__(256)
gemm_prep_wave_kernel(const XT* __restrict__ x, int M, int K, const XT* __restrict__ scales,
                      const XT* __restrict__ biases, int N, int G, f16_t* __restrict__ x16,
                      int* __restrict__ xexp, int* __restrict__ wexp, uint32_t* __restrict__ sbt) {
  constexpr int PER = 32 / BITS;
  constexpr int HALF = PER / 2;
  constexpr int G16 = EPT / 16;
  const int col_blocks = (N + 63) / 64;
  if ((int)blockIdx.x < col_blocks) {
    column_block<BITS, XT>(scales, biases, (int)blockIdx.x * 64, N, K / G, wexp, sbt);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int m0 = (((int)blockIdx.x - col_blocks) * 4 + (threadIdx.x >> 6)) * RPW;
  if (m0 >= M) return;
  // every row's loads first: the first row's conversion and stores then
  // overlap the later rows' reads
  float e[RPW][EPT];
  bool in[G16];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const XT* xr = x + (int64_t)(m0 + r < M ? m0 + r : m0) * K;
#pragma unroll
    for (int g = 0; g < G16; ++g) {
      const int k = (g * 64 + lane) * 16;
      in[g] = k < K;
      float t[16];
      load16<XT>(xr + (in[g] ? k : 0), t);
#pragma unroll
      for (int i = 0; i < 16; ++i) e[r][g * 16 + i] = in[g] ? t[i] : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int m = m0 + r;
    if (m >= M) break;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < EPT; ++i) amax = fmaxf(amax, fabsf(e[r][i]));
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
        const f16x2_v h = {(f16_t)ldexpf(e[r][g * 16 + i0], -ex), (f16_t)ldexpf(e[r][g * 16 + i1], -ex)};
        w[p] = __builtin_bit_cast(uint32_t, h);
      }
      uint4* dst = reinterpret_cast<uint4*>(out + (g * 64 + lane) * 16);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
  }
}

// General K: one block per row (rows), then the column exponents.
template <int BITS, typename XT>
__global__ void __launch_bounds__(256)
gemm_prep_kernel(const XT* __restrict__ x, int M, int K, const XT* __restrict__ scales,
                 const XT* __restrict__ biases, int N, int G, f16_t* __restrict__ x16,
                 int* __restrict__ xexp, int* __restrict__ wexp, uint32_t* __restrict__ sbt) {
  constexpr int PER = 32 / BITS;  // codes per word = x block permuted together
  constexpr int HALF = PER / 2;
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= M) {
    column_block<BITS, XT>(scales, biases, ((int)blockIdx.x - M) * 64, N, K / G, wexp, sbt);
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
// Block: 4 waves, tile BMT x 128 (BMT = 128 or 256).  Wave (wm, wn) owns the
// (BMT/2) x 64 sub-tile (wm, wn) and takes every k-step; two blocks share a
// compute unit.  Per stage of the LDS ring:
//   A  : BMT rows of x16, BK values (2*BK bytes) each, 16-byte chunks swizzled
//   B  : 128 packed rows, RB = BK*BITS/8 bytes each, chunks swizzled
//   SB : per 64-k sub-block, 512 bytes per group it touches: (s', b') of the
//        block's 128 columns
// all filled by buffer-to-LDS loads (out-of-range offsets write zeros).
//
// k order inside a 64-k sub-block.  The MFMA 32x32x16 f16 lane l holds 8
// k-values of its row/column; half h = l / 32 and k-step s (0..3) pick which
// 8.  Any order works if A and B agree, so the order is chosen to make each
// lane's codes contiguous:
//   4-bit: word 4h + s        (8 codes, pairs (j, j+4))        A chunk 4h + s
//   8-bit: words 8h+2s, +1    (2 x 4 codes, pairs (0,2),(1,3)) A chunk 4h + s
// (x16 already holds every word's values in the pair order).  1- to 3-bit
// codes reach this kernel rewritten as 4-bit codes, 5- and 6-bit ones as
// 8-bit codes.
namespace gemm {
template <int BITS, int BK, int STAGES, int WV, int BMT> struct Cfg {
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit packed codes");
  static constexpr int MI = BMT / 64;               // MFMA row tiles per wave (wave tile BMT/2 x 64)
  static constexpr int SPW = 4;                     // k-steps per 64-k sub-block
  static constexpr int U = BK / 64;                 // 64-k sub-blocks per k-iteration
  static constexpr int A_ROW = 2 * BK;              // bytes per A row
  static constexpr int A_CB = A_ROW / 16;           // chunks per A row
  static constexpr int A_TILE = BMT * A_ROW;
  static constexpr int RB = BK * BITS / 8;          // bytes per packed row per k-iteration
  static constexpr int B_CB = RB / 16;              // chunks per packed row
  static constexpr int B_TILE = BN * RB;
  // LDS, slot-major within each operand: [A slot 0..S-1][B slot 0..S-1][SB slot 0..S-1],
  // so that a fragment address is a fixed register plus a constant per slot
  static constexpr int B_BASE = STAGES * A_TILE;
  static constexpr int SB_BASE = B_BASE + STAGES * B_TILE;
  static constexpr int SB_TILE = U * 1024;
  static constexpr int STAGE = A_TILE + B_TILE + SB_TILE;
  static constexpr int A_RPI = 1024 / A_ROW;        // A rows per wave-wide load
  static constexpr int B_RPI = 1024 / RB;           // B rows per wave-wide load
  static constexpr int A_LOADS = A_TILE / 1024;     // wave-wide loads per stage
  static constexpr int B_LOADS = B_TILE / 1024;
  static constexpr int APW = A_LOADS / WV;          // A loads per wave
  static constexpr int NO = B_LOADS + U;            // B and SB loads, dealt round-robin
  static constexpr int LW = APW + NO / WV;          // loads per wave per stage (waves < NO % WV: +1)
  static constexpr int LDS = STAGES * STAGE;
  static_assert(WV == 4, "waves: a 2 x 2 grid of wave tiles");
  static_assert(BMT % 64 == 0 && BMT <= 256, "block rows");
  static_assert(A_LOADS % WV == 0 && B_TILE % 1024 == 0, "tile split");
  static_assert(STAGES == 2, "double buffer: every wait drains this wave's loads");
  static_assert(BK == 64, "K % 64 == 0 on this path: no k-iteration crosses K");
  static_assert(2 * LDS <= 160 * 1024, "LDS: two blocks per compute unit");
};
}  // namespace gemm

template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BITS, typename XT, int BK, int STAGES, int WV, int BMT>
__global__ void __launch_bounds__(64 * WV, 8 / WV)
affine_gemm_kernel(const f16_t* __restrict__ x16, const int* __restrict__ xexp, int M, int K,
                   const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sbt,
                   const int* __restrict__ wexp, int N, int G, const XT* __restrict__ bias,
                   XT* __restrict__ y, int tn_full, float* __restrict__ part, int n_split) {
  using namespace gemm;
  using C = Cfg<BITS, BK, STAGES, WV, BMT>;
  constexpr int MI = C::MI;
  constexpr int PER = 32 / BITS;
  constexpr int SPW = C::SPW;
  constexpr uint32_t MASK = ((1u << BITS) - 1u) * 0x00010001u;
  __shared__ __attribute__((aligned(16))) int8_t smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches below
  const int wm = wid >> 1, wn = wid & 1, h = lane >> 5;
  // Blocks below tiles_m * tn_full take whole tiles of columns [0, n_split);
  // the rest take one k-half of a tile of the last tile columns (block j of
  // them: half j / tail, tile j % tail) and leave fp32 partial sums
  int tm, tn, half = -1;
  const int tiles_m = (M + BMT - 1) / BMT, tiles_n = (N + BN - 1) / BN;
  const int full = tiles_m * tn_full;
  int nk = (K + BK - 1) / BK;  // K % 64 == 0; a last half-iteration reads zeros
  int kb = 0;                  // first k-iteration
  if ((int)blockIdx.x < full) {
    tile_coords<8>(blockIdx.x, tiles_m, tn_full, tm, tn);
  } else {
    const int j = (int)blockIdx.x - full, tail = tiles_m * (tiles_n - tn_full);
    half = j / tail;
    tile_coords<8>(j - half * tail, tiles_m, tiles_n - tn_full, tm, tn);
    tn += tn_full;
    nk /= 2;  // K % 128 == 0 on this path
    kb = half * nk;
  }
  const int m_blk = tm * BMT, n_blk = tn * BN;
  const int rowb = K / PER * 4;      // bytes per packed row
  const int ng = K / G, NP = (N + 3) & ~3;
  const int lg_g = 31 - __builtin_clz(G);  // G is a power of two

  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(x16 + (int64_t)m_blk * K, min(BMT, M - m_blk) * K * 2);
  const __amdgpu_buffer_rsrc_t rsb =
      make_rsrc(reinterpret_cast<const int8_t*>(packed) + (int64_t)n_blk * rowb, min(BN, N - n_blk) * rowb);
  const __amdgpu_buffer_rsrc_t rss = make_rsrc(sbt, ng * NP * 4);

  // ---- loads of one stage: this wave's A loads, then its share of the B
  // and SB loads (other-load o goes to wave o % WV).  Per-lane offsets are
  // fixed; the k-iteration's offset goes in the scalar offset.  K % 64 == 0,
  // so no load crosses K; rows past M / N lie past their buffer and read 0.
  int a_off[C::APW];
#pragma unroll
  for (int j = 0; j < C::APW; ++j) {
    const int r = (wid * C::APW + j) * C::A_RPI + lane / C::A_CB;
    const int c = (lane % C::A_CB) ^ lds_swz<C::A_CB>(r);
    a_off[j] = r * K * 2 + c * 16;
  }
  constexpr int OMAX = (C::NO + WV - 1) / WV;
  int o_off[OMAX];  // B: byte offset in the packed rows; SB: byte offset in the table
#pragma unroll
  for (int t = 0; t < OMAX; ++t) {
    const int o = wid + WV * t;
    o_off[t] = 0;
    if (o < C::B_LOADS) {
      const int r = o * C::B_RPI + lane / C::B_CB;
      const int c = (lane % C::B_CB) ^ lds_swz<C::B_CB>(r);
      o_off[t] = r * rowb + c * 16;
    } else if (o < C::NO) {
      // sub-block u = o - B_LOADS: lanes 0-31 its first group, lanes 32-63
      // the second one when a sub-block spans two groups (else the first again)
      const int u = o - C::B_LOADS;
      const int gd = ((u * 64) >> lg_g) + (G < 64 ? lane >> 5 : 0);  // group after the iteration's first
      // a lane's 4 columns are clamped to the table's width: columns past N
      // are never stored, and every address stays inside the table
      const int c4 = min(n_blk + 4 * (lane & 31), NP - 4);
      o_off[t] = (gd * NP + c4) * 4;
    }
  }
  const int n_other = C::NO / WV + (wid < C::NO % WV ? 1 : 0);

#define QLQ_ISSUE(T, SLOT)                                                                        \
  do {                                                                                            \
    const int k0_ = (kb + (T)) * BK;                                                              \
    _Pragma("unroll") for (int j = 0; j < C::APW; ++j)                                            \
        load_lds_b128(rsa, smem + (SLOT) * C::A_TILE + (wid * C::APW + j) * 1024, a_off[j], k0_ * 2); \
    _Pragma("unroll") for (int t = 0; t < OMAX; ++t) {                                            \
      const int o_ = wid + WV * t;                                                                \
      if (t < n_other) {                                                                          \
        if (o_ < C::B_LOADS)                                                                      \
          load_lds_b128(rsb, smem + C::B_BASE + (SLOT) * C::B_TILE + o_ * 1024, o_off[t], k0_ / PER * 4); \
        else                                                                                      \
          load_lds_b128(rss, smem + C::SB_BASE + (SLOT) * C::SB_TILE + (o_ - C::B_LOADS) * 1024, o_off[t], \
                        (k0_ >> lg_g) * NP * 4);                                                  \
      }                                                                                           \
    }                                                                                             \
  } while (0)

  // ---- fragment addresses in slot 0 (slot s adds s times a tile).  This
  // wave takes every k-step s < SPW of a sub-block.
  // B: the words of those steps are contiguous: NBW words from byte boff
  constexpr int NBW = BITS == 8 ? 2 * SPW : SPW;
  constexpr int NBR = NBW == 8 ? 2 : 1;  // 16-byte B reads per fragment
  int aoff[MI][C::U][SPW];
  int boff[2][C::U][NBR];
  int soff[2][C::U];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int ra = wm * (BMT / 2) + 32 * i + (lane & 31);
#pragma unroll
    for (int u = 0; u < C::U; ++u)
#pragma unroll
      for (int sl = 0; sl < SPW; ++sl) {
        const int st = sl;
        const int c = 8 * u + 4 * h + st;
        aoff[i][u][sl] = ra * C::A_ROW + (c ^ lds_swz<C::A_CB>(ra)) * 16;
      }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rb = wn * 64 + 32 * i + (lane & 31);
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      // first word of this wave's steps within the row's sub-block
      const int w0 = BITS == 4 ? 4 * h : 8 * h;
      const int cb = (C::RB / C::U / 16) * u + w0 / 4;  // chunk (4 words per chunk)
#pragma unroll
      for (int q = 0; q < NBR; ++q)
        boff[i][u][q] = C::B_BASE + rb * C::RB + ((cb + q) ^ lds_swz<C::B_CB>(rb)) * 16 + (w0 % 4) * 4;
      const int gi = G < 64 ? h : 0;
      soff[i][u] = C::SB_BASE + u * 1024 + gi * 512 + rb * 4;
    }
  }

  f32x16_v acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_v{};

#define QLQ_COMPUTE(SLOT)                                                                          \
  do {                                                                                             \
    const int8_t* sa_ = smem + (SLOT) * C::A_TILE;                                                 \
    const int8_t* sb_ = smem + (SLOT) * C::B_TILE;                                                 \
    const int8_t* ss_ = smem + (SLOT) * C::SB_TILE;                                                \
    _Pragma("unroll") for (int u = 0; u < C::U; ++u) {                                             \
      u32x4_v af[MI][SPW];                                                                         \
      _Pragma("unroll") for (int i = 0; i < MI; ++i)                                               \
          _Pragma("unroll") for (int sl = 0; sl < SPW; ++sl)                                       \
              af[i][sl] = *reinterpret_cast<const u32x4_v*>(sa_ + aoff[i][u][sl]);                 \
      u32x4_v bq[2][SPW]; /* [j][sl]: dequantized B operands */                                    \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                              \
        const uint32_t ee = *reinterpret_cast<const uint32_t*>(ss_ + soff[j][u]);                 \
        uint32_t w[NBW];                                                                           \
        if constexpr (NBW == 2) {                                                                  \
          const uint2 v = *reinterpret_cast<const uint2*>(sb_ + boff[j][u][0]);                    \
          w[0] = v.x; w[1] = v.y;                                                                  \
        } else {                                                                                   \
          _Pragma("unroll") for (int q = 0; q < NBR; ++q) {                                        \
            const u32x4_v v = *reinterpret_cast<const u32x4_v*>(sb_ + boff[j][u][q]);              \
            w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];       \
          }                                                                                        \
        }                                                                                          \
        const f16x2_v e2 = __builtin_bit_cast(f16x2_v, ee); /* halves: s', b' */                   \
        const f16x2_v s2 = __builtin_shufflevector(e2, e2, 0, 0);                                  \
        const f16x2_v b2 = __builtin_shufflevector(e2, e2, 1, 1);                                  \
        /* 4-bit: odd nibbles are masked where they sit (16 q 2^-24, still */                       \
        /* subnormal) and take s' 2^-4: the same product unless s' < 2^-10, */                      \
        /* i.e. unless a group's scale is 2^24 below its column's largest */                        \
        const f16x2_v s2h = s2 * (f16x2_v){(f16_t)0.0625f, (f16_t)0.0625f};                        \
        _Pragma("unroll") for (int sl = 0; sl < SPW; ++sl) {                                       \
          _Pragma("unroll") for (int p = 0; p < 4; ++p) {                                          \
            uint32_t qd;                                                                           \
            if constexpr (BITS == 4) qd = (p < 2 ? w[sl] : w[sl] >> 8) & (p & 1 ? MASK << 4 : MASK); \
            else qd = (w[2 * sl + (p >> 1)] >> (8 * (p & 1))) & MASK;                              \
            bq[j][sl][p] = __builtin_bit_cast(                                                     \
                uint32_t, __builtin_elementwise_fma(BITS == 4 && (p & 1) ? s2h : s2,               \
                                                    __builtin_bit_cast(f16x2_v, qd), b2));         \
          }                                                                                        \
        }                                                                                          \
      }                                                                                            \
      _Pragma("unroll") for (int sl = 0; sl < SPW; ++sl)                                           \
          _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
              _Pragma("unroll") for (int j = 0; j < 2; ++j)                                        \
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(                              \
                      __builtin_bit_cast(f16x8_v, af[i][sl]), __builtin_bit_cast(f16x8_v, bq[j][sl]), \
                      acc[i][j], 0, 0, 0);                                                         \
    }                                                                                              \
  } while (0)

  // Double buffer, one barrier per k-iteration: wait for this wave's loads
  // of tile it (the only ones in flight), barrier (everyone's have landed and
  // everyone is done with the other slot), issue tile it+1 into the other
  // slot, compute tile it.  Unrolled by the two slots so that every LDS
  // address above is a constant offset from a fixed register.
  QLQ_ISSUE(0, 0);
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    wait_loads_and_barrier<0>();
    QLQ_ISSUE(it + 1, 1);
    QLQ_COMPUTE(0);
    wait_loads_and_barrier<0>();
    if (it + 2 < nk) QLQ_ISSUE(it + 2, 0);
    QLQ_COMPUTE(1);
  }
  if (it < nk) {  // odd nk: slot 0 holds the last tile
    wait_loads_and_barrier<0>();
    QLQ_COMPUTE(0);
  }
#undef QLQ_ISSUE
#undef QLQ_COMPUTE

  if (half >= 0) {
    // ---- a k-half of a tail tile: its fp32 sums as they stand (no scaling);
    // each store instruction writes two rows of 32 consecutive columns
    float* P = part + (int64_t)half * M * (N - n_split);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m_blk + wm * (BMT / 2) + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int n = n_blk + wn * 64 + 32 * j + (lane & 31);
          if (m < M && n < N) P[(int64_t)m * (N - n_split) + (n - n_split)] = acc[i][j][e];
        }
    return;
  }

  // ---- epilogue: y = 2^(e_m + f_n) * acc + bias, one rounding; each wave
  // stages its rows 64 at a time in its own LDS area and stores them whole
  int fcol[2];
  float bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = min(n_blk + wn * 64 + 32 * j + (lane & 31), N - 1);
    fcol[j] = wexp[n];
    bcol[j] = bias ? Elem<XT>::load(bias, n) : 0.0f;
  }
  static_assert(4 * kTileStageBytes <= C::LDS, "staging fits");
  __syncthreads();  // every wave is done with the ring
  int8_t* stage = smem + wid * kTileStageBytes;
  const int col0 = n_blk + wn * 64;
#pragma unroll
  for (int hf = 0; hf < MI / 2; ++hf) {
    const int row0 = m_blk + wm * (BMT / 2) + 64 * hf;
    float v[2][2][16];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = row0 + 32 * i2 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int em = m < M ? xexp[m] : 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float t = ldexpf(acc[2 * hf + i2][j][e], em + fcol[j]);
          if (bias) t = t + bcol[j];
          v[i2][j][e] = t;
        }
      }
    store_tile64_16<XT>(v, y, N, row0, col0, M - row0, N - col0, stage, lane);
  }
}

// The tail tiles' two k-halves joined: y[m, n] = 2^(e_m + f_n) * (P0 + P1)
// (+ bias), one rounding, for n in [n_split, N) -- the GEMM epilogue's
// arithmetic on the sum of the halves.  Four consecutive outputs per thread.
template <typename XT>
__global__ void __launch_bounds__(256)
gemm_tail_join_kernel(const float* __restrict__ part, int M, int N, int n_split, const int* __restrict__ xexp,
                      const int* __restrict__ wexp, const XT* __restrict__ bias, XT* __restrict__ y) {
  const int W = N - n_split;
  const int64_t MW = (int64_t)M * W;
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t i = i0 + u;
    if (i >= MW) return;
    const int m = (int)(i / W), n = n_split + (int)(i - (int64_t)m * W);
    float t = ldexpf(part[i] + part[MW + i], xexp[m] + wexp[n]);
    if (bias) t = t + Elem<XT>::load(bias, n);
    Elem<XT>::store(y, (int64_t)m * N + n, t);
  }
}

// Tail split of the tall 4-bit GEMM: 2 * 256 tiles run at once (two blocks
// per CU), and a tile alone on a CU finishes in about 0.4 of the time a pair
// sharing it takes.  When the tiles past the last whole paired round are
// whole tile columns and their k-halves fit one per CU (at most 128 tiles),
// the halves run as separate blocks and a join kernel adds them; with more
// tail tiles the halves would share CUs and take longer than the whole tiles.
struct TailPlan {
  int tn_full, n_split;
  bool split;
  TailPlan(int64_t M, int64_t K, int64_t N, int G, int bits) {
    const int64_t tiles_m = cdiv(M, gemm::TILE_M_TALL), tiles_n = cdiv(N, gemm::BN);
    const int64_t T = tiles_m * tiles_n, S = 2 * 256;
    const int64_t r = T % S;
    split = bits == 4 && T >= S && r > 0 && 2 * r <= 256 && r % tiles_m == 0 && K % 128 == 0 && (K / 2) % G == 0;
    tn_full = (int)(split ? tiles_n - r / tiles_m : tiles_n);
    n_split = split ? tn_full * gemm::BN : (int)N;
  }
};

// Workspace: x16 [M, K] fp16 | e_m [M] | f_n [N] | (s', b') [K/G, NP] |
// with a tail split, the two k-halves' partial sums fp32 [2][M][N - n_split];
// each part 256-byte aligned.
struct GemmWs {
  size_t x16, xe, we, sb, pt, total;
  GemmWs(int64_t M, int64_t K, int64_t N, int G, int bits) {
    const auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const TailPlan tp(M, K, N, G, bits);
    x16 = 0;
    xe = al((size_t)M * (size_t)K * 2);
    we = xe + al((size_t)M * 4);
    sb = we + al((size_t)N * 4);
    pt = sb + al((size_t)(K / G) * (size_t)((N + 3) & ~3) * 4);
    total = pt + (tp.split ? (size_t)2 * (size_t)M * (size_t)(N - tp.n_split) * 4 : 0);
  }
};

size_t affine_gemm_workspace(int64_t M, int64_t K, int64_t N, int G, int bits) {
  return GemmWs(M, K, N, G, bits).total;
}

template <int BITS, typename XT>
static hipError_t gemm_launch(const void* x, int64_t M, int64_t K, const uint32_t* packed,
                              const void* scales, const void* biases, int64_t N, int G,
                              const void* bias, void* y, void* ws, hipStream_t s) {
  const GemmWs L(M, K, N, G, BITS);
  f16_t* x16 = (f16_t*)((char*)ws + L.x16);
  int* xexp = (int*)((char*)ws + L.xe);
  int* wexp = (int*)((char*)ws + L.we);
  uint32_t* sbt = (uint32_t*)((char*)ws + L.sb);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (K <= 64 * 64) {
    constexpr int RPW = QLQ_PREP_ROWS_PER_WAVE;
    const unsigned blocks = (unsigned)(cdiv(M, 4 * RPW) + cdiv(N, 64));
#define QLQ_PREP(EPT_)                                                                                  \
  hipLaunchKernelGGL((gemm_prep_wave_kernel<BITS, XT, EPT_, RPW>), dim3(blocks), dim3(256), 0, s, (const XT*)x, \
                     m, k, (const XT*)scales, (const XT*)biases, n, G, x16, xexp, wexp, sbt)
    if (K <= 64 * 16) QLQ_PREP(16);
    else if (K <= 64 * 32) QLQ_PREP(32);
    else QLQ_PREP(64);
#undef QLQ_PREP
  } else {
    hipLaunchKernelGGL((gemm_prep_kernel<BITS, XT>), dim3((unsigned)(M + cdiv(N, 64))), dim3(256), 0, s,
                       (const XT*)x, m, k, (const XT*)scales, (const XT*)biases, n, G, x16, xexp, wexp, sbt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 4-bit codes only: an 8-bit 256-row stage does not fit twice in a compute
  // unit's LDS
  const int64_t tall_tiles = cdiv(M, gemm::TILE_M_TALL) * cdiv(N, gemm::BN);
  const bool tall = BITS == 4 && tall_tiles >= 2 * 256;
  const int64_t tiles = tall ? tall_tiles : cdiv(M, gemm::TILE_M) * cdiv(N, gemm::BN);
  const TailPlan tp(M, K, N, G, BITS);  // splits only tall tiles
  float* part = (float*)((char*)ws + L.pt);
  const int64_t tail = tp.split ? cdiv(M, gemm::TILE_M_TALL) * (cdiv(N, gemm::BN) - tp.tn_full) : 0;
  auto kern = affine_gemm_kernel<BITS, XT, gemm::KB, gemm::NSTAGES, gemm::WAVES, gemm::TILE_M>;
  if constexpr (BITS == 4)
    if (tall) kern = affine_gemm_kernel<BITS, XT, gemm::KB, gemm::NSTAGES, gemm::WAVES, gemm::TILE_M_TALL>;
  const int tn_full = tp.split ? tp.tn_full : (int)cdiv(N, gemm::BN);
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles + tail)), dim3(64 * gemm::WAVES), 0, s, (const f16_t*)x16,
                     (const int*)xexp, m, k, packed, (const uint32_t*)sbt, (const int*)wexp, n, G,
                     (const XT*)bias, (XT*)y, tn_full, part, tp.n_split);
  if (tp.split) {
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t outs = M * (N - tp.n_split);
    hipLaunchKernelGGL(gemm_tail_join_kernel<XT>, dim3((unsigned)cdiv(outs, 1024)), dim3(256), 0, s,
                       (const float*)part, m, n, tp.n_split, (const int*)xexp, (const int*)wexp,
                       (const XT*)bias, (XT*)y);
  }
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
  // 4- or 8-bit packed codes (the caller transcodes the other widths)
  if (bits == 4) return gemm_dispatch_x<4>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, workspace, s);
  if (bits == 8) return gemm_dispatch_x<8>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, workspace, s);
  return hipErrorInvalidValue;
}

}  // namespace qlq
