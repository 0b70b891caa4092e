// Skinny (decode-shaped) affine forward: y = x . dequant(W)^T (+ bias) for
// small M, computed straight from the packed codes.
//
// "Struct QuantizedLinear" (nuvec-nn docs), forward: x W^T + b from the packed
// weight, scales and biases; dequantization w = scale*q + bias (MLX affine
// docstring of pergroup_linear, "cider/ops.py").  The split of M == 1 onto a
// matrix-vector kernel with on-the-fly dequantization follows the dispatch
// described in the same docstring.
//
// Design (HBM-bound; every weight byte is read exactly once):
//  * one wave owns R consecutive output rows; its 64 lanes stride over the
//    row in 16-byte chunks (lane + 64*i), so each load instruction of a wave
//    covers 1 KiB of contiguous codes.  At M == 1 a wave takes one row in
//    blocks of 16 waves, and with 4-bit codes and N >= QLQ_GEMV_LARGE_N two
//    rows in blocks of 8 (more bytes in flight per wave, half the block
//    turnover);
//  * a chunk never straddles a group (group_size is a multiple of the chunk's
//    code count), so per chunk and row:  acc += s * P + b * X  with
//    P = sum x*q and X = sum x;  X is shared by the R rows;
//  * 16-bit x (bf16/f16) and 2/4-bit codes: a code pair sharing one uint32 at
//    a distance of 16 bits becomes one packed 16-bit float pair with a single
//    and-or:  (w >> bits*j) & mask | MAGIC  gives (OFF + q_j, OFF + q_j')
//    exactly (OFF = 128 for bf16, 1024 for f16), and one v_dot2 multiplies it
//    against the matching x pair, which is built once per chunk by a byte
//    permute.  The OFF offset folds into the group term:
//    s*(P' - OFF*X) + b*X = s*P' + (b - OFF*s)*X;
//  * the K-split partial sums are reduced across the wave with DPP/permute
//    shuffles, and one rounding to the output dtype happens at the end.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

#ifndef QLQ_GEMV_WAVES_PER_BLOCK
#define QLQ_GEMV_WAVES_PER_BLOCK 16
#endif
#ifndef QLQ_GEMV_R1
#define QLQ_GEMV_R1 1  // output rows per wave at M == 1
#endif
#ifndef QLQ_GEMV_R2
#define QLQ_GEMV_R2 4  // output rows per wave at M == 2
#endif
#ifndef QLQ_GEMV_LARGE_N
#define QLQ_GEMV_LARGE_N 12288  // M == 1, 4-bit codes: from this N on, 2 rows per wave, 8 waves per block
#endif

namespace qlq {

constexpr int64_t kGemvLargeN = QLQ_GEMV_LARGE_N;

template <typename XT> struct PairTraits;
template <> struct PairTraits<bf16_t> {
  static constexpr uint32_t MAGIC = 0x43004300u;  // bf16 (128, 128)
  static constexpr uint32_t ONES = 0x3F803F80u;   // bf16 (1, 1)
  static constexpr float OFF = 128.0f;
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                           __builtin_bit_cast(bf16x2_v, b), c, false);
  }
};
template <> struct PairTraits<f16_t> {
  static constexpr uint32_t MAGIC = 0x64006400u;  // f16 (1024, 1024)
  static constexpr uint32_t ONES = 0x3C003C00u;   // f16 (1, 1)
  static constexpr float OFF = 1024.0f;
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_v, a), __builtin_bit_cast(f16x2_v, b), c,
                                  false);
  }
};

// Codes per chunk: one unit of 32 codes (BITS words) for 1- to 6-bit codes,
// 16 for 8-bit (4 words).
template <int BITS> struct Chunk {
  static constexpr int CODES = BITS == 8 ? 16 : 32;
  static constexpr int WORDS = CODES * BITS / 32;  // BITS, or 4 at 8 bits
};

template <int WORDS> struct WordsT { uint32_t w[WORDS]; };

// a chunk's words; 16- and 8-byte chunks are one load (their offsets are
// multiples of their size), 3-, 5- and 6-word chunks are dword loads.  Every
// code word is read once per launch: streaming loads.
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_v;
template <int WORDS>
__device__ __forceinline__ WordsT<WORDS> load_words(const uint32_t* p) {
  WordsT<WORDS> r;
  if constexpr (WORDS == 4) {
    const u32x4_v v = stream_load(reinterpret_cast<const u32x4_v*>(p));
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
  } else if constexpr (WORDS == 2) {
    const u32x2_v v = stream_load(reinterpret_cast<const u32x2_v*>(p));
    r.w[0] = v[0]; r.w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < WORDS; ++i) r.w[i] = stream_load(p + i);
  }
  return r;
}
// the same through a buffer descriptor of one row (offset in bytes, 32-bit)
template <int WORDS>
__device__ __forceinline__ WordsT<WORDS> load_words(__amdgpu_buffer_rsrc_t rw, int off) {
  WordsT<WORDS> r;
  if constexpr (WORDS == 4) {
    const u32x4_v v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, kStreamAux);
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
  } else if constexpr (WORDS == 2) {
    const u32x2_v v = __builtin_amdgcn_raw_buffer_load_b64(rw, off, 0, kStreamAux);
    r.w[0] = v[0]; r.w[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < WORDS; ++i) r.w[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, off + 4 * i, 0, kStreamAux);
  }
  return r;
}

// ---------------------------------------------------------------------------
// Fast path: 16-bit x, 2- or 4-bit codes.
// ---------------------------------------------------------------------------
template <int BITS, typename XT, int MT, int R>
__global__ void __launch_bounds__(64 * QLQ_GEMV_WAVES_PER_BLOCK)
gemv_pair_kernel(const XT* __restrict__ x, int64_t M, int64_t K, const uint32_t* __restrict__ packed,
                 const XT* __restrict__ scales, const XT* __restrict__ biases, int64_t N, int G,
                 const XT* __restrict__ bias, XT* __restrict__ y) {
  using PT = PairTraits<XT>;
  constexpr int CODES = Chunk<BITS>::CODES;   // 32
  constexpr int WORDS = Chunk<BITS>::WORDS;   // 2 (2-bit) or 4 (4-bit)
  constexpr int PER = 32 / BITS;              // codes per word: 16 or 8
  constexpr int XDW = CODES / 2;              // x dwords per chunk: 16
  constexpr uint32_t MASK = ((1u << BITS) - 1u) * 0x00010001u;

  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * QLQ_GEMV_WAVES_PER_BLOCK + (threadIdx.x >> 6);
  const int64_t n0 = wave * R;
  if (n0 >= N) return;
  const int64_t m0 = (int64_t)blockIdx.y * MT;
  const int64_t cpr = K / CODES;              // chunks per row
  const int64_t wpr = K / PER;                // words per row
  const int64_t gpr = K / G;                  // groups per row

  float acc[MT][R];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int64_t c = lane; c < cpr; c += kWave) {
    // ---- issue every load of this chunk first: codes, group params, x
    WordsT<WORDS> wv[R];
    float s[R], b[R];
    const int64_t g = c * CODES / G;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t n = (n0 + r < N) ? n0 + r : N - 1;  // clamp: rows past N are computed, not stored
      wv[r] = load_words<WORDS>(packed + n * wpr + c * WORDS);
      s[r] = stream_elem<XT>(scales, n * gpr + g);
      b[r] = stream_elem<XT>(biases, n * gpr + g);
    }
    uint32_t xd[MT][XDW];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int64_t mm = (m0 + m < M) ? m0 + m : M - 1;
      const uint4* xp = reinterpret_cast<const uint4*>(x + mm * K + c * CODES);
#pragma unroll
      for (int i = 0; i < XDW / 4; ++i) {
        uint4 v = xp[i];
        xd[m][4 * i] = v.x; xd[m][4 * i + 1] = v.y; xd[m][4 * i + 2] = v.z; xd[m][4 * i + 3] = v.w;
      }
    }
    // ---- x pairs matching the code pairs, and X = sum of the chunk's x
    // word t of the chunk covers x dwords [t*PER/2, (t+1)*PER/2); its pair j
    // is (x_j, x_{j+PER/2}) relative to the word's first element.
    float X[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float xs = 0.0f;
#pragma unroll
      for (int i = 0; i < XDW; ++i) xs = PT::dot2(xd[m][i], PT::ONES, xs);
      X[m] = xs;
      uint32_t xp[XDW];
#pragma unroll
      for (int t = 0; t < WORDS; ++t) {
        constexpr int HALF = PER / 4;  // dwords in half a word's x span
#pragma unroll
        for (int j = 0; j < PER / 2; ++j) {
          const uint32_t lo = xd[m][t * (PER / 2) + j / 2];
          const uint32_t hi = xd[m][t * (PER / 2) + HALF + j / 2];
          xp[t * (PER / 2) + j] = __builtin_amdgcn_perm(hi, lo, (j & 1) ? 0x07060302u : 0x05040100u);
        }
      }
#pragma unroll
      for (int i = 0; i < XDW; ++i) xd[m][i] = xp[i];
    }
    // ---- per row: decode pairs, dot, apply the group's affine parameters
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float cb = __fmaf_rn(-PT::OFF, s[r], b[r]);  // b - OFF*s
      float P[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) P[m] = 0.0f;
#pragma unroll
      for (int t = 0; t < WORDS; ++t) {
        const uint32_t w = wv[r].w[t];
#pragma unroll
        for (int j = 0; j < PER / 2; ++j) {
          const uint32_t qp = ((w >> (BITS * j)) & MASK) | PT::MAGIC;
#pragma unroll
          for (int m = 0; m < MT; ++m) P[m] = PT::dot2(xd[m][t * (PER / 2) + j], qp, P[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][r] = __fmaf_rn(s[r], P[m], __fmaf_rn(cb, X[m], acc[m][r]));
    }
  }

  // ---- reduce across the wave and store
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_sum_dpp(acc[m][r]);
  if (lane < MT * R) {
    float v = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == m * R + r) v = acc[m][r];
    const int m = lane / R, r = lane % R;
    const int64_t n = n0 + r, mm = m0 + m;
    if (n < N && mm < M) {
      if (bias) v = v + Elem<XT>::load(bias, n);
      Elem<XT>::store(y, mm * N + n, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Latency-bound fast path (16-bit x, codes of 1-6 bits, M <= 2, K <= 64*NCH*32).
//  * x is staged once per block in LDS (one 16-byte load per thread per
//    2048 bytes of x), so the wave's vector-memory instructions are almost
//    all weight loads;
//  * lane l owns NCH consecutive chunks [l*NCH, l*NCH + NCH), i.e. whole
//    groups when G >= 32*NCH, so a row needs one scale and one bias load per
//    group the lane touches (group size is a template parameter);
//  * the x loads are issued first, then every code / scale / bias load of the
//    wave (codes through one buffer descriptor per row, all of them with the
//    non-temporal policy: each byte is read once), then x goes to LDS: one
//    memory round trip per wave;
//  * after the barrier the lane reads all its x chunks out of LDS before
//    anything waits for the weights, and the chunk loop has no branch;
//  * 1-, 3-, 5- and 6-bit codes: code j and code j + 16 of the chunk's 32 are
//    taken out of its BITS-word stream at compile-time offsets and joined
//    into one 16-bit pair, against the x pair (x_j, x_j+16), which the block
//    forms once while staging x (at 3, 5 and 6 bits no two codes sit 16 bits
//    apart in one word).
// ---------------------------------------------------------------------------
template <int BITS> constexpr bool kStreamPairs = BITS == 1 || BITS == 3 || BITS == 5 || BITS == 6;

// Pair j = (code j, code j + 16) of a 3-bit unit as two 16-bit lanes.  The
// two codes lie 48 stream bits apart, so in the words s0, s1, s2 whose halves
// hold stream bits [16 t, 16 t + 16) and [16 t + 48, 16 t + 64) (byte
// permutes of the unit's words) both sit at offset 3j mod 16 of their half:
// one shift and one mask (mask2 = 0x00070007, held in a register) take the
// pair out.  Pairs 5 and 10 cross a half and take the per-code extraction.
__device__ __forceinline__ uint32_t unit3_pair(const uint32_t* w, int j, uint32_t mask2) {
  const int p = 3 * j, t = p >> 4, off = p & 15;
  if (off + 3 > 16) return unit_code<3>(w, j) | (unit_code<3>(w, j + 16) << 16);
  const uint32_t sw = t == 0   ? __builtin_amdgcn_perm(w[1], w[0], 0x07060100u)   // w0 lo | w1 hi
                      : t == 1 ? __builtin_amdgcn_perm(w[2], w[0], 0x05040302u)   // w0 hi | w2 lo
                               : __builtin_amdgcn_perm(w[2], w[1], 0x07060100u);  // w1 lo | w2 hi
  return (sw >> off) & mask2;
}

template <int BITS, typename XT, int MT, int R, int NCH, int G, int WPB>
__global__ void __launch_bounds__(64 * WPB)
gemv_flat_kernel(const XT* __restrict__ x, int64_t M, int64_t K, const uint32_t* __restrict__ packed,
                 const XT* __restrict__ scales, const XT* __restrict__ biases, int64_t N,
                 const XT* __restrict__ bias, XT* __restrict__ y) {
  using PT = PairTraits<XT>;
  constexpr int CODES = Chunk<BITS>::CODES;          // 32 codes per chunk
  constexpr int WORDS = Chunk<BITS>::WORDS;
  constexpr int PER = kStreamPairs<BITS> ? 1 : 32 / BITS;  // codes per word (2, 4 bits)
  constexpr int XDW = CODES / 2;                     // x dwords per chunk (16)
  constexpr int CPG = G / CODES;                     // chunks per group (1, 2, 4)
  // a lane's chunks c = lane + 64 i lie 64 chunks apart, each in its own group
  constexpr int NG = NCH;
  constexpr int THREADS = 64 * WPB;
  constexpr int XROW = 64 * NCH * 4;                 // 16-byte x units per (padded) row
  constexpr int XU4 = (MT * XROW + THREADS - 1) / THREADS;  // x units staged per thread
  constexpr uint32_t MASK = ((1u << BITS) - 1u) * 0x00010001u;
  static_assert(XDW == 16, "four 16-byte x units per chunk");

  // x in code-pair order, laid out [unit q][chunk-in-lane i][lane l] so that
  // 8 consecutive lanes read 8 consecutive 16-byte units (no bank conflicts),
  // and the per-unit partial sums of x in the same order.
  __shared__ __attribute__((aligned(16))) uint4 xs[MT][XROW];
  __shared__ float xsum[MT][XROW];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n0 = wave * R;
  const int m0 = blockIdx.y * MT;
  const int cpr = (int)(K / CODES);
  const int wpr = (int)(K * BITS / 32);
  const int gpr = (int)(K / G);
  const int kx = (int)(K / 8);  // x units per row

  // ---- 1. x loads first (they gate the LDS staging).  Code streams pair x_j
  // with x_j+16 of each 32-value chunk, so staged unit o = 2q + h of a chunk
  // takes halves h of the chunk's units q and q + 2 (xr and xr2).
  constexpr bool PAIRS16 = kStreamPairs<BITS>;
  uint4 xr[XU4], xr2[PAIRS16 ? XU4 : 1];
#pragma unroll
  for (int i = 0; i < XU4; ++i) {
    const int idx = tid + THREADS * i, m = idx / XROW, u = idx % XROW;
    const int mm = (m0 + m < M) ? m0 + m : (int)M - 1;
    const uint4* xrow = reinterpret_cast<const uint4*>(x + (int64_t)mm * K);
    const bool in = m < MT && u < kx;
    if constexpr (PAIRS16) {
      const int ua = (u & ~3) + ((u & 3) >> 1);  // unit q of the chunk; q + 2 is two units on
      xr[i] = in ? xrow[ua] : make_uint4(0, 0, 0, 0);
      xr2[i] = in ? xrow[ua + 2] : make_uint4(0, 0, 0, 0);
    } else {
      xr[i] = in ? xrow[u] : make_uint4(0, 0, 0, 0);
    }
  }
  // ---- 2. every weight load of this wave, chunk by chunk
  WordsT<WORDS> wv[NCH][R];
  uint16_t sr[NG][R], br[NG][R];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int c = i * 64 + lane;  // a load instruction covers 64 consecutive chunks
    c = c < cpr ? c : cpr - 1;  // lanes past the row re-read the last chunk and drop it
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = (n0 + r < N) ? n0 + r : (int)N - 1;
      // rows are wave-uniform: one descriptor per row, the lane's chunk in the offset
      wv[i][r] = load_words<WORDS>(make_rsrc(packed + (int64_t)n * wpr, wpr * 4), c * WORDS * 4);
      const int g = c / CPG;
      sr[i][r] = stream_load(reinterpret_cast<const uint16_t*>(scales) + (int64_t)n * gpr + g);
      br[i][r] = stream_load(reinterpret_cast<const uint16_t*>(biases) + (int64_t)n * gpr + g);
    }
  }
  // ---- 3. stage x: pair order within each word's span, partial sums
#pragma unroll
  for (int i = 0; i < XU4; ++i) {
    const int idx = tid + THREADS * i, m = idx / XROW, u = idx % XROW;
    if (m < MT) {
      const uint4 v = xr[i];
      uint4 p;
      if constexpr (BITS == 4) {  // one unit = one word's 8 x: pairs (j, j+4)
        p.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
        p.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
        p.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
        p.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
      } else if constexpr (PAIRS16) {  // pairs (x_j, x_j+16): half h of units q and q + 2
        const uint4 v2 = xr2[i];
        const bool hi = (u & 1) != 0;
        const uint32_t a0 = hi ? v.z : v.x, a1 = hi ? v.w : v.y;
        const uint32_t b0 = hi ? v2.z : v2.x, b1 = hi ? v2.w : v2.y;
        p.x = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
        p.y = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
        p.z = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
        p.w = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
      } else {  // 2-bit codes: pairs (j, j+8) span units; permuted after the LDS read
        p = v;
      }
      // the staged unit's 8 values (any split of a chunk's 32 works for X)
      const float ps = PT::dot2(p.w, PT::ONES, PT::dot2(p.z, PT::ONES, PT::dot2(p.y, PT::ONES, PT::dot2(p.x, PT::ONES, 0.0f))));
      const int c = u >> 2, q = u & 3;
      const int pos = q * (64 * NCH) + c;  // chunk c = lane + 64 i
      xs[m][pos] = p;
      xsum[m][pos] = ps;
    }
  }
  __syncthreads();
  if (n0 >= N) return;

  float acc[MT][R];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  // every x chunk of this lane out of LDS first, before anything waits for
  // the weights, so the LDS latency overlaps the HBM latency; no branch, so
  // all of these reads can be issued at once (lanes past the row compute on
  // the re-read last chunk and drop the result below)
  float X[NCH][MT];
  uint32_t xp[NCH][MT][XDW];
  uint4 xu[NCH][MT][4];
  float xf[NCH][MT][4];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pos = q * (64 * NCH) + i * 64 + lane;
        xu[i][m][q] = xs[m][pos];
        xf[i][m][q] = xsum[m][pos];
      }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      uint32_t xd[XDW];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xu[i][m][q];
        xd[4 * q] = v.x; xd[4 * q + 1] = v.y; xd[4 * q + 2] = v.z; xd[4 * q + 3] = v.w;
      }
      X[i][m] = ((xf[i][m][0] + xf[i][m][1]) + xf[i][m][2]) + xf[i][m][3];
      if constexpr (BITS == 4) {
#pragma unroll
        for (int q = 0; q < XDW; ++q) xp[i][m][q] = xd[q];
      } else if constexpr (PAIRS16) {  // staged as pairs (j, j+16) already
#pragma unroll
        for (int q = 0; q < XDW; ++q) xp[i][m][q] = xd[q];
      } else {  // 2-bit word t covers 8 x dwords: pairs (j, j+8)
#pragma unroll
        for (int t = 0; t < WORDS; ++t)
#pragma unroll
          for (int j = 0; j < PER / 2; ++j)
            xp[i][m][t * (PER / 2) + j] = __builtin_amdgcn_perm(xd[t * (PER / 2) + PER / 4 + j / 2],
                                                                xd[t * (PER / 2) + j / 2],
                                                                (j & 1) ? 0x07060302u : 0x05040100u);
      }
    }
  }

  // the code mask held in a vector register the compiler cannot fold, so that
  // mask-and-or with the exponent pattern is one v_and_or_b32 per pair (a
  // VALU instruction reads at most one literal or scalar operand here)
  uint32_t maskv;
  asm("" : "=v"(maskv) : "0"(MASK));
  constexpr uint32_t magic = PT::MAGIC;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const bool live = i * 64 + lane < cpr;
    const int gi = i;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = bits16_to_f32<XT>(sr[gi][r]), b = bits16_to_f32<XT>(br[gi][r]);
      const float cb = __fmaf_rn(-PT::OFF, s, b);  // b - OFF*s
      float P[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) P[m] = 0.0f;
      if constexpr (kStreamPairs<BITS>) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          uint32_t qp;
          if constexpr (BITS == 3) qp = unit3_pair(wv[i][r].w, j, maskv) | magic;
          else qp = unit_code<BITS>(wv[i][r].w, j) | (unit_code<BITS>(wv[i][r].w, j + 16) << 16) | magic;
#pragma unroll
          for (int m = 0; m < MT; ++m) P[m] = PT::dot2(xp[i][m][j], qp, P[m]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < WORDS; ++t) {
          const uint32_t w = wv[i][r].w[t];
#pragma unroll
          for (int j = 0; j < PER / 2; ++j) {
            const uint32_t qp = ((w >> (BITS * j)) & maskv) | magic;
#pragma unroll
            for (int m = 0; m < MT; ++m) P[m] = PT::dot2(xp[i][m][t * (PER / 2) + j], qp, P[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float a = __fmaf_rn(s, P[m], __fmaf_rn(cb, X[i][m], acc[m][r]));
        acc[m][r] = live ? a : acc[m][r];
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_sum_dpp(acc[m][r]);
  if (lane < MT * R) {
    float v = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == m * R + r) v = acc[m][r];
    const int m = lane / R, r = lane % R;
    const int n = n0 + r, mm = m0 + m;
    if (n < N && mm < M) {
      if (bias) v = v + Elem<XT>::load(bias, n);
      Elem<XT>::store(y, (int64_t)mm * N + n, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Generic path: any x dtype and bit width; code -> fp32, fp32 FMA.  Codes
// come out of the chunk's bit stream at compile-time offsets.
// ---------------------------------------------------------------------------
template <int BITS, typename XT, int MT, int R>
__global__ void __launch_bounds__(64 * QLQ_GEMV_WAVES_PER_BLOCK)
gemv_generic_kernel(const XT* __restrict__ x, int64_t M, int64_t K, const uint32_t* __restrict__ packed,
                    const XT* __restrict__ scales, const XT* __restrict__ biases, int64_t N, int G,
                    const XT* __restrict__ bias, XT* __restrict__ y) {
  constexpr int CODES = Chunk<BITS>::CODES;
  constexpr int WORDS = Chunk<BITS>::WORDS;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * QLQ_GEMV_WAVES_PER_BLOCK + (threadIdx.x >> 6);
  const int64_t n0 = wave * R;
  if (n0 >= N) return;
  const int64_t m0 = (int64_t)blockIdx.y * MT;
  const int64_t cpr = K / CODES, wpr = K * BITS / 32, gpr = K / G;

  float acc[MT][R];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int64_t c = lane; c < cpr; c += kWave) {
    WordsT<WORDS> wv[R];
    float s[R], b[R];
    const int64_t g = c * CODES / G;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t n = (n0 + r < N) ? n0 + r : N - 1;
      wv[r] = load_words<WORDS>(packed + n * wpr + c * WORDS);
      s[r] = stream_elem<XT>(scales, n * gpr + g);
      b[r] = stream_elem<XT>(biases, n * gpr + g);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int64_t mm = (m0 + m < M) ? m0 + m : M - 1;
      const XT* xr = x + mm * K + c * CODES;
      float xv[CODES];
      float X = 0.0f;
#pragma unroll
      for (int i = 0; i < CODES; ++i) {
        xv[i] = Elem<XT>::load(xr, i);
        X += xv[i];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float P = 0.0f;
#pragma unroll
        for (int i = 0; i < CODES; ++i) P = __fmaf_rn(xv[i], (float)unit_code<BITS>(wv[r].w, i), P);
        acc[m][r] = __fmaf_rn(s[r], P, __fmaf_rn(b[r], X, acc[m][r]));
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_sum_dpp(acc[m][r]);
  if (lane < MT * R) {
    float v = 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (lane == m * R + r) v = acc[m][r];
    const int m = lane / R, r = lane % R;
    const int64_t n = n0 + r, mm = m0 + m;
    if (n < N && mm < M) {
      if (bias) v = v + Elem<XT>::load(bias, n);
      Elem<XT>::store(y, mm * N + n, v);
    }
  }
}

// ---------------------------------------------------------------------------
// FWPB: waves per block of the flat kernel (the other kernels use
// QLQ_GEMV_WAVES_PER_BLOCK)
template <int BITS, typename XT, int MT, int R, int FWPB = QLQ_GEMV_WAVES_PER_BLOCK>
static hipError_t gemv_launch(const void* x, int64_t M, int64_t K, const uint32_t* packed,
                              const void* scales, const void* biases, int64_t N, int G,
                              const void* bias, void* y, hipStream_t s) {
  const int64_t waves = cdiv(N, R);
  dim3 grid((unsigned)cdiv(waves, QLQ_GEMV_WAVES_PER_BLOCK), (unsigned)cdiv(M, MT));
  dim3 block(64 * QLQ_GEMV_WAVES_PER_BLOCK);
  const dim3 fgrid((unsigned)cdiv(waves, FWPB), (unsigned)cdiv(M, MT)), fblock(64 * FWPB);
  constexpr bool pair = (BITS == 2 || BITS == 4) && !std::is_same<XT, float>::value;
  constexpr bool flat3 = kStreamPairs<BITS> && !std::is_same<XT, float>::value;
  const int64_t nch = cdiv(K / Chunk<BITS>::CODES, kWave);
  if constexpr (flat3) {
    // 1-, 3-, 5-, 6-bit codes: the flat kernel where it applies, else the generic one
    if (MT <= 2 && (nch == 1 || nch == 2 || nch == 4)) {
#define QLQ_FLAT3(NCH_, G_)                                                                                   \
  hipLaunchKernelGGL((gemv_flat_kernel<BITS, XT, MT, R, NCH_, G_, FWPB>), fgrid, fblock, 0, s, (const XT*)x,  \
                     M, K, packed, (const XT*)scales, (const XT*)biases, N, (const XT*)bias, (XT*)y)
#define QLQ_FLAT3_G(NCH_)                 \
  do {                                    \
    if (G == 32) QLQ_FLAT3(NCH_, 32);     \
    else if (G == 64) QLQ_FLAT3(NCH_, 64); \
    else QLQ_FLAT3(NCH_, 128);            \
  } while (0)
      if (nch == 1) QLQ_FLAT3_G(1);
      else if (nch == 2) QLQ_FLAT3_G(2);
      else QLQ_FLAT3_G(4);
#undef QLQ_FLAT3_G
#undef QLQ_FLAT3
    } else {
      hipLaunchKernelGGL((gemv_generic_kernel<BITS, XT, MT, R>), grid, block, 0, s, (const XT*)x, M, K,
                         packed, (const XT*)scales, (const XT*)biases, N, G, (const XT*)bias, (XT*)y);
    }
  } else if constexpr (pair) {
#define QLQ_FLAT(NCH_, G_)                                                                                    \
  hipLaunchKernelGGL((gemv_flat_kernel<BITS, XT, MT, R, NCH_, G_, FWPB>), fgrid, fblock, 0, s, (const XT*)x,  \
                     M, K, packed, (const XT*)scales, (const XT*)biases, N, (const XT*)bias, (XT*)y)
#define QLQ_FLAT_G(NCH_)           \
  do {                             \
    if (G == 32) QLQ_FLAT(NCH_, 32);  \
    else if (G == 64) QLQ_FLAT(NCH_, 64); \
    else QLQ_FLAT(NCH_, 128);      \
  } while (0)
    if (MT <= 2 && nch == 1) QLQ_FLAT_G(1);
    else if (MT <= 2 && nch == 2) QLQ_FLAT_G(2);
    else if (MT <= 2 && nch == 4) QLQ_FLAT_G(4);
    else
      hipLaunchKernelGGL((gemv_pair_kernel<BITS, XT, MT, R>), grid, block, 0, s, (const XT*)x, M, K,
                         packed, (const XT*)scales, (const XT*)biases, N, G, (const XT*)bias, (XT*)y);
#undef QLQ_FLAT_G
#undef QLQ_FLAT
  } else {
    hipLaunchKernelGGL((gemv_generic_kernel<BITS, XT, MT, R>), grid, block, 0, s, (const XT*)x, M, K,
                       packed, (const XT*)scales, (const XT*)biases, N, G, (const XT*)bias, (XT*)y);
  }
  return hipGetLastError();
}

template <int BITS, typename XT>
static hipError_t gemv_dispatch_m(const void* x, int64_t M, int64_t K, const uint32_t* packed,
                                  const void* scales, const void* biases, int64_t N, int G,
                                  const void* bias, void* y, hipStream_t s) {
  if (M == 1) {
    // 4-bit codes and many rows: two rows per wave in blocks of 8 waves keep
    // more bytes in flight per wave and turn blocks over half as often
    if (BITS == 4 && N >= kGemvLargeN)
      return gemv_launch<BITS, XT, 1, 2, 8>(x, M, K, packed, scales, biases, N, G, bias, y, s);
    return gemv_launch<BITS, XT, 1, QLQ_GEMV_R1>(x, M, K, packed, scales, biases, N, G, bias, y, s);
  }
  if (M == 2) return gemv_launch<BITS, XT, 2, QLQ_GEMV_R2>(x, M, K, packed, scales, biases, N, G, bias, y, s);
  if (M <= 4) return gemv_launch<BITS, XT, 4, 2>(x, M, K, packed, scales, biases, N, G, bias, y, s);
  return gemv_launch<BITS, XT, 8, 1>(x, M, K, packed, scales, biases, N, G, bias, y, s);
}

template <int BITS>
static hipError_t gemv_dispatch_x(const void* x, int x_dtype, int64_t M, int64_t K,
                                  const uint32_t* packed, const void* scales, const void* biases,
                                  int64_t N, int G, const void* bias, void* y, hipStream_t s) {
  switch (x_dtype) {
    case F32: return gemv_dispatch_m<BITS, float>(x, M, K, packed, scales, biases, N, G, bias, y, s);
    case BF16: return gemv_dispatch_m<BITS, bf16_t>(x, M, K, packed, scales, biases, N, G, bias, y, s);
    default: return gemv_dispatch_m<BITS, f16_t>(x, M, K, packed, scales, biases, N, G, bias, y, s);
  }
}

hipError_t launch_affine_gemv(const void* x, int x_dtype, int64_t M, int64_t K,
                              const uint32_t* packed, const void* scales, const void* biases,
                              int64_t N, int bits, int G, const void* bias, void* y, hipStream_t s) {
  switch (bits) {
    case 1: return gemv_dispatch_x<1>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    case 2: return gemv_dispatch_x<2>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    case 3: return gemv_dispatch_x<3>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    case 4: return gemv_dispatch_x<4>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    case 5: return gemv_dispatch_x<5>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    case 6: return gemv_dispatch_x<6>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
    default: return gemv_dispatch_x<8>(x, x_dtype, M, K, packed, scales, biases, N, G, bias, y, s);
  }
}

}  // namespace qlq
