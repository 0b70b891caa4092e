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
// Tiling: block tile 128x128, k-iteration BK (256), 8 waves: 4 sub-tiles of 64x64
// (2x2 MFMA 32x32x32 tiles) times 2 halves of each k-iteration's k-steps, so
// two waves share each SIMD while one block covers a CU; the halves are summed
// through LDS at the end.  XCD-aware tile order.
//
// Operand tiles go from global memory straight into a ring of STAGES LDS
// buffers (buffer loads with the LDS-destination bit: no register staging,
// no LDS store instructions).  A load whose offset lies past the buffer's
// size writes zeros, which covers rows past M / N and k past K.  Each
// 128-byte LDS row holds its eight 16-byte k-chunks in swizzled slots (chunk
// c of row r at slot c ^ swz(r)), so the fragment reads of 8 or 16 lanes
// (consecutive rows, same chunk) fall on distinct banks.
#include "common.hpp"
#include "int4.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace qlq {

namespace i8 {
constexpr int BM = 128, BN = 128, KS = 32;  // KS: MFMA k-step
constexpr int WAVES = 8;   // 4 sub-tiles x 2 halves of each k-iteration
constexpr int THREADS = 64 * WAVES;
constexpr int ROWS_W = BM / WAVES;  // tile rows each wave loads (per operand)
// k-iteration BK bytes, ring of STAGES slots
template <int BK, int STAGES> struct Cfg {
  static constexpr int CPR = BK / 16;           // 16-byte chunks per LDS row
  static constexpr int RPI = 1024 / BK;         // rows one wave-wide load fills
  static constexpr int TILE = BM * BK;          // bytes of one operand tile (BM == BN)
  static constexpr int STAGE = 2 * TILE;        // A tile then B tile
  static constexpr int LPW = ROWS_W / RPI;      // loads per thread per operand tile
  static constexpr int LPT = 2 * LPW;           // loads per thread per k-iteration
  static constexpr int QN = BK / KS / 2;        // k-steps per wave per k-iteration
  static constexpr int VMCNT = (STAGES - 2) * LPT;  // loads allowed outstanding at the wait
  static_assert(BM == BN && (BK == 128 || BK == 256) && ROWS_W % RPI == 0, "tile shape");
  static_assert(STAGES >= 2 && VMCNT < 64, "ring depth");
  static __device__ __forceinline__ int swz(int r) { return lds_swz<CPR>(r); }
};
}  // namespace i8

typedef __attribute__((ext_vector_type(16))) int i32x16_v;
// 32x32x32 int8 MFMA.  Operands: lane l holds 16 consecutive k (bytes) of row
// (A) or column (B) l % 32, k offset 16 * (l / 32).  Result: lane l, element e
// is row 8*(e/4) + 4*(l/32) + e%4, column l % 32.
__device__ __forceinline__ i32x16_v mma_i8(u32x4_v a, u32x4_v b, i32x16_v c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_v, a), __builtin_bit_cast(i32x4_v, b),
                                                c, 0, 0, 0);
}

// ---- packed int4 B operand (BSRC != 0; layout and unpacking in int4.hpp).
// The MFMA wants 16 consecutive k of one column per lane, so the tile is
// turned around on its way to LDS: thread (rg, cg) loads k-pair rows
// 8 rg .. 8 rg + 7 of columns 4 cg .. 4 cg + 3, and writes per column one
// 16-byte chunk of int8 values 16 (code - 8), in the chunk order the
// activations are stored in.  The factor 16 comes off the int32 sum exactly
// (>> 4).
namespace w4 {
// slot of chunk c in B row r: the 8-lane groups that write rows 4 cg + j
// (cg = 8a .. 8a+7) and the fragment reads of 8 or 16 consecutive rows both
// meet distinct slots
__device__ __forceinline__ int swz(int r) { return (r & 15) ^ ((r >> 4) & 1); }

// this thread's 8 packed rows of the 128-row tile starting at k-pair kp0;
// columns past N repeat the last in-range column group (never stored)
template <bool BYTES>
__device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int kp0, int K2, int N, int ncols, int rg, int cg,
                                     uint32_t (&bw)[8]) {
  const int col = BYTES ? 4 * cg : min(4 * cg, ncols - 4);
  int4::load8<BYTES>(r, kp0, 8 * rg, kp0 + 128 <= K2, K2, N, ncols, col, bw);
}

// unpack and write this thread's four 16-byte chunks into the B tile (rows of
// BK bytes)
template <int BK>
__device__ __forceinline__ void store(int8_t* tile, const uint32_t (&bw)[8], int rg, int cg) {
  uint32_t lo[4], hi[4];
  int4::transpose4(bw[0], bw[1], bw[2], bw[3], lo);
  int4::transpose4(bw[4], bw[5], bw[6], bw[7], hi);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = 4 * cg + c;
    *reinterpret_cast<u32x4_v*>(tile + row * BK + ((rg ^ swz(row)) << 4)) = int4::unpack16(lo[c], hi[c]);
  }
}
}  // namespace w4

// ---- A operand quantized in the kernel (ASRC != 0: a is fp16 / bf16 x and
// sa its row scales from a pre-pass).  Thread t owns row t / 4 of the
// 128-row tile and its 64 consecutive k from 64 (t % 4): eight 16-byte loads
// one tile ahead into registers, then the row quantizer's arithmetic
// (RowDivider quotient, clamp, round half to even) and four 16-byte chunks of
// codes into the swizzled A tile, so the codes equal those the standalone
// quantizer writes.
namespace qa {
template <int BK>
__device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int row, int k0, int K, uint4 (&xa)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = k0 + 8 * i;  // K % 16 == 0: a 16-byte chunk is inside K or past it
    const u32x4_v v = __builtin_amdgcn_raw_buffer_load_b128(r, k < K ? (row * K + k) * 2 : kOutOfRange, 0, 0);
    xa[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}
template <int ASRC>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
  if constexpr (ASRC == 1) return (float)__builtin_bit_cast(f16_t, (uint16_t)h);
  else return __uint_as_float(h << 16);
}
template <int ASRC, int BK, int CPR>
__device__ __forceinline__ void store(int8_t* tile, const uint4 (&xa)[8], const RowDivider& dv, int row, int cq) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // chunk 4 cq + j: 16 codes from loads 2j and 2j + 1
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 v = xa[2 * j + h];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
      uint32_t c[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[2 * e] = int8_code_bits(dv.div(half_to_f32<ASRC>(d[e] & 0xFFFFu)));
        c[2 * e + 1] = int8_code_bits(dv.div(half_to_f32<ASRC>(d[e] >> 16)));
      }
      w[2 * h] = pack_low_bytes(c[0], c[1], c[2], c[3]);
      w[2 * h + 1] = pack_low_bytes(c[4], c[5], c[6], c[7]);
    }
    const int c = 4 * cq + j;
    *reinterpret_cast<u32x4_v*>(tile + row * BK + ((c ^ lds_swz<CPR>(row)) << 4)) = u32x4_v{w[0], w[1], w[2], w[3]};
  }
}
}  // namespace qa

// Pipeline (one barrier per k-iteration).  Before iteration `it`, tiles
// it .. it+STAGES-2 are in flight to their ring slots.  Iteration it: wait
// until this thread's loads of tile it have landed, barrier (every thread's
// have, and every wave has finished reading slot (it-1) % STAGES), issue the
// loads of tile it+STAGES-1 into that slot, compute tile it.  Tiles past the
// last one load as zeros and are never computed.
//
// PG > 0 (per-group weights, group of PG input values): sb is the per-group
// scale table [K/PG, N]; the int32 accumulators are flushed into fp32 as
// acc * sb[g, n] at every group boundary of a wave's k-steps (a group longer
// than a wave's half of an iteration is flushed once per half: the scale is
// the same, the sum is linear), and y = acc_f * sa[m] (+ bias).  The int32
// partial of one flush is below 2^24, so its conversion is exact.  With one
// flush per k-iteration (groups of 128 or 256) the int32 sums alternate
// between two register sets: iteration it's sums are rescaled between the
// MFMAs of iteration it + 1, one 32x32 sub-tile per k-step, in the same
// order as a flush at the end of the iteration would take them.
//
// BSRC != 0: b is packed int4 [K/2, N] (namespace w4), loaded into registers
// one tile ahead and written to the B half of the ring slot after the MFMAs
// of the current tile (BSRC 2: byte loads, for N % 4 != 0).
//
// ASRC != 0 (1: fp16, 2: bf16): a is the activations x [M, K], quantized to
// the A tile in the kernel with the row scales sa (namespace qa), the same
// way: registers one tile ahead, LDS after the current tile's MFMAs.
template <int OUT, int BK, int STAGES, int PG = 0, int BSRC = 0, int ASRC = 0>
__global__ void __launch_bounds__(i8::THREADS, 1)
int8_gemm_kernel(const int8_t* __restrict__ a, const void* __restrict__ b, int M, int N, int K,
                 const float* __restrict__ sa, const float* __restrict__ sb, const void* __restrict__ bias,
                 void* __restrict__ out) {
  using namespace i8;
  using C = Cfg<BK, STAGES>;
  constexpr bool W4 = BSRC != 0;
  constexpr bool QA = ASRC != 0;
  static_assert(!QA || (!W4 && PG == 0 && OUT != 0 && BK == 256 && STAGES == 2 && THREADS == 512),
                "quantized A: 128 rows x 256 k, 64 k per thread, double buffer, scaled output");
  static_assert(PG == 0 || (OUT != 0 && PG % KS == 0), "per-group scales need a scaled output");
  static_assert(!W4 || (PG == 0 && OUT != 0 && BK == 256 && STAGES == 2 && THREADS == 512),
                "int4 B: 128 k-pair rows x 128 columns, 32 bytes per thread, double buffer");
  constexpr int FS = PG == 0 ? C::QN : (PG / KS < C::QN ? PG / KS : C::QN);  // k-steps per flush
  constexpr int NF = C::QN / FS;                                              // flushes per k-iteration
  constexpr bool PIPE = PG != 0 && NF == 1;  // flushes overlap the next iteration's MFMAs
  static_assert(!PIPE || 4 % C::QN == 0, "whole sub-tiles per k-step");
  // the ring during the K loop, then the 64 KiB of int32 partial sums that
  // join the two k-halves
  __shared__ __attribute__((aligned(16))) int8_t smem[STAGES * C::STAGE];
  static_assert(STAGES * C::STAGE >= 4 * 64 * 64 * 4, "reduction area fits");

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wq = wid & 3, kh = wid >> 2;  // 64x64 sub-tile, half of the k-steps
  const int wm = wq >> 1, wn = wq & 1;
  int tm, tn;
  tile_coords<8>(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m_blk = tm * BM, n_blk = tn * BN;
  const int nk = (K + BK - 1) / BK;

  const int rows_a = min(BM, M - m_blk), rows_b = min(BN, N - n_blk);
  const __amdgpu_buffer_rsrc_t rsa = QA ? make_rsrc((const uint16_t*)(const void*)a + (int64_t)m_blk * K, rows_a * K * 2)
                                        : make_rsrc(a + (int64_t)m_blk * K, rows_a * K);
  const int K2 = K / 2;
  const __amdgpu_buffer_rsrc_t rsb =
      W4 ? make_rsrc((const uint8_t*)b + n_blk, K2 * N - n_blk)
         : make_rsrc((const int8_t*)b + (int64_t)n_blk * K, rows_b * K);
  const int cg = tid & 31, rg = tid >> 5;  // int4 B: column group, k-pair row group
  // load j of this thread: row wid*ROWS_W + RPI*j + lane/CPR of both tiles,
  // chunk (lane % CPR) ^ swz(row), i.e. LDS slot lane % CPR
  int voff[C::LPW], kc[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int r = wid * ROWS_W + C::RPI * j + lane / C::CPR, c = (lane % C::CPR) ^ C::swz(r);
    voff[j] = r * K + c * 16;
    kc[j] = c * 16;
  }
#define QLQ_ISSUE(T)                                                                            \
  do {                                                                                          \
    const int k0_ = (T) * BK;                                                                   \
    int8_t* dst_ = smem + ((T) % STAGES) * C::STAGE + wid * ROWS_W * BK;                        \
    _Pragma("unroll") for (int j = 0; j < C::LPW; ++j) {                                        \
      const int o_ = k0_ + kc[j] < K ? voff[j] + k0_ : kOutOfRange;                             \
      if constexpr (!QA) load_lds_b128(rsa, dst_ + 1024 * j, o_);                               \
      if constexpr (!W4) load_lds_b128(rsb, dst_ + C::TILE + 1024 * j, o_);                     \
    }                                                                                           \
  } while (0)

  // fragment offsets inside a stage: [operand i/j][k-step q]
  int aoff[2][C::QN], boff[2][C::QN];
#pragma unroll
  for (int q = 0; q < C::QN; ++q) {
    const int c = (kh * C::QN + q) * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ra = wm * 64 + 32 * i + (lane & 31), rb = wn * 64 + 32 * i + (lane & 31);
      aoff[i][q] = ra * BK + (c ^ C::swz(ra)) * 16;
      boff[i][q] = C::TILE + rb * BK + (c ^ (W4 ? w4::swz(rb) : C::swz(rb))) * 16;
    }
  }

  i32x16_v acc[2][2];
  f32x16_v accf[2][2];  // per-group mode: rescaled sums
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = i32x16_v{};
      accf[i][j] = f32x16_v{};
    }
  int ncol[2];  // this lane's output columns (clamped)
#pragma unroll
  for (int j = 0; j < 2; ++j) ncol[j] = min(n_blk + wn * 64 + 32 * j + (lane & 31), N - 1);
  const int ng = PG ? K / (PG ? PG : 1) : 1;

  uint32_t bw[8];  // int4 B: the next tile's packed rows
  if constexpr (W4) w4::load<BSRC == 2>(rsb, 0, K2, N, N - n_blk, rg, cg, bw);
  // quantized A: this thread's row (t / 4) and 64 k (from 64 (t % 4)), the
  // row's divisor from its scale
  const int qa_row = tid >> 2, qa_cq = tid & 3;
  uint4 xa[8];
  const RowDivider qa_dv(QA && m_blk + qa_row < M ? sa[m_blk + qa_row] : 1.0f);
  if constexpr (QA) qa::load<BK>(rsa, qa_row, 64 * qa_cq, K, xa);
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) QLQ_ISSUE(t);
  if constexpr (W4) w4::store<BK>(smem + C::TILE, bw, rg, cg);
  if constexpr (QA) qa::store<ASRC, BK, C::CPR>(smem, xa, qa_dv, qa_row, qa_cq);
  if constexpr (PIPE) {
    i32x16_v acc2[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc2[i][j] = i32x16_v{};
    float sc0[2] = {0.0f, 0.0f}, sc1[2] = {0.0f, 0.0f};
    // rescale sub-tile t of the int32 sums `sums` into accf and clear it
    auto flush_tile = [&](i32x16_v (&sums)[2][2], const float (&scl)[2], int t) {
      const int i = t >> 1, j = t & 1;
#pragma unroll
      for (int e = 0; e < 16; ++e) accf[i][j][e] = __builtin_fmaf((float)sums[i][j][e], scl[j], accf[i][j][e]);
      sums[i][j] = i32x16_v{};
    };
    // k-iteration it: MFMAs into cur, the previous iteration's sums (prev,
    // scales scp) rescaled between them; this iteration's scales into scc
    auto step = [&](int it, i32x16_v (&cur)[2][2], i32x16_v (&prev)[2][2], float (&scc)[2], float (&scp)[2]) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(C::VMCNT) : "memory");
      // scp was loaded an iteration ago and the wait above has drained it:
      // from here on it is an ordinary value (no wait on the newer loads)
      asm volatile("" : "+v"(scp[0]), "+v"(scp[1]));
      {
        const int g = min((it * BK + kh * C::QN * KS) / PG, ng - 1);  // past K: zero sums
#pragma unroll
        for (int j = 0; j < 2; ++j) scc[j] = sb[(int64_t)g * N + ncol[j]];
      }
      QLQ_ISSUE(it + STAGES - 1);
      const int8_t* st_ = smem + (it % STAGES) * C::STAGE;
      u32x4_v af[2][C::QN], bf[2][C::QN];
#pragma unroll
      for (int q = 0; q < C::QN; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i][q] = *reinterpret_cast<const u32x4_v*>(st_ + aoff[i][q]);
          bf[i][q] = *reinterpret_cast<const u32x4_v*>(st_ + boff[i][q]);
        }
#pragma unroll
      for (int q = 0; q < C::QN; ++q) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) cur[i][j] = mma_i8(af[i][q], bf[j][q], cur[i][j]);
#pragma unroll
        for (int t = q * 4 / C::QN; t < (q + 1) * 4 / C::QN; ++t) flush_tile(prev, scp, t);
      }
    };
    int it = 0;
    for (; it + 1 < nk; it += 2) {
      step(it, acc, acc2, sc0, sc1);
      step(it + 1, acc2, acc, sc1, sc0);
    }
    if (it < nk) {
      step(it, acc, acc2, sc0, sc1);
#pragma unroll
      for (int t = 0; t < 4; ++t) flush_tile(acc, sc0, t);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) flush_tile(acc2, sc1, t);
    }
  } else
  for (int it = 0; it < nk; ++it) {
    // this thread's loads of tile it are done when at most the later
    // STAGES-2 tiles' loads are outstanding; then the barrier
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(C::VMCNT) : "memory");
    // per-group scales of this iteration's flushes, requested before the
    // tile loads so that waiting for them does not wait for those
    float scf[NF][2];
    if constexpr (PG != 0) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int g = min((it * BK + (kh * C::QN + f * FS) * KS) / PG, ng - 1);  // past K: zero sums
#pragma unroll
        for (int j = 0; j < 2; ++j) scf[f][j] = sb[(int64_t)g * N + ncol[j]];
      }
    }
    const bool more = (W4 || QA) && it + 1 < nk;
    if constexpr (W4)
      if (more) w4::load<BSRC == 2>(rsb, (it + 1) * (BK / 2), K2, N, N - n_blk, rg, cg, bw);
    if constexpr (QA)
      if (more) qa::load<BK>(rsa, qa_row, (it + 1) * BK + 64 * qa_cq, K, xa);
    QLQ_ISSUE(it + STAGES - 1);
    const int8_t* st_ = smem + (it % STAGES) * C::STAGE;
    u32x4_v af[2][C::QN], bf[2][C::QN];
#pragma unroll
    for (int q = 0; q < C::QN; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i][q] = *reinterpret_cast<const u32x4_v*>(st_ + aoff[i][q]);
        bf[i][q] = *reinterpret_cast<const u32x4_v*>(st_ + boff[i][q]);
      }
#pragma unroll
    for (int q = 0; q < C::QN; ++q) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma_i8(af[i][q], bf[j][q], acc[i][j]);
      if constexpr (PG != 0) {
        if ((q + 1) % FS == 0) {
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
              for (int e = 0; e < 16; ++e)
                accf[i][j][e] = __builtin_fmaf((float)acc[i][j][e], scf[q / FS][j], accf[i][j][e]);
              acc[i][j] = i32x16_v{};
            }
        }
      }
    }
    if constexpr (W4)
      if (more) w4::store<BK>(smem + ((it + 1) % STAGES) * C::STAGE + C::TILE, bw, rg, cg);
    if constexpr (QA)
      if (more) qa::store<ASRC, BK, C::CPR>(smem + ((it + 1) % STAGES) * C::STAGE, xa, qa_dv, qa_row, qa_cq);
  }
#undef QLQ_ISSUE
  // the zero tiles issued past the end may still be landing in the ring
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue operands, loaded before the join so that their latency overlaps it
  float sam[2][16], sbn[2], bn[2];
  if constexpr (OUT != 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m_blk + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        sam[i][e] = m < M ? sa[m] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = min(n_blk + wn * 64 + 32 * j + (lane & 31), N - 1);
      sbn[j] = PG == 0 ? sb[n] : 1.0f;
      bn[j] = !bias ? 0.0f
                    : OUT == 1 ? Elem<f16_t>::load((const f16_t*)bias, n)
                               : Elem<bf16_t>::load((const bf16_t*)bias, n);
    }
  }

  // ---- join the two k-halves: waves 4-7 park their sums in LDS (the tile
  // buffers are free now), waves 0-3 add them and run the epilogue
  int32_t* red = reinterpret_cast<int32_t*>(smem);  // 4 sub-tiles x 64 values x 64 lanes
  float* redf = reinterpret_cast<float*>(smem);      // the same area, per-group mode
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ix = (wq * 64 + (i * 2 + j) * 16 + e) * 64 + lane;
          if constexpr (PG == 0) red[ix] = acc[i][j][e];
          else redf[ix] = accf[i][j][e];
        }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int ix = (wq * 64 + (i * 2 + j) * 16 + e) * 64 + lane;
        if constexpr (PG == 0) acc[i][j][e] += red[ix];
        else accf[i][j][e] += redf[ix];
      }

  if constexpr (OUT == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m_blk + wm * 64 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n_blk + wn * 64 + 32 * j + (lane & 31);
          if (n < N) reinterpret_cast<int32_t*>(out)[(int64_t)m * N + n] = acc[i][j][e];
        }
      }
  } else {
    // y = fp32(c) * sa[m] * sb[n] (+ bias[n]), or acc_f * sa[m] (+ bias[n])
    // per group, rounded once; this wave's own part of the join area
    // (already read) stages the 16-bit tile
    float v[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (PG == 0) v[i][j][e] = ((float)(W4 ? acc[i][j][e] >> 4 : acc[i][j][e]) * sam[i][e]) * sbn[j];
          else v[i][j][e] = accf[i][j][e] * sam[i][e];
          if (bias) v[i][j][e] = v[i][j][e] + bn[j];
        }
    static_assert(kTileStageBytes <= 64 * 64 * 4, "staging fits the wave's join area");
    int8_t* stage = smem + wq * 64 * 64 * 4;
    const int row0 = m_blk + wm * 64, col0 = n_blk + wn * 64;
    if constexpr (OUT == 1)
      store_tile64_16<f16_t>(v, (f16_t*)out, N, row0, col0, M - row0, N - col0, stage, lane);
    else
      store_tile64_16<bf16_t>(v, (bf16_t*)out, N, row0, col0, M - row0, N - col0, stage, lane);
  }
}

template <int BK, int STAGES>
hipError_t launch_int8_gemm_cfg(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                const float* sa, const float* sb, const void* bias, int out_dtype,
                                void* out, hipStream_t s) {
  const int64_t tiles = cdiv(M, i8::BM) * cdiv(N, i8::BN);
  dim3 grid((unsigned)tiles), block(i8::THREADS);
  const int m = (int)M, n = (int)N, k = (int)K;
  if (out_dtype < 0)
    hipLaunchKernelGGL((int8_gemm_kernel<0, BK, STAGES>), grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  else if (out_dtype == F16)
    hipLaunchKernelGGL((int8_gemm_kernel<1, BK, STAGES>), grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  else
    hipLaunchKernelGGL((int8_gemm_kernel<2, BK, STAGES>), grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out);
  return hipGetLastError();
}

// Per-group weights (group_size 64, 128 or 256): scale_w [K/group_size, N].
hipError_t launch_int8_gemm_pergroup(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                     const float* sa, const float* scale_w, int group_size,
                                     const void* bias, int out_dtype, void* out, hipStream_t s) {
  const int64_t tiles = cdiv(M, i8::BM) * cdiv(N, i8::BN);
  dim3 grid((unsigned)tiles), block(i8::THREADS);
  const int m = (int)M, n = (int)N, k = (int)K;
#define QLQ_PG_LAUNCH(OUTV, PGV)                                                                       \
  hipLaunchKernelGGL((int8_gemm_kernel<OUTV, 256, 2, PGV>), grid, block, 0, s, a, b, m, n, k, sa, scale_w, \
                     bias, out)
  const bool h = out_dtype == F16;
  switch (group_size) {
    case 64: if (h) QLQ_PG_LAUNCH(1, 64); else QLQ_PG_LAUNCH(2, 64); break;
    case 128: if (h) QLQ_PG_LAUNCH(1, 128); else QLQ_PG_LAUNCH(2, 128); break;
    default: if (h) QLQ_PG_LAUNCH(1, 256); else QLQ_PG_LAUNCH(2, 256); break;
  }
#undef QLQ_PG_LAUNCH
  return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const int8_t* a, const uint8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, const void* bias, int out_dtype, void* out,
                            hipStream_t s) {
  const int64_t tiles = cdiv(M, i8::BM) * cdiv(N, i8::BN);
  dim3 grid((unsigned)tiles), block(i8::THREADS);
  const int m = (int)M, n = (int)N, k = (int)K;
#define QLQ_W4_LAUNCH(OUTV, SRC) \
  hipLaunchKernelGGL((int8_gemm_kernel<OUTV, 256, 2, 0, SRC>), grid, block, 0, s, a, b, m, n, k, sa, sb, bias, out)
  const bool h = out_dtype == F16;
  if (N % 4 == 0) {
    if (h) QLQ_W4_LAUNCH(1, 1); else QLQ_W4_LAUNCH(2, 1);
  } else {
    if (h) QLQ_W4_LAUNCH(1, 2); else QLQ_W4_LAUNCH(2, 2);
  }
#undef QLQ_W4_LAUNCH
  return hipGetLastError();
}

hipError_t launch_int8_gemm_quant_a(const void* x, int x_dtype, const int8_t* b, int64_t M, int64_t N, int64_t K,
                                    const float* sx, const float* sb, const void* bias, void* out, hipStream_t s) {
  const int64_t tiles = cdiv(M, i8::BM) * cdiv(N, i8::BN);
  dim3 grid((unsigned)tiles), block(i8::THREADS);
  const int m = (int)M, n = (int)N, k = (int)K;
  const int8_t* a = (const int8_t*)x;  // reinterpreted by the kernel as 16-bit x
  if (x_dtype == F16)
    hipLaunchKernelGGL((int8_gemm_kernel<1, 256, 2, 0, 0, 1>), grid, block, 0, s, a, b, m, n, k, sx, sb, bias, out);
  else
    hipLaunchKernelGGL((int8_gemm_kernel<2, 256, 2, 0, 0, 2>), grid, block, 0, s, a, b, m, n, k, sx, sb, bias, out);
  return hipGetLastError();
}

hipError_t launch_int8_gemm(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                            const float* sa, const float* sb, const void* bias, int out_dtype,
                            void* out, hipStream_t s) {
  // 256-byte k-iterations, double-buffered: fewer barriers per MFMA than
  // 128-byte iterations in a deeper ring (measured faster on 1024x4096x4096
  // and 2048x11008x4096)
  return launch_int8_gemm_cfg<256, 2>(a, b, M, N, K, sa, sb, bias, out_dtype, out, s);
}

}  // namespace qlq
