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

#ifndef QLQ_TERN_WAVES
#define QLQ_TERN_WAVES 4  // waves per block; they split K
#endif
#ifndef QLQ_TERN_NB
#define QLQ_TERN_NB 5     // windows a wave loads before computing
#endif

namespace tern {
constexpr int ROWS = 8;                // packed rows per block (32 outputs)
constexpr int WAVES = QLQ_TERN_WAVES;
constexpr int KW = 128;                // k window: a lane loads 32 consecutive k of it
constexpr int NB = QLQ_TERN_NB;
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

// One block: 8 packed rows (32 outputs) x MB rows of x (8 or 16); its waves
// split K in windows of 128 k.
//  * MFMA column n (= lane % 16) is packed row n % 8; MFMA t covers field
//    2t + n / 8 of it, so two MFMAs per k-step cover the 4 fields.  The
//    field's two code bits are masked where they sit, after a shift by 4t
//    shared by the lanes: (w >> 4t) & (0x00030003 << 2f) | MAGIC is the pair
//    (OFF + 4^f c, OFF + 4^f c') with f = n / 8, exact; the epilogue divides
//    by 4^f.  A third MFMA against ones gives X = sum x per row.
//  * Loads: every load instruction reads whole 128-byte lines of distinct
//    rows, straight into LDS (buffer_load ... lds): per window, one
//    instruction for the 8 packed rows' 128 bytes and MB/4 for the x rows'
//    256 bytes; lane L takes row L / 8 and 16-byte chunk (L % 8) ^ (row % 8),
//    which lands in LDS slot L, so that the fragment reads below hit distinct
//    banks.  MFMA k-step s takes k = 32s + 8q .. + 7 from lane group q
//    (= lane / 16), for both operands; each lane reads its 16 bytes of x and
//    8 bytes of codes back from LDS.
//  * A wave issues the loads of NB windows (indexes clamped, no branch),
//    then computes them in issue order, so each window waits only for its
//    own loads (explicit vmcnt, the issue order pinned by scheduling
//    barriers) and all NB windows are in flight at once without holding
//    registers.  The LDS reads of a window sit in one asm block that waits
//    for them: written as plain LDS reads, they would make the compiler wait
//    for every direct-to-LDS load in flight (it cannot tell which LDS bytes
//    those write), later windows' included.
//  * MASK: K is not a multiple of 128 or the windows do not split evenly;
//    k-steps past K and clamped windows then take zeros for x (K % 32 == 0:
//    a k-step is all inside K or all past it).  Rows of x past M read zeros
//    through the buffer range check (no memory traffic); their outputs are
//    never stored.  weight_scale and the bias are loaded before the loop.

// vmcnt wait with an immediate (the loads of later windows stay in flight)
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// until window b's loads have landed: LPW loads per window, issued window by
// window, so the NB - 1 - b later windows' loads may stay in flight (b is a
// constant once the window loop is unrolled, and the switch folds away)
template <int NB, int LPW>
__device__ __forceinline__ void wait_window(int b) {
  static_assert(NB <= 8, "windows in flight");
  switch (NB - 1 - b) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<LPW>(); break;
    case 2: wait_vm<2 * LPW>(); break;
    case 3: wait_vm<3 * LPW>(); break;
    case 4: wait_vm<4 * LPW>(); break;
    case 5: wait_vm<5 * LPW>(); break;
    case 6: wait_vm<6 * LPW>(); break;
    default: wait_vm<7 * LPW>(); break;
  }
}

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// 16 bytes per lane from a buffer straight into LDS at byte address lds_addr
// (wave-uniform; lane i writes lds_addr + 16 i), with cache policy AUX
template <int AUX>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(uintptr_t)lds_addr, 16, off, 0, 0, AUX);
}

// One window's fragments out of LDS: x for k-steps 0..3 at xa0, xa1,
// xa0 + 1 KiB, xa1 + 1 KiB and codes at wa[0..3], each plus the window's
// offsets XO and WO; one asm block that waits for its reads (see above).
template <int XO, int WO>
__device__ __forceinline__ void read_window(uint32_t xa0, uint32_t xa1, const uint32_t (&wa)[4],
                                            u32x4_v (&xv)[4], u32x2_t (&cv)[4]) {
  static_assert(XO + 1024 < 65536 && WO < 65536, "16-bit LDS offsets");
  asm volatile(
      "ds_read_b128 %0, %8 offset:%14\n\t"
      "ds_read_b128 %1, %9 offset:%14\n\t"
      "ds_read_b128 %2, %8 offset:%15\n\t"
      "ds_read_b128 %3, %9 offset:%15\n\t"
      "ds_read_b64 %4, %10 offset:%16\n\t"
      "ds_read_b64 %5, %11 offset:%16\n\t"
      "ds_read_b64 %6, %12 offset:%16\n\t"
      "ds_read_b64 %7, %13 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(xv[0]), "=&v"(xv[1]), "=&v"(xv[2]), "=&v"(xv[3]), "=&v"(cv[0]), "=&v"(cv[1]), "=&v"(cv[2]),
        "=&v"(cv[3])
      : "v"(xa0), "v"(xa1), "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "n"(XO), "n"(XO + 1024), "n"(WO)
      : "memory");
}

template <typename XT, int MB, bool MASK>
__global__ void __launch_bounds__(64 * tern::WAVES)
ternary_mfma_kernel(const XT* __restrict__ x, int M, int K, const uint8_t* __restrict__ packed,
                    int R, const XT* __restrict__ wscale, int invert,
                    const XT* __restrict__ bias, XT* __restrict__ y) {
  using namespace tern;
  using TT = TernT<XT>;
  static_assert(MB == 8 || MB == 16, "x rows per block");
  static_assert(NB <= 5, "window offsets below");
  static_assert(64 * WAVES * 2 >= 512, "two outputs per thread cover the block");
  constexpr int XLW = MB / 4;        // x load instructions per window (256 bytes per row)
  constexpr int XWIN = MB * 256;     // x bytes per window
  constexpr int LPW = 1 + XLW;       // load instructions per window
  // per wave: NB windows of x, then (after every wave's x) NB windows of codes
  __shared__ __attribute__((aligned(16))) uint8_t lds[WAVES * NB * (XWIN + 1024)];
  __shared__ float red[WAVES][3][4][64];  // [wave][mfma][elem][lane]

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r0 = blockIdx.x * ROWS;
  const int m0 = blockIdx.y * MB;
  const int N = 4 * R;
  const int n = lane & 15, q = lane >> 4;
  const uint32_t fmask = 0x00030003u << (2 * (n >> 3));

  // scale and bias first, as raw bits with no branch (an out-of-range offset
  // reads 0): their latency hides under the main loop
  const uint16_t ws_bits = *reinterpret_cast<const uint16_t*>(wscale);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, bias ? N * 2 : 0);
  uint16_t bv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = tid + 64 * WAVES * u;
    const int ri = o & 7, j = o >> 7;
    const int off = o < 512 && r0 + ri < R ? (r0 + ri + j * R) * 2 : kOutOfRange;
    bv[u] = __builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0);
  }

  // the block's packed rows and x rows, one buffer descriptor each
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed + (int64_t)r0 * K, (min(R, r0 + ROWS) - r0) * K);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (int64_t)m0 * K, (min(M, m0 + MB) - m0) * K * 2);
  // load lane L: row L / 8 of its group of 8 rows, chunk (L % 8) ^ (row % 8)
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;
  const int w_off = lr * K + 16 * lc;                  // + window * 128
  int x_off[XLW];                                      // + window * 256
#pragma unroll
  for (int i = 0; i < XLW; ++i) x_off[i] = (8 * (i >> 1) + lr) * K * 2 + 16 * (8 * (i & 1) + lc);
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);   // LDS byte address
  const uint32_t xw_base = lds0 + wid * NB * XWIN;                    // this wave's x windows
  const uint32_t ww_base = lds0 + WAVES * NB * XWIN + wid * NB * 1024;  // and its code windows
  // fragment addresses: x row n (chunk 4s + q of the window; x load i holds
  // chunks 8 (i % 2) .. of rows 8 (i / 2) ..), codes of packed row n % 8
  // (bytes 8 (q % 2) .. of chunk 2s + q / 2)
  const int nr = n & 7;
  const uint32_t xrow_base = xw_base + (MB == 16 ? (n >> 3) * 2048 : 0) + 128 * nr;
  const uint32_t xa0 = xrow_base + 16 * (q ^ nr);
  const uint32_t xa1 = xrow_base + 16 * ((4 + q) ^ nr);
  uint32_t wa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) wa[s] = ww_base + 128 * nr + 16 * ((2 * s + (q >> 1)) ^ nr) + 8 * (q & 1);
  const bool xrow_live = MB == 16 || n < 8;  // A rows 8..15 are zero when the block holds 8 x rows

  f32x4_v P[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) P[t] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  u32x4_v ones;
  ones[0] = ones[1] = ones[2] = ones[3] = TT::ONES;

  const int nwin = (K + KW - 1) / KW;
  for (int base = wid; base < nwin; base += WAVES * NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int win = min(base + b * WAVES, nwin - 1);
      // each packed byte is read once: streaming policy; x is read by every block
      load_to_lds<kStreamAux>(rw, ww_base + b * 1024, w_off + win * KW);
#pragma unroll
      for (int i = 0; i < XLW; ++i) load_to_lds<0>(rx, xw_base + b * XWIN + i * 1024, x_off[i] + win * 2 * KW);
      // the waits below count loads in this order: window by window
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      wait_window<NB, LPW>(b);
      u32x4_v xv[4];
      u32x2_t cv[4];
      // b is a constant after unrolling; the offsets are immediates
      switch (b) {
        case 0: read_window<0 * XWIN, 0 * 1024>(xa0, xa1, wa, xv, cv); break;
        case 1: read_window<1 * XWIN, 1 * 1024>(xa0, xa1, wa, xv, cv); break;
        case 2: read_window<2 * XWIN, 2 * 1024>(xa0, xa1, wa, xv, cv); break;
        case 3: read_window<3 * XWIN, 3 * 1024>(xa0, xa1, wa, xv, cv); break;
        default: read_window<4 * XWIN, 4 * 1024>(xa0, xa1, wa, xv, cv); break;
      }
      const int wv = base + b * WAVES;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bool use = xrow_live && (!MASK || (wv < nwin && wv * KW + 32 * st < K));
        const u32x4_v v = use ? xv[st] : u32x4_v{0, 0, 0, 0};
        // x pairs in the code order of a dword: (k0,k2), (k1,k3) per 4 k
        u32x4_v a;
        a[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
        a[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
        a[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
        a[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
        const uint32_t w0 = cv[st][0], w1 = cv[st][1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4_v bq;
          bq[0] = ((w0 >> (4 * t)) & fmask) | TT::MAGIC;
          bq[1] = ((w0 >> (4 * t + 8)) & fmask) | TT::MAGIC;
          bq[2] = ((w1 >> (4 * t)) & fmask) | TT::MAGIC;
          bq[3] = ((w1 >> (4 * t + 8)) & fmask) | TT::MAGIC;
          P[t] = TT::mma(a, bq, P[t]);
        }
        P[2] = TT::mma(a, ones, P[2]);  // X: every column holds its row's sum
      }
      // window b's MFMAs before the wait for window b + 1
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wid][t][e][lane] = P[t][e];
  __syncthreads();

  const float ws = bits16_to_f32<XT>(ws_bits);
  const float sigma = invert ? __fdiv_rn(1.0f, ws) : ws;
  // block outputs: 16 m x 4 fields x 8 packed rows = 512, two per thread
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o = tid + 64 * WAVES * u;
    if (o >= 512) break;
    const int ri = o & 7, mi = (o >> 3) & 15, j = o >> 7;
    // D layout: lane (mi / 4) * 16 + column holds row mi at element mi % 4;
    // field j is MFMA j / 2, column ri + 8 (j % 2), scaled by 4^(j % 2)
    const int t = j >> 1, src_lane = (mi >> 2) * 16 + ri + 8 * (j & 1), e = mi & 3;
    float p = 0.0f, X = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      p += red[w][t][e][src_lane];
      X += red[w][2][e][src_lane];
    }
    const int m = m0 + mi, r = r0 + ri;
    if (mi < MB && m < M && r < R) {
      const int nn = r + j * R;
      // sum x (c - 1) = (P - OFF X) / 4^f - X
      const float c = __fmaf_rn(-TT::OFF, X, p) * ((j & 1) ? 0.25f : 1.0f);
      float v = sigma * (c - X);
      if (bias) v = v + bits16_to_f32<XT>(bv[u]);
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
  const int mb = M <= 8 ? 8 : 16;  // x rows per block
  dim3 grid((unsigned)cdiv(R, ROWS), (unsigned)cdiv(M, mb)), block(64 * WAVES);
  const int m = (int)M, k = (int)K, r = (int)R;
  const int64_t nwin = cdiv(K, KW);
  const bool mask = K % KW != 0 || nwin % (WAVES * NB) != 0;
#define QLQ_TERN(XT_, MB_, MASK_)                                                                               \
  hipLaunchKernelGGL((ternary_mfma_kernel<XT_, MB_, MASK_>), grid, block, 0, s, (const XT_*)x, m, k, packed, r, \
                     (const XT_*)weight_scale, invert, (const XT_*)bias, (XT_*)y)
#define QLQ_TERN_MB(XT_, MASK_)              \
  do {                                       \
    if (mb == 8) QLQ_TERN(XT_, 8, MASK_);    \
    else QLQ_TERN(XT_, 16, MASK_);           \
  } while (0)
  if (x_dtype == BF16) {
    if (mask) QLQ_TERN_MB(bf16_t, true); else QLQ_TERN_MB(bf16_t, false);
  } else {
    if (mask) QLQ_TERN_MB(f16_t, true); else QLQ_TERN_MB(f16_t, false);
  }
#undef QLQ_TERN_MB
#undef QLQ_TERN
  return hipGetLastError();
}

}  // namespace qlq
