// W4A8 linear for a few rows of x (M <= 8): y = dequant(quant_a(x) .
// unpack4(w)) with the packed int4 weight [K/2, N] read once.
//
// "cider/ops.py": w4a8_linear (per-column int4 weights from pack_weight_int4,
// per-row int8 activations, y = acc * sx[m] * scale_w[n]).
//
// With a handful of rows the 128 x 128 GEMM tiles leave most of the chip idle,
// so the weight is split over K as well: block (bx, by) takes 256 columns and
// the 64 k-pair rows (128 k) starting at 64 by.  Each block quantizes x
// itself: it reads the whole rows for their absmax (the scale of quant_a),
// then quantizes only its own 128 k into LDS, in the chunk order of the
// unpacked weight (int4.hpp).  A lane takes 4 columns; each of the 4 waves
// takes two groups of 8 k-pair rows, loads them as one dword per row (with
// the non-temporal policy: each weight byte is read once), transposes and
// unpacks them to 16 (code - 8), and accumulates int8 dot
// products of four into int32 per row of x.  The waves' sums meet in LDS and
// the block writes one exact int32 partial per (row, column).  A second
// kernel adds the partials of an output, takes the factor 16 off (>> 4) and
// applies y = fp32(acc) * sx[m] * scale_w[n] (+ bias), rounded once: the same
// arithmetic as the GEMM's epilogue, on the same exact sum, so both paths
// give identical outputs.
#include "common.hpp"
#include "int4.hpp"
#include "launch.hpp"

namespace qlq {

namespace w4s {
constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int COLS = 256;            // columns per block (4 per lane)
constexpr int KPS = 64;              // k-pair rows per block
constexpr int NCK = KPS / 8;         // 16-value chunks per block
constexpr int GPW = NCK / WAVES;     // 8-row groups per wave
constexpr int MAX_M = 8;
static_assert(WAVES == 4, "the absmax and partial-sum joins add four waves");
static_assert(NCK % WAVES == 0 && MAX_M * NCK <= THREADS, "whole 8-row groups per wave; one thread per chunk and row");
}  // namespace w4s

template <typename XT, int MR, bool BYTES>
__global__ void __launch_bounds__(w4s::THREADS)
w4a8_skinny_kernel(const XT* __restrict__ x, int M, int K, const uint8_t* __restrict__ b, int N,
                   int32_t* __restrict__ part, float* __restrict__ sx_out) {
  using namespace w4s;
  __shared__ float red[WAVES][MR];
  __shared__ float scl[MR];
  __shared__ u32x4_v xs[MR][NCK];                       // this block's quantized x chunks
  __shared__ int32_t rsum[WAVES - 1][MR][4][64];        // waves 1..3's sums
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K2 = K / 2;
  const int kp0 = blockIdx.y * KPS;
  const int col = blockIdx.x * COLS + 4 * lane;  // this lane's first column

  // x first (the vector memory counter drains in order, so whatever is
  // waited for first must be issued first): the whole rows for their absmax,
  // and this thread's chunk of the block's own k-range (chunk c holds k =
  // 2 kp0 + 16 c .. + 15), then the weight, which is only needed after the
  // quantization
  float a[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) a[m] = 0.0f;
  for (int k = tid * 16; k < K; k += THREADS * 16) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m >= M) break;
      float e[16];
      load16<XT>(x + (int64_t)m * K + k, e);
#pragma unroll
      for (int i = 0; i < 16; ++i) a[m] = fmaxf(a[m], fabsf(e[i]));
    }
  }
  const int cm = tid / NCK, cc = tid % NCK, ck = 2 * kp0 + 16 * cc;
  const bool chunk = tid < MR * NCK && cm < M && ck < K;
  float ce[16];
  load16<XT>(x + (chunk ? (int64_t)cm * K + ck : 0), ce);

  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b, K2 * N);
  const int lcol = BYTES ? col : min(col, N - 4);
  uint32_t bw[GPW][8];
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int srow = kp0 + 8 * (wid + WAVES * j);
    if (srow < K2) int4::load8<BYTES, kStreamAux>(rb, srow, 0, srow + 8 <= K2, K2, N, N, lcol, bw[j]);
  }

  // quant_a: s = absmax / 127 (1 if 0) per row
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    a[m] = wave_max_dpp(a[m]);
    if (lane == 0) red[wid][m] = a[m];
  }
  __syncthreads();
  if (tid < MR) {
    const float am = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    float s = __fdiv_rn(am, 127.0f);
    if (s == 0.0f) s = 1.0f;
    scl[tid] = s;
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid < M) sx_out[tid] = s;
  }
  __syncthreads();
  // the chunk, quantized in unpacked order (zeros past K and for rows >= M)
  if (tid < MR * NCK) {
    u32x4_v q = {0u, 0u, 0u, 0u};
    if (chunk) {
      const RowDivider dv(scl[cm]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float r = rintf(dv.div(ce[int4::act_slot(4 * i + j)]));
          r = fminf(fmaxf(r, -128.0f), 127.0f);
          word |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * j);
        }
        q[i] = word;
      }
    }
    xs[cm][cc] = q;
  }
  __syncthreads();

  int32_t acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = 0;
#pragma unroll
  for (int j = 0; j < GPW; ++j) {
    const int g = wid + WAVES * j;
    if (kp0 + 8 * g >= K2) break;
    uint32_t lo[4], hi[4];
    int4::transpose4(bw[j][0], bw[j][1], bw[j][2], bw[j][3], lo);
    int4::transpose4(bw[j][4], bw[j][5], bw[j][6], bw[j][7], hi);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_v w = int4::unpack16(lo[c], hi[c]);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const u32x4_v xq = xs[m][g];
        int32_t t = acc[m][c];
        t = __builtin_amdgcn_sdot4((int)w[0], (int)xq[0], t, false);
        t = __builtin_amdgcn_sdot4((int)w[1], (int)xq[1], t, false);
        t = __builtin_amdgcn_sdot4((int)w[2], (int)xq[2], t, false);
        t = __builtin_amdgcn_sdot4((int)w[3], (int)xq[3], t, false);
        acc[m][c] = t;
      }
    }
  }

  if (wid != 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) rsum[wid - 1][m][c][lane] = acc[m][c];
  }
  __syncthreads();
  if (wid != 0) return;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] += rsum[0][m][c][lane] + rsum[1][m][c][lane] + rsum[2][m][c][lane];
    int32_t* dst = part + ((int64_t)blockIdx.y * M + m) * N;
    if (!BYTES && col + 3 < N) {
      *reinterpret_cast<i32x4_v*>(dst + col) = i32x4_v{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (col + c < N) dst[col + c] = acc[m][c];
    }
  }
}

// y[m, n] = fp32(sum_s part[s, m, n] >> 4) * sx[m] * sw[n] (+ bias[n]).  A
// block takes 64 outputs; its four waves add every fourth split (eight loads
// in flight per lane) and meet in LDS.
template <typename OT>
__global__ void __launch_bounds__(256)
w4a8_finalize_kernel(const int32_t* __restrict__ part, int S, int M, int N, const float* __restrict__ sx,
                     const float* __restrict__ sw, const OT* __restrict__ bias, OT* __restrict__ y) {
  __shared__ int32_t red[3][64];
  const int t = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t MN = (int64_t)M * N;
  const int64_t i = (int64_t)blockIdx.x * 64 + t;
  const bool in = i < MN;
  int32_t acc = 0;
  if (in) {
    const int32_t* p = part + i;
#pragma unroll 8
    for (int s = q; s < S; s += 4) acc += p[s * MN];
  }
  if (q != 0) red[q - 1][t] = acc;
  __syncthreads();
  if (q != 0 || !in) return;
  acc += red[0][t] + red[1][t] + red[2][t];
  const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
  float v = ((float)(acc >> 4) * sx[m]) * sw[n];
  if (bias) v = v + Elem<OT>::load(bias, n);
  Elem<OT>::store(y, i, v);
}

static int64_t skinny_splits(int64_t K) { return cdiv(K / 2, w4s::KPS); }

size_t w4a8_skinny_workspace(int64_t M, int64_t K, int64_t N) {
  const size_t part = (size_t)skinny_splits(K) * (size_t)M * (size_t)N * sizeof(int32_t);
  return ((part + 255) & ~(size_t)255) + (size_t)M * sizeof(float);
}

template <typename XT>
static void skinny_launch(const XT* x, int M, int K, const uint8_t* b, int N, int32_t* part, float* sx,
                          hipStream_t s) {
  const dim3 grid((unsigned)cdiv(N, w4s::COLS), (unsigned)skinny_splits(K)), block(w4s::THREADS);
#define QLQ_SK(MR, BY) \
  hipLaunchKernelGGL((w4a8_skinny_kernel<XT, MR, BY>), grid, block, 0, s, x, M, K, b, N, part, sx)
  const bool by = N % 4 != 0;
  if (M == 1) { if (by) QLQ_SK(1, true); else QLQ_SK(1, false); }
  else if (M == 2) { if (by) QLQ_SK(2, true); else QLQ_SK(2, false); }
  else if (M <= 4) { if (by) QLQ_SK(4, true); else QLQ_SK(4, false); }
  else { if (by) QLQ_SK(8, true); else QLQ_SK(8, false); }
#undef QLQ_SK
}

hipError_t launch_w4a8_skinny(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* b, int64_t N,
                              const float* sw, const void* bias, void* y, void* workspace, hipStream_t s) {
  int32_t* part = (int32_t*)workspace;
  const size_t pbytes = (size_t)skinny_splits(K) * (size_t)M * (size_t)N * sizeof(int32_t);
  float* sx = (float*)((char*)workspace + ((pbytes + 255) & ~(size_t)255));
  const int m = (int)M, k = (int)K, n = (int)N, S = (int)skinny_splits(K);
  const dim3 fgrid((unsigned)cdiv(M * N, 64)), fblock(256);
  if (x_dtype == BF16) {
    skinny_launch<bf16_t>((const bf16_t*)x, m, k, b, n, part, sx, s);
    hipLaunchKernelGGL(w4a8_finalize_kernel<bf16_t>, fgrid, fblock, 0, s, part, S, m, n, sx, sw,
                       (const bf16_t*)bias, (bf16_t*)y);
  } else {
    skinny_launch<f16_t>((const f16_t*)x, m, k, b, n, part, sx, s);
    hipLaunchKernelGGL(w4a8_finalize_kernel<f16_t>, fgrid, fblock, 0, s, part, S, m, n, sx, sw,
                       (const f16_t*)bias, (f16_t*)y);
  }
  return hipGetLastError();
}

}  // namespace qlq
