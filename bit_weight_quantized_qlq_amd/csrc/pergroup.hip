// Per-group int8 linear, M == 1 branch: y[n] = sum_g s[g, n] *
// sum_{k in g} x[k] w[n, k] (+ bias[n]) with x kept in floating point and
// each weight dequantized as it is used.
//
// "cider/ops.py": pergroup_linear (int8 weights [N, K] quantized per group
// of group_size input values, scales [num_groups, N] stored transposed, the
// M == 1 branch computes a matrix-vector product with float activations and
// on-the-fly weight dequantization).  The M > 1 branch quantizes the
// activations and runs the int8 GEMM with per-group rescaling (int8.hip).
//
// One wave per output row; lane l covers the 16-byte chunks l, l+64, ... of
// the row (a chunk lies inside one group: group_size >= 64).  x is staged
// once per block in LDS as fp32, split into four quarter arrays so that
// consecutive lanes read consecutive 16-byte units, with per-chunk sums.  A
// weight byte w becomes float through the unsigned byte conversion of
// w ^ 0x80 = w + 128, and sum x (w + 128) - 128 sum x = sum x w.
#include "common.hpp"
#include "launch.hpp"

namespace qlq {

namespace pgmv {
constexpr int WAVES = 16, THREADS = 64 * WAVES;
constexpr int KMAX = 16384;   // x staged whole in LDS
constexpr int BATCH = 4;      // chunks a lane loads before computing
}  // namespace pgmv

template <typename XT>
__global__ void __launch_bounds__(pgmv::THREADS)
pergroup_mv_kernel(const XT* __restrict__ x, int K, const int8_t* __restrict__ w,
                   const float* __restrict__ scale, int N, int G, const XT* __restrict__ bias,
                   XT* __restrict__ y) {
  using namespace pgmv;
  __shared__ __attribute__((aligned(16))) float4 xq4[4][KMAX / 16];  // quarter q of chunk c
  __shared__ float xsum[KMAX / 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int nch = K / 16;
  const int n = blockIdx.x * WAVES + (tid >> 6);
  const int nr = n < N ? n : N - 1;
  const int8_t* wr = w + (int64_t)nr * K;

  // the first batch of weights and scales goes out before x is staged
  uint4 wv[BATCH];
  float sc[BATCH];
#define QLQ_MV_LOAD(BASE)                                                   \
  do {                                                                      \
    _Pragma("unroll") for (int b = 0; b < BATCH; ++b) {                     \
      const int c_ = min((BASE) + 64 * b, nch - 1);                         \
      wv[b] = stream_u4(wr + 16 * c_); /* read once: streaming loads */   \
      sc[b] = scale[(int64_t)(16 * c_ / G) * N + nr]; /* lines shared */    \
    }                                                                       \
  } while (0)
  QLQ_MV_LOAD(lane);

  for (int c = tid; c < nch; c += THREADS) {
    float e[16];
    load16<XT>(x + 16 * c, e);
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xq4[q][c] = make_float4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
      t += (e[4 * q] + e[4 * q + 1]) + (e[4 * q + 2] + e[4 * q + 3]);
    }
    xsum[c] = t;
  }
  __syncthreads();
  if (n >= N) return;

  float acc = 0.0f;
  for (int base = lane; base < nch; base += 64 * BATCH) {
    if (base != lane) QLQ_MV_LOAD(base);
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = base + 64 * b;
      if (c >= nch) break;
      const uint32_t wd[4] = {wv[b].x ^ 0x80808080u, wv[b].y ^ 0x80808080u, wv[b].z ^ 0x80808080u,
                              wv[b].w ^ 0x80808080u};
      float p = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 xv = xq4[q][c];
        // (float)(byte j): one unsigned-byte conversion each
        p = __builtin_fmaf(xv.x, (float)(wd[q] & 0xFFu), p);
        p = __builtin_fmaf(xv.y, (float)((wd[q] >> 8) & 0xFFu), p);
        p = __builtin_fmaf(xv.z, (float)((wd[q] >> 16) & 0xFFu), p);
        p = __builtin_fmaf(xv.w, (float)(wd[q] >> 24), p);
      }
      acc = __builtin_fmaf(sc[b], __builtin_fmaf(-128.0f, xsum[c], p), acc);
    }
  }
#undef QLQ_MV_LOAD
  acc = wave_sum_dpp(acc);
  if (lane == 0) {
    if (bias) acc = acc + Elem<XT>::load(bias, n);
    Elem<XT>::store(y, n, acc);
  }
}

hipError_t launch_pergroup_mv(const void* x, int x_dtype, int64_t K, const int8_t* w, const float* scale,
                              int64_t N, int group_size, const void* bias, void* y, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(N, pgmv::WAVES)), block(pgmv::THREADS);
  if (x_dtype == BF16)
    hipLaunchKernelGGL(pergroup_mv_kernel<bf16_t>, grid, block, 0, s, (const bf16_t*)x, (int)K, w, scale,
                       (int)N, group_size, (const bf16_t*)bias, (bf16_t*)y);
  else
    hipLaunchKernelGGL(pergroup_mv_kernel<f16_t>, grid, block, 0, s, (const f16_t*)x, (int)K, w, scale,
                       (int)N, group_size, (const f16_t*)bias, (f16_t*)y);
  return hipGetLastError();
}

}  // namespace qlq
