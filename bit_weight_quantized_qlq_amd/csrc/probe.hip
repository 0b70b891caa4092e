// Read-rate probes for the measurement of the HBM-bound kernels: what a launch
// that only reads (and does no arithmetic on) the same bytes achieves.
//
//  * qlq_probe_read_rows: the byte pattern of the decode GEMV on 4-bit codes
//    at one x row in the launch shape the GEMV takes for that N (one wave per
//    output row in blocks of 16 waves; from N = 12288 on, two rows per wave
//    in blocks of 8), each lane loading its NCH 16-byte code chunks (chunk
//    lane + 64 i, so a load instruction covers 1 KiB of contiguous codes)
//    through one buffer descriptor per row and the 16-bit scale and bias of
//    each chunk's group, all with the non-temporal policy, after the block's x loads; x
//    staged in LDS behind a barrier.  Every loaded word is XOR-folded and one
//    word per row is stored, so no load can be dropped.
//  * qlq_probe_read_flat: a plain read of a contiguous buffer, four 16-byte
//    non-temporal loads per thread, one word stored per block.
//
// These kernels are measurement tools, not part of the layer: they compute
// nothing of it.
#include "common.hpp"

namespace qlq {
namespace {

constexpr int64_t kProbeLargeN = 12288;  // the decode GEMV's large-N launch shape from here

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v ^= (uint32_t)__shfl_xor((int)v, d, kWave);
  return v;
}

template <int NCH, int G, int R, int WPB>
__global__ void __launch_bounds__(64 * WPB)
read_rows_kernel(const uint16_t* __restrict__ x, int K, const uint32_t* __restrict__ packed,
                 const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int N,
                 uint32_t* __restrict__ out) {
  constexpr int THREADS = 64 * WPB;
  constexpr int XROW = 64 * NCH * 4;                   // 16-byte x units the block stages
  constexpr int XU4 = (XROW + THREADS - 1) / THREADS;
  constexpr int CPG = G / 32;                          // 32-code chunks per group
  __shared__ uint4 xs[XROW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int n0 = (blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(tid >> 6)) * R;
  const int cpr = K / 32, wpr = K / 8, gpr = K / G, kx = K / 8;

  uint4 xr[XU4];
#pragma unroll
  for (int i = 0; i < XU4; ++i) {
    const int u = tid + THREADS * i;
    xr[i] = u < kx ? reinterpret_cast<const uint4*>(x)[u] : make_uint4(0, 0, 0, 0);
  }
  u32x4_v w[R][NCH];
  uint16_t s[R][NCH], b[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int nn = n0 + r < N ? n0 + r : N - 1;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(packed + (int64_t)nn * wpr, wpr * 4);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = i * 64 + lane;  // the GEMV's chunks: lane + 64 i, each in its own group
      c = c < cpr ? c : cpr - 1;
      w[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, c * 16, 0, kStreamAux);
      s[r][i] = stream_load(scales + (int64_t)nn * gpr + c / CPG);
      b[r][i] = stream_load(biases + (int64_t)nn * gpr + c / CPG);
    }
  }
#pragma unroll
  for (int i = 0; i < XU4; ++i) {
    const int u = tid + THREADS * i;
    if (u < XROW) xs[u] = xr[i];
  }
  __syncthreads();
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint4 xv = xs[(i * 64 + lane) % XROW];
      v ^= w[r][i][0] ^ w[r][i][1] ^ w[r][i][2] ^ w[r][i][3] ^ xv.x ^ xv.y ^ xv.z ^ xv.w ^ s[r][i] ^
           ((uint32_t)b[r][i] << 16);
    }
  v = wave_xor(v);
  if (lane == 0 && n0 < N) out[n0] = v;
}

constexpr int kFlatThreads = 256, kFlatUnits = 4;

__global__ void __launch_bounds__(kFlatThreads)
read_flat_kernel(const u32x4_v* __restrict__ p, int64_t units, uint32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kFlatThreads * kFlatUnits + threadIdx.x;
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < kFlatUnits; ++i) {
    const int64_t u = base + (int64_t)i * kFlatThreads;
    if (u < units) {
      const u32x4_v a = stream_load(p + u);
      v ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
  }
  v = wave_xor(v);
  __shared__ uint32_t red[kFlatThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace
}  // namespace qlq

#define QLQ_PROBE_API extern "C" __attribute__((visibility("default")))

// Bytes read: N rows of K/2 code bytes and 2*(K/G)*2 scale and bias bytes,
// plus K*2 bytes of x per block.  out: N uint32.  K % 32 == 0, K/32 <= 256
// (at most 4 chunks per lane), G in {32, 64, 128}, every byte range below
// 2^31.  Returns a hipError_t code (0 on success), or -1 on invalid sizes.
QLQ_PROBE_API int qlq_probe_read_rows(const void* x, int64_t K, const void* packed, const void* scales,
                                      const void* biases, int64_t N, int group_size, void* out, void* stream) {
  using namespace qlq;
  if (!x || !packed || !scales || !biases || !out || N < 1 || K < 32 || K % 32 || K % group_size ||
      K / 32 > 256 || N * K >= ((int64_t)1 << 31))
    return -1;
  const int64_t nch = cdiv(K / 32, 64);
  const bool large = N >= kProbeLargeN;
  const int R = large ? 2 : 1, WPB = large ? 8 : 16;
  const dim3 grid((unsigned)cdiv(cdiv(N, R), WPB)), block(64 * WPB);
  hipStream_t s = (hipStream_t)stream;
#define QLQ_PROBE_ROWS(NCH_, G_)                                                                                 \
  do {                                                                                                           \
    if (large)                                                                                                   \
      hipLaunchKernelGGL((read_rows_kernel<NCH_, G_, 2, 8>), grid, block, 0, s, (const uint16_t*)x, (int)K,      \
                         (const uint32_t*)packed, (const uint16_t*)scales, (const uint16_t*)biases, (int)N,      \
                         (uint32_t*)out);                                                                        \
    else                                                                                                         \
      hipLaunchKernelGGL((read_rows_kernel<NCH_, G_, 1, 16>), grid, block, 0, s, (const uint16_t*)x, (int)K,     \
                         (const uint32_t*)packed, (const uint16_t*)scales, (const uint16_t*)biases, (int)N,      \
                         (uint32_t*)out);                                                                        \
  } while (0)
#define QLQ_PROBE_G(NCH_)                                   \
  do {                                                      \
    if (group_size == 32) QLQ_PROBE_ROWS(NCH_, 32);         \
    else if (group_size == 64) QLQ_PROBE_ROWS(NCH_, 64);    \
    else if (group_size == 128) QLQ_PROBE_ROWS(NCH_, 128);  \
    else return -1;                                         \
  } while (0)
  if (nch == 1) QLQ_PROBE_G(1);
  else if (nch == 2) QLQ_PROBE_G(2);
  else if (nch <= 4) QLQ_PROBE_G(4);
  else return -1;
#undef QLQ_PROBE_G
#undef QLQ_PROBE_ROWS
  return (int)hipGetLastError();
}

// Blocks of qlq_probe_read_flat for `bytes` (the size of its out array, in uint32).
QLQ_PROBE_API int64_t qlq_probe_read_flat_blocks(int64_t bytes) {
  return qlq::cdiv(bytes / 16, (int64_t)qlq::kFlatThreads * qlq::kFlatUnits);
}

// Reads `bytes` (a multiple of 16) starting at p (16-byte aligned).
QLQ_PROBE_API int qlq_probe_read_flat(const void* p, int64_t bytes, void* out, void* stream) {
  using namespace qlq;
  if (!p || !out || bytes < 16 || bytes % 16 || ((uintptr_t)p & 15)) return -1;
  const int64_t blocks = qlq_probe_read_flat_blocks(bytes);
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(read_flat_kernel, dim3((unsigned)blocks), dim3(kFlatThreads), 0, (hipStream_t)stream,
                     (const u32x4_v*)p, bytes / 16, (uint32_t*)out);
  return (int)hipGetLastError();
}
