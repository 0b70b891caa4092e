// Bit-exact quantize / pack / unpack / dequantize kernels.
//
// Affine format: "Struct QuantizedLinear" (nuvec-nn docs), Fields and
// from_linear; formula from the MLX affine docstring of pergroup_linear in
// "cider/ops.py".  Ternary format: make_bitlinear_kernel in
// "mlx-lm/mlx_lm/models/bitlinear_layers.py".  Row int8 quantizer:
// quantize_weight_int8 (absmax branch) in "cider/ops.py".
//
// Every floating-point step that decides an integer is a single IEEE fp32
// operation with round-to-nearest-even (__fsub_rn, __fdiv_rn, rintf), so the
// codes equal those of an fp32 reference bit for bit.  The packing kernels
// run offline and favour plain indexing; the row int8 quantizer also
// quantizes activations on the W8A8 forward path and is written for
// bandwidth (one wave per row, the row held in registers).
#include "common.hpp"
#include "int4.hpp"
#include "launch.hpp"

namespace qlq {

// ---------------------------------------------------------------- affine pack
// One thread per (row n, group g).  The thread reads its G weights, forms the
// fp32 min/max, the stored scale and bias, and writes the group's G/32 units
// of BITS words (32 codes each; G is a multiple of 32).
template <int BITS, typename SB>
__global__ void __launch_bounds__(256)
affine_pack_kernel(const float* __restrict__ w, int64_t N, int64_t K, int G,
                   uint32_t* __restrict__ packed, SB* __restrict__ scales,
                   SB* __restrict__ biases, int* __restrict__ err) {
  const int64_t ngroups = K / G;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= N * ngroups) return;
  const int64_t n = t / ngroups, g = t % ngroups;
  const float* wg = w + n * K + g * G;
  constexpr uint32_t qmax = (1u << BITS) - 1u;

  float mn = wg[0], mx = wg[0];
  bool finite = true;
  for (int i = 0; i < G; i += 4) {
    float4 v = *reinterpret_cast<const float4*>(wg + i);
    finite &= is_finite_f32(v.x) & is_finite_f32(v.y) & is_finite_f32(v.z) & is_finite_f32(v.w);
    mn = fminf(mn, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
    mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  // scale = (max - min) / (2^b - 1), bias = min; both rounded to the storage dtype
  const float s32 = __fdiv_rn(__fsub_rn(mx, mn), (float)qmax);
  float s = Elem<SB>::round(s32);
  const float b = Elem<SB>::round(mn);
  finite &= is_finite_f32(s) & is_finite_f32(b);
  if (!finite) atomicOr(err, 1);
  if (s == 0.0f) s = 1.0f;
  Elem<SB>::store(scales, t, s);
  Elem<SB>::store(biases, t, b);

  uint32_t* out = packed + (n * K + g * G) / 32 * BITS;
  for (int u = 0; u < G / 32; ++u) {
    uint32_t wd[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) wd[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float q = rintf(__fdiv_rn(__fsub_rn(wg[32 * u + j], b), s));
      q = fminf(fmaxf(q, 0.0f), (float)qmax);
      unit_put<BITS>(wd, j, (uint32_t)q);
    }
#pragma unroll
    for (int i = 0; i < BITS; ++i) out[u * BITS + i] = wd[i];
  }
}

template <int BITS>
static hipError_t pack_dispatch_sb(const float* w, int64_t N, int64_t K, int G, uint32_t* packed,
                                   void* scales, void* biases, int sb, int* err, hipStream_t s) {
  const int64_t total = N * (K / G);
  dim3 grid((unsigned)cdiv(total, 256)), block(256);
  switch (sb) {
    case F32:
      hipLaunchKernelGGL((affine_pack_kernel<BITS, float>), grid, block, 0, s, w, N, K, G, packed,
                         (float*)scales, (float*)biases, err);
      break;
    case BF16:
      hipLaunchKernelGGL((affine_pack_kernel<BITS, bf16_t>), grid, block, 0, s, w, N, K, G, packed,
                         (bf16_t*)scales, (bf16_t*)biases, err);
      break;
    default:
      hipLaunchKernelGGL((affine_pack_kernel<BITS, f16_t>), grid, block, 0, s, w, N, K, G, packed,
                         (f16_t*)scales, (f16_t*)biases, err);
      break;
  }
  return hipGetLastError();
}

// every affine bit width the layer supports
#define QLQ_AFFINE_BITS_SWITCH(bits, CALL) \
  switch (bits) {                          \
    case 1: return CALL(1);                \
    case 2: return CALL(2);                \
    case 3: return CALL(3);                \
    case 4: return CALL(4);                \
    case 5: return CALL(5);                \
    case 6: return CALL(6);                \
    default: return CALL(8);               \
  }

hipError_t launch_affine_pack(const float* w, int64_t N, int64_t K, int bits, int G,
                              uint32_t* packed, void* scales, void* biases, int sb_dtype,
                              int* err_flag, hipStream_t s) {
#define QLQ_CALL(B) pack_dispatch_sb<B>(w, N, K, G, packed, scales, biases, sb_dtype, err_flag, s)
  QLQ_AFFINE_BITS_SWITCH(bits, QLQ_CALL)
#undef QLQ_CALL
}

// -------------------------------------------------------------- affine unpack
// The rows of a packed matrix are whole words, so all N*K codes form one
// stream; a thread takes one unit of 32 codes (the last may be partial).
// VEC: codes 16-byte aligned and N*K % 32 == 0, two 16-byte stores per unit.
template <int BITS, bool VEC>
__global__ void __launch_bounds__(256)
affine_unpack_kernel(const uint32_t* __restrict__ packed, int64_t ncodes, uint8_t* __restrict__ codes) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t k0 = u * 32;
  if (k0 >= ncodes) return;
  const int64_t nwords = ncodes * BITS / 32;
  uint32_t wd[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) wd[i] = u * BITS + i < nwords ? packed[u * BITS + i] : 0u;
  if constexpr (VEC) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[i] = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[i] |= unit_code<BITS>(wd, 4 * i + j) << (8 * j);
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + k0);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (k0 + j < ncodes) codes[k0 + j] = (uint8_t)unit_code<BITS>(wd, j);
  }
}

template <int BITS>
static hipError_t unpack_dispatch(const uint32_t* packed, int64_t ncodes, uint8_t* codes, hipStream_t s) {
  dim3 grid((unsigned)cdiv(cdiv(ncodes, 32), 256)), block(256);
  if (ncodes % 32 == 0 && ((uintptr_t)codes & 15) == 0)
    hipLaunchKernelGGL((affine_unpack_kernel<BITS, true>), grid, block, 0, s, packed, ncodes, codes);
  else
    hipLaunchKernelGGL((affine_unpack_kernel<BITS, false>), grid, block, 0, s, packed, ncodes, codes);
  return hipGetLastError();
}

hipError_t launch_affine_unpack(const uint32_t* packed, int64_t N, int64_t K, int bits,
                                uint8_t* codes, hipStream_t s) {
#define QLQ_CALL(B) unpack_dispatch<B>(packed, N * K, codes, s)
  QLQ_AFFINE_BITS_SWITCH(bits, QLQ_CALL)
#undef QLQ_CALL
}

// ------------------------------------------------ affine codes to nibbles
// Codes of at most 4 bits rewritten in the 4-bit packed layout (code k at
// bits 4 (k mod 8) of word k / 8).  Rows are whole words in both layouts, so
// the N*K codes are one stream on both sides; a thread takes one unit of 32
// codes and writes its four words (N*K % 32 == 0).
template <int BITS>
__global__ void __launch_bounds__(256)
affine_to_nibbles_kernel(const uint32_t* __restrict__ packed, int64_t units, uint4* __restrict__ out) {
  static_assert(BITS <= 4, "codes must fit a nibble");
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  uint32_t wd[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) wd[i] = packed[u * BITS + i];
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[i] |= unit_code<BITS>(wd, 8 * i + j) << (4 * j);
  }
  out[u] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_affine_to_nibbles(const uint32_t* packed, int64_t N, int64_t K, int bits,
                                    uint32_t* out, hipStream_t s) {
  const int64_t units = N * K / 32;
  dim3 grid((unsigned)cdiv(units, 256)), block(256);
  if (bits == 1)
    hipLaunchKernelGGL(affine_to_nibbles_kernel<1>, grid, block, 0, s, packed, units, (uint4*)out);
  else if (bits == 2)
    hipLaunchKernelGGL(affine_to_nibbles_kernel<2>, grid, block, 0, s, packed, units, (uint4*)out);
  else if (bits == 3)
    hipLaunchKernelGGL(affine_to_nibbles_kernel<3>, grid, block, 0, s, packed, units, (uint4*)out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ----------------------------------------------------------- affine dequantize
// w = fma(scale, q, bias): one rounding of the exact value, in fp32.  One
// thread per unit of 32 codes (a unit never straddles a group: G % 32 == 0).
template <int BITS, typename SB>
__global__ void __launch_bounds__(256)
affine_dequant_kernel(const uint32_t* __restrict__ packed, const SB* __restrict__ scales,
                      const SB* __restrict__ biases, int64_t N, int64_t K, int G,
                      float* __restrict__ w) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t units_per_row = K / 32;
  if (t >= N * units_per_row) return;
  const int64_t n = t / units_per_row, k0 = (t % units_per_row) * 32;
  const int64_t gi = n * (K / G) + k0 / G;
  const float s = Elem<SB>::load(scales, gi), b = Elem<SB>::load(biases, gi);
  uint32_t wd[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) wd[i] = packed[t * BITS + i];
#pragma unroll
  for (int j = 0; j < 32; ++j) w[n * K + k0 + j] = __fmaf_rn(s, (float)unit_code<BITS>(wd, j), b);
}

template <int BITS>
static hipError_t dequant_dispatch_sb(const uint32_t* packed, const void* scales, const void* biases,
                                      int sb, int64_t N, int64_t K, int G, float* w, hipStream_t s) {
  const int64_t total = N * (K / 32);
  dim3 grid((unsigned)cdiv(total, 256)), block(256);
  switch (sb) {
    case F32:
      hipLaunchKernelGGL((affine_dequant_kernel<BITS, float>), grid, block, 0, s, packed,
                         (const float*)scales, (const float*)biases, N, K, G, w);
      break;
    case BF16:
      hipLaunchKernelGGL((affine_dequant_kernel<BITS, bf16_t>), grid, block, 0, s, packed,
                         (const bf16_t*)scales, (const bf16_t*)biases, N, K, G, w);
      break;
    default:
      hipLaunchKernelGGL((affine_dequant_kernel<BITS, f16_t>), grid, block, 0, s, packed,
                         (const f16_t*)scales, (const f16_t*)biases, N, K, G, w);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_affine_dequant(const uint32_t* packed, const void* scales, const void* biases,
                                 int sb_dtype, int64_t N, int64_t K, int bits, int G, float* w,
                                 hipStream_t s) {
#define QLQ_CALL(B) dequant_dispatch_sb<B>(packed, scales, biases, sb_dtype, N, K, G, w, s)
  QLQ_AFFINE_BITS_SWITCH(bits, QLQ_CALL)
#undef QLQ_CALL
}

// ---------------------------------------------------------------- ternary pack
// byte[r, k] = sum_j (t[r + j*R, k] + 1) << 2j  with R = N/4.
__global__ void __launch_bounds__(256)
ternary_pack_kernel(const int8_t* __restrict__ t, int64_t R, int64_t K, uint8_t* __restrict__ packed,
                    int* __restrict__ err) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= R * K) return;
  const int64_t r = i / K, k = i % K;
  uint32_t byte = 0;
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = t[(r + j * R) * K + k];
    ok &= (v >= -1) & (v <= 1);
    byte |= (uint32_t)((v + 1) & 3) << (2 * j);
  }
  if (!ok) atomicOr(err, 1);
  packed[i] = (uint8_t)byte;
}

hipError_t launch_ternary_pack(const int8_t* t, int64_t N, int64_t K, uint8_t* packed, int* err_flag,
                               hipStream_t s) {
  const int64_t R = N / 4;
  dim3 grid((unsigned)cdiv(R * K, 256)), block(256);
  hipLaunchKernelGGL(ternary_pack_kernel, grid, block, 0, s, t, R, K, packed, err_flag);
  return hipGetLastError();
}

// ------------------------------------------------------ row int8 quantization
// One 256-thread block per row.  Pass 1: exact fp32 absmax (block reduction).
// Pass 2: q = clamp(rint(v / s), -128, 127) with s = a / 127 (1 if 0).
// Each thread handles 16 consecutive elements per step (K % 16 == 0).

// Output order inside each 16-byte chunk: k order, or (NIB) the order packed
// int4 bytes unpack to (int4::act_slot).
template <bool NIB>
__host__ __device__ constexpr int chunk_src(int s) {
  return NIB ? int4::act_slot(s) : s;
}

template <typename T, bool NIB>
__global__ void __launch_bounds__(256)
quantize_rows_int8_kernel(const T* __restrict__ v, int64_t K, int8_t* __restrict__ q,
                          float* __restrict__ scale) {
  __shared__ float red[256 / kWave];
  const int64_t row = blockIdx.x;
  const T* vr = v + row * K;
  int8_t* qr = q + row * K;
  const int tid = threadIdx.x;

  float a = 0.0f;
  for (int64_t k = (int64_t)tid * 16; k < K; k += 256 * 16) {
    float e[16];
    load16<T>(vr + k, e);
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(e[i]));
  }
  a = wave_max(a);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = __fdiv_rn(a, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (tid == 0) scale[row] = s;
  const RowDivider dv(s);

  for (int64_t k = (int64_t)tid * 16; k < K; k += 256 * 16) {
    float e[16];
    load16<T>(vr + k, e);
    uint32_t packed4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = int8_code_bits(dv.div(e[chunk_src<NIB>(4 * i + j)]));
      packed4[i] = pack_low_bytes(c[0], c[1], c[2], c[3]);
    }
    *reinterpret_cast<uint4*>(qr + k) = make_uint4(packed4[0], packed4[1], packed4[2], packed4[3]);
  }
}

// Register-resident variant for K <= 64 * EPT: one wave per row, each lane
// keeps its EPT consecutive elements (16-byte loads) in registers, so the row
// is read once; max by DPP; no block barrier.
template <typename T, int EPT, bool NIB>
__global__ void __launch_bounds__(256)
quantize_rows_int8_wave_kernel(const T* __restrict__ v, int R, int K, int8_t* __restrict__ q,
                               float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const T* vr = v + (int64_t)row * K;
  constexpr int G16 = EPT / 16;  // groups of 16 elements per lane
  float e[EPT];
  bool in[G16];
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    const int k = (g * 64 + lane) * 16;  // lanes interleave 16-element groups: coalesced
    in[g] = k < K;
    float t[16];
    load16<T>(vr + (in[g] ? k : 0), t);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[g * 16 + i] = in[g] ? t[i] : 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) a = fmaxf(a, fabsf(e[i]));
  a = wave_max_dpp(a);
  float s = __fdiv_rn(a, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (lane == 0) scale[row] = s;
  const RowDivider dv(s);
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    if (!in[g]) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = int8_code_bits(dv.div(e[g * 16 + chunk_src<NIB>(4 * i + j)]));
      w[i] = pack_low_bytes(c[0], c[1], c[2], c[3]);
    }
    *reinterpret_cast<uint4*>(q + (int64_t)row * K + (g * 64 + lane) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One 256-thread block per row, EPT elements per thread (16-element groups
// interleaved across the block: coalesced 16-byte loads and stores); the row
// stays in registers between the max and the quantization.
template <typename T, int EPT, bool NIB>
__global__ void __launch_bounds__(256)
quantize_rows_int8_block_kernel(const T* __restrict__ v, int K, int8_t* __restrict__ q,
                                float* __restrict__ scale) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const T* vr = v + row * K;
  constexpr int G16 = EPT / 16;
  float e[EPT];
  bool in[G16];
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    const int k = (g * 256 + tid) * 16;
    in[g] = k < K;
    float t[16];
    load16<T>(vr + (in[g] ? k : 0), t);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[g * 16 + i] = in[g] ? t[i] : 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < EPT; ++i) a = fmaxf(a, fabsf(e[i]));
  a = wave_max_dpp(a);
  if ((tid & 63) == 0) red[tid >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = __fdiv_rn(a, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (tid == 0) scale[row] = s;
  const RowDivider dv(s);
#pragma unroll
  for (int g = 0; g < G16; ++g) {
    if (!in[g]) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = int8_code_bits(dv.div(e[g * 16 + chunk_src<NIB>(4 * i + j)]));
      w[i] = pack_low_bytes(c[0], c[1], c[2], c[3]);
    }
    *reinterpret_cast<uint4*>(q + row * K + (g * 256 + tid) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The row scales of the row quantizer alone (s = absmax / 127, 1 if 0):
// one wave per row, four 16-element groups per lane in flight.  The codes
// are left to the consumer, which divides by these same scales.
template <typename T>
__global__ void __launch_bounds__(256)
row_scales_int8_kernel(const T* __restrict__ v, int R, int K, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const T* vr = v + (int64_t)row * K;
  float a = 0.0f;
#pragma unroll 4
  for (int k = lane * 16; k < K; k += 64 * 16) {  // K % 16 == 0
    float e[16];
    load16<T>(vr + k, e);
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(e[i]));
  }
  a = wave_max_dpp(a);
  float s = __fdiv_rn(a, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (lane == 0) scale[row] = s;
}

hipError_t launch_row_scales_int8(const void* v, int v_dtype, int64_t R, int64_t K, float* scale, hipStream_t s) {
  const dim3 grid((unsigned)cdiv(R, 4)), block(256);
  const int r = (int)R, k = (int)K;
  switch (v_dtype) {
    case F32: hipLaunchKernelGGL(row_scales_int8_kernel<float>, grid, block, 0, s, (const float*)v, r, k, scale); break;
    case BF16: hipLaunchKernelGGL(row_scales_int8_kernel<bf16_t>, grid, block, 0, s, (const bf16_t*)v, r, k, scale); break;
    default: hipLaunchKernelGGL(row_scales_int8_kernel<f16_t>, grid, block, 0, s, (const f16_t*)v, r, k, scale); break;
  }
  return hipGetLastError();
}

// Per-group symmetric int8 quantization: w [N, K] -> q [N, K] int8 and
// scale [K/G, N] fp32 (group-major).  One wave per (row, 1024-element
// chunk): lane l holds elements 16l .. 16l+15 of the chunk, so a group is G/16
// consecutive lanes and its absmax is a shuffle reduction over them.  Same
// rule as the row quantizer, per group.
template <typename T, int G>
__global__ void __launch_bounds__(256)
quantize_groups_int8_kernel(const T* __restrict__ w, int N, int K, int8_t* __restrict__ q,
                            float* __restrict__ scale) {
  static_assert(G % 16 == 0 && 1024 % G == 0 && G / 16 <= 64, "group shape");
  const int lane = threadIdx.x & 63;
  const int chunks = (K + 1023) / 1024;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (int64_t)N * chunks) return;
  const int n = (int)(wv / chunks), ch = (int)(wv % chunks);
  const int k = ch * 1024 + lane * 16;
  const bool in = k < K;
  float e[16];
  load16<T>(w + (int64_t)n * K + (in ? k : 0), e);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, in ? fabsf(e[i]) : 0.0f);
#pragma unroll
  for (int o = 1; o < G / 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
  float s = __fdiv_rn(a, 127.0f);
  if (s == 0.0f) s = 1.0f;
  if (!in) return;
  if (lane % (G / 16) == 0) scale[(int64_t)(k / G) * N + n] = s;
  const RowDivider dv(s);
  uint32_t wd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = int8_code_bits(dv.div(e[4 * i + j]));
    wd[i] = pack_low_bytes(c[0], c[1], c[2], c[3]);
  }
  *reinterpret_cast<uint4*>(q + (int64_t)n * K + k) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

template <typename T>
static void quant_groups_launch(const void* w, int64_t N, int64_t K, int G, int8_t* q, float* scale,
                                hipStream_t s) {
  const dim3 grid((unsigned)cdiv(N * cdiv(K, 1024), 4)), block(256);
  const int n = (int)N, k = (int)K;
  if (G == 64)
    hipLaunchKernelGGL((quantize_groups_int8_kernel<T, 64>), grid, block, 0, s, (const T*)w, n, k, q, scale);
  else if (G == 128)
    hipLaunchKernelGGL((quantize_groups_int8_kernel<T, 128>), grid, block, 0, s, (const T*)w, n, k, q, scale);
  else
    hipLaunchKernelGGL((quantize_groups_int8_kernel<T, 256>), grid, block, 0, s, (const T*)w, n, k, q, scale);
}

hipError_t launch_quantize_groups_int8(const void* w, int w_dtype, int64_t N, int64_t K, int group_size,
                                       int8_t* q, float* scale, hipStream_t s) {
  switch (w_dtype) {
    case F32: quant_groups_launch<float>(w, N, K, group_size, q, scale, s); break;
    case BF16: quant_groups_launch<bf16_t>(w, N, K, group_size, q, scale, s); break;
    default: quant_groups_launch<f16_t>(w, N, K, group_size, q, scale, s); break;
  }
  return hipGetLastError();
}

template <typename T, bool NIB>
static void quant_rows_launch(const void* v, int64_t R, int64_t K, int8_t* q, float* scale, hipStream_t s) {
  // short rows: a wave per row; up to 16384: a block per row (four times the
  // waves, so the per-element work spreads over every SIMD); longer: two
  // passes over the row
  if (K <= 64 * 16) {
    hipLaunchKernelGGL((quantize_rows_int8_wave_kernel<T, 16, NIB>), dim3((unsigned)cdiv(R, 4)), dim3(256), 0, s,
                       (const T*)v, (int)R, (int)K, q, scale);
  } else if (K <= 256 * 64) {
    dim3 grid((unsigned)R), block(256);
    if (K <= 256 * 16)
      hipLaunchKernelGGL((quantize_rows_int8_block_kernel<T, 16, NIB>), grid, block, 0, s, (const T*)v, (int)K, q,
                         scale);
    else if (K <= 256 * 32)
      hipLaunchKernelGGL((quantize_rows_int8_block_kernel<T, 32, NIB>), grid, block, 0, s, (const T*)v, (int)K, q,
                         scale);
    else
      hipLaunchKernelGGL((quantize_rows_int8_block_kernel<T, 64, NIB>), grid, block, 0, s, (const T*)v, (int)K, q,
                         scale);
  } else {
    hipLaunchKernelGGL((quantize_rows_int8_kernel<T, NIB>), dim3((unsigned)R), dim3(256), 0, s, (const T*)v, K, q,
                       scale);
  }
}

hipError_t launch_quantize_rows_int8(const void* v, int v_dtype, int64_t R, int64_t K, int8_t* q,
                                     float* scale, hipStream_t s, bool nibble_order) {
#define QLQ_QR(T) nibble_order ? quant_rows_launch<T, true>(v, R, K, q, scale, s) \
                               : quant_rows_launch<T, false>(v, R, K, q, scale, s)
  switch (v_dtype) {
    case F32: QLQ_QR(float); break;
    case BF16: QLQ_QR(bf16_t); break;
    default: QLQ_QR(f16_t); break;
  }
#undef QLQ_QR
  return hipGetLastError();
}

// ------------------------------------------- row int8 with a percentile clip
// quantize_weight_int8 with clip_percentile: the row's clip is the given
// percentile of |w| (NumPy's linear method, every step in fp32: q = p/100,
// v = (K-1) q, i = floor(v), t = v - i, sorted values a, b at i, i+1, then
// a + (b-a) t for t < 0.5 else b - (b-a)(1-t); v >= K-1 gives the maximum),
// a zero clip falls back to the row's maximum, scale = clip/127 (1 if 0), and
// q = clamp(rint(clamp(w, -clip, clip) / scale), -128, 127).
// One block per row: |w| sorted in LDS by a bitonic network over P2 (the
// next power of two >= K) slots, the tail padded with +inf.
constexpr int kClipThreads = 256;
constexpr int kClipMaxK = 16384;  // 64 KiB of LDS
template <typename T>
__global__ void __launch_bounds__(kClipThreads)
quantize_rows_int8_clip_kernel(const T* __restrict__ v, int K, int P2, float pct, int8_t* __restrict__ q,
                               float* __restrict__ scale) {
  extern __shared__ float srt[];
  __shared__ float clip_s;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const T* vr = v + row * K;
  for (int i = tid; i < P2; i += kClipThreads)
    srt[i] = i < K ? fabsf(Elem<T>::load(vr, i)) : __builtin_inff();
  __syncthreads();
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int pi = tid; pi < P2 / 2; pi += kClipThreads) {
        const int i = ((pi & ~(j - 1)) << 1) | (pi & (j - 1));  // lower slot of the pair
        const int l = i | j;
        const float a = srt[i], b = srt[l];
        if ((a > b) == ((i & k) == 0)) {
          srt[i] = b;
          srt[l] = a;
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) {
    const float qf = __fdiv_rn(pct, 100.0f);
    const float vi = __fmul_rn((float)(K - 1), qf);
    float c;
    if (vi >= (float)(K - 1)) {
      c = srt[K - 1];
    } else {
      const int i = (int)floorf(vi);
      const float t = __fsub_rn(vi, (float)i);
      const float a = srt[i], b = srt[i + 1];
      const float d = __fsub_rn(b, a);
      c = t >= 0.5f ? __fsub_rn(b, __fmul_rn(d, __fsub_rn(1.0f, t))) : __fadd_rn(a, __fmul_rn(d, t));
    }
    if (c == 0.0f) c = srt[K - 1];
    clip_s = c;
    float sc = __fdiv_rn(c, 127.0f);
    if (sc == 0.0f) sc = 1.0f;
    scale[row] = sc;
  }
  __syncthreads();
  const float c = clip_s;
  float sc = __fdiv_rn(c, 127.0f);
  if (sc == 0.0f) sc = 1.0f;
  const RowDivider dv(sc);
  for (int i = tid; i < K; i += kClipThreads) {
    const float x = fminf(fmaxf(Elem<T>::load(vr, i), -c), c);
    const float r = fminf(fmaxf(rintf(dv.div(x)), -128.0f), 127.0f);
    q[row * K + i] = (int8_t)(int32_t)r;
  }
}

hipError_t launch_quantize_rows_int8_clip(const void* v, int v_dtype, int64_t R, int64_t K, float pct, int8_t* q,
                                          float* scale, hipStream_t s) {
  int P2 = 1;
  while (P2 < K) P2 <<= 1;
  const dim3 grid((unsigned)R), block(kClipThreads);
  const size_t lds = (size_t)P2 * sizeof(float);
  switch (v_dtype) {
    case F32:
      hipLaunchKernelGGL(quantize_rows_int8_clip_kernel<float>, grid, block, lds, s, (const float*)v, (int)K, P2,
                         pct, q, scale);
      break;
    case BF16:
      hipLaunchKernelGGL(quantize_rows_int8_clip_kernel<bf16_t>, grid, block, lds, s, (const bf16_t*)v, (int)K,
                         P2, pct, q, scale);
      break;
    default:
      hipLaunchKernelGGL(quantize_rows_int8_clip_kernel<f16_t>, grid, block, lds, s, (const f16_t*)v, (int)K, P2,
                         pct, q, scale);
      break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------ per-column int4 packing
// w [K, N] (row-major, N contiguous) -> packed [K/2, N] uint8 with the even k
// in the high nibble, and scale [N] fp32: s = absmax of the column / 7 (1 if
// 0), code = clamp(rint(w / s) + 8, 0, 15), the quotient correctly rounded.
// A block covers 64 consecutive columns (a wave reads 64 neighbours of one
// row) with its sixteen waves splitting the rows: pass 1 takes each wave's
// column maxima over rows k = wave, wave + 16, ..., LDS joins the sixteen;
// pass 2 writes k-pair rows kp = wave, wave + 16, ...  Loops are unrolled so
// that eight loads are in flight per lane.
constexpr int kPackInt4Slices = 16;
template <typename T>
__global__ void __launch_bounds__(64 * kPackInt4Slices)
pack_int4_cols_kernel(const T* __restrict__ w, int K, int N, uint8_t* __restrict__ packed,
                      float* __restrict__ scale) {
  constexpr int SL = kPackInt4Slices;
  __shared__ float red[SL][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + tx;
  const bool in = n < N;
  float a = 0.0f;
  if (in) {
#pragma unroll 8
    for (int k = ty; k < K; k += SL) a = fmaxf(a, fabsf(Elem<T>::load(w, (int64_t)k * N + n)));
  }
  red[ty][tx] = a;
  __syncthreads();
  a = red[0][tx];
#pragma unroll
  for (int i = 1; i < SL; ++i) a = fmaxf(a, red[i][tx]);
  float sc = __fdiv_rn(a, 7.0f);
  if (sc == 0.0f) sc = 1.0f;
  if (!in) return;
  if (ty == 0) scale[n] = sc;
  const RowDivider dv(sc);
#pragma unroll 4
  for (int kp = ty; kp < K / 2; kp += SL) {
    const float h = fminf(fmaxf(rintf(dv.div(Elem<T>::load(w, (int64_t)(2 * kp) * N + n))) + 8.0f, 0.0f), 15.0f);
    const float l = fminf(fmaxf(rintf(dv.div(Elem<T>::load(w, (int64_t)(2 * kp + 1) * N + n))) + 8.0f, 0.0f), 15.0f);
    packed[(int64_t)kp * N + n] = (uint8_t)(((int)h << 4) | (int)l);
  }
}

hipError_t launch_pack_int4_cols(const void* w, int w_dtype, int64_t K, int64_t N, uint8_t* packed, float* scale,
                                 hipStream_t s) {
  const dim3 grid((unsigned)cdiv(N, 64)), block(64 * kPackInt4Slices);
  switch (w_dtype) {
    case F32:
      hipLaunchKernelGGL(pack_int4_cols_kernel<float>, grid, block, 0, s, (const float*)w, (int)K, (int)N, packed,
                         scale);
      break;
    case BF16:
      hipLaunchKernelGGL(pack_int4_cols_kernel<bf16_t>, grid, block, 0, s, (const bf16_t*)w, (int)K, (int)N,
                         packed, scale);
      break;
    default:
      hipLaunchKernelGGL(pack_int4_cols_kernel<f16_t>, grid, block, 0, s, (const f16_t*)w, (int)K, (int)N, packed,
                         scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace qlq
