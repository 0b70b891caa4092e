// Shared device helpers for the qlq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlq {

// Storage dtype codes (match enum qlq_dtype in qlq.h).
enum DType : int { F32 = 0, F16 = 1, BF16 = 2 };

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef _Float16 f16_t;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_v;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;
typedef __attribute__((ext_vector_type(16))) float f32x16_v;
typedef __attribute__((ext_vector_type(4))) int i32x4_v;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_v;  // 16 bytes in registers

constexpr int kWave = 64;

// ---- scalar conversions ------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Typed element access for the three storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = (bf16_t)f32_to_bf16_rne(v); }
  static __device__ __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16_rne(v)); }
  static __device__ __forceinline__ uint16_t bits(float v) { return (uint16_t)f32_to_bf16_rne(v); }
};
template <> struct Elem<f16_t> {
  static __device__ __forceinline__ float load(const f16_t* p, int64_t i) { return (float)p[i]; }
  static __device__ __forceinline__ void store(f16_t* p, int64_t i, float v) { p[i] = (f16_t)v; }
  static __device__ __forceinline__ float round(float v) { return (float)(f16_t)v; }
  static __device__ __forceinline__ uint16_t bits(float v) { return __builtin_bit_cast(uint16_t, (f16_t)v); }
};

// Loads of data that one launch reads once (weight streams): the
// non-temporal hint streams them through the caches.
template <typename T> __device__ __forceinline__ T stream_load(const T* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint4 stream_u4(const void* p) {
  const u32x4_v v = stream_load(reinterpret_cast<const u32x4_v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// cache-policy operand of the raw buffer loads for the same streams (NT)
constexpr int kStreamAux = 2;
template <typename T> __device__ __forceinline__ float stream_elem(const T* p, int64_t i);
template <> __device__ __forceinline__ float stream_elem<float>(const float* p, int64_t i) { return stream_load(p + i); }
template <> __device__ __forceinline__ float stream_elem<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_to_f32(stream_load(p + i));
}
template <> __device__ __forceinline__ float stream_elem<f16_t>(const f16_t* p, int64_t i) {
  return (float)stream_load(p + i);
}

// 16-bit storage bits -> fp32 value for a 16-bit storage type.
template <typename T> __device__ __forceinline__ float bits16_to_f32(uint16_t h);
template <> __device__ __forceinline__ float bits16_to_f32<bf16_t>(uint16_t h) { return bf16_to_f32(h); }
template <> __device__ __forceinline__ float bits16_to_f32<f16_t>(uint16_t h) {
  return (float)__builtin_bit_cast(f16_t, h);
}

__device__ __forceinline__ bool is_finite_f32(float v) {
  return (__float_as_uint(v) & 0x7F800000u) != 0x7F800000u;
}

// ---- wave reductions (wave64) ---------------------------------------------
// DPP sum: two quad permutes and two row rotates leave every lane of each
// 16-lane row holding the row's sum; four readlanes add the rows.  The result
// is uniform across the wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x124>(v);  // row_ror:4
  v += dpp_f32<0x128>(v);  // row_ror:8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}
// DPP max (same pattern as wave_sum_dpp); the result is uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  v = fmaxf(v, dpp_f32<0x128>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Store a 64x64 tile of outputs held in the 32x32 MFMA result layout (lane l,
// element e of sub-tile (i, j) is row 32i + 8(e/4) + 4(l/32) + e%4, column
// 32j + l%32) as 16-bit values at out[row0 + r, col0 + c] (r < nrows, c <
// ncols, leading dimension ldo).  The values are rounded once, parked in the
// calling wave's LDS area (64 rows x 144 bytes: the 16-byte pad keeps the two
// half-waves' writes on different banks) and leave as 16-byte row-contiguous
// stores where the row is aligned, else element by element.
constexpr int kTileStageBytes = 64 * 144;
template <typename OT>
__device__ __forceinline__ void store_tile64_16(const float (&v)[2][2][16], OT* __restrict__ out, int64_t ldo,
                                                int row0, int col0, int nrows, int ncols, int8_t* lds, int lane) {
  constexpr int STRIDE = 144;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), c = 32 * j + (lane & 31);
        *reinterpret_cast<uint16_t*>(lds + r * STRIDE + c * 2) = Elem<OT>::bits(v[i][j][e]);
      }
  // one wave's LDS accesses complete in order: the reads below see the writes
  const bool vec = ldo % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 8 + (lane >> 3), c = (lane & 7) * 8;
    const u32x4_v d = *reinterpret_cast<const u32x4_v*>(lds + r * STRIDE + c * 2);
    if (r >= nrows || c >= ncols) continue;
    uint16_t* dst = reinterpret_cast<uint16_t*>(out + (int64_t)(row0 + r) * ldo + col0 + c);
    if (vec && c + 8 <= ncols) {
      *reinterpret_cast<u32x4_v*>(dst) = d;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (c + t < ncols) dst[t] = (uint16_t)(d[t >> 1] >> (16 * (t & 1)));
    }
  }
}

// 16 consecutive elements (16-byte aligned) widened to fp32.
template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&v)[16]);
template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 f = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
}
template <>
__device__ __forceinline__ void load16<bf16_t>(const bf16_t* p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint4 u = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}
template <>
__device__ __forceinline__ void load16<f16_t>(const f16_t* p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f16x8_v h = reinterpret_cast<const f16x8_v*>(p)[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[8 * i + j] = (float)h[j];
  }
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Raw buffer access (stride 0): the hardware checks every byte offset against
// the descriptor's size and returns zero for reads past it.  kOutOfRange is an
// offset past any buffer made here (sizes stay below 2^31 bytes).  0x00020000
// is the gfx9-family word 3 of a raw buffer descriptor (32-bit data format).
constexpr int kOutOfRange = (int)0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_v load_b128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane from global memory straight into LDS: lane i writes
// dst + 16 i (dst wave-uniform); an out-of-range offset writes zeros.
__device__ __forceinline__ void load_lds_b128(__amdgpu_buffer_rsrc_t r, void* dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
// Same with a wave-uniform byte offset soff added in the scalar unit (an
// offset of a whole operand tile, for instance); voff stays per lane.
__device__ __forceinline__ void load_lds_b128(__amdgpu_buffer_rsrc_t r, void* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// LDS rows of CB 16-byte chunks keep chunk c of row r in slot c ^ lds_swz<CB>(r):
// the chunk-c reads of 8 (or 16) consecutive rows then fall in 8 (16)
// distinct 16-byte bank slots of a 128-byte (256-byte) window.
template <int CB>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(CB == 1 || CB == 2 || CB == 4 || CB == 8 || CB == 16, "chunks per row");
  if constexpr (CB == 1) return 0;
  else if constexpr (CB == 2) return ((r >> 2) ^ (r >> 3)) & 1;
  else if constexpr (CB == 4) return ((r >> 1) ^ (r >> 2)) & 3;
  else if constexpr (CB == 8) return (r ^ (r >> 3)) & 7;
  else return r & 15;
}

// ---------------------------------------------- quotient by a row's scale
// x / s rounded to nearest for one divisor s shared by a whole row: the
// correctly rounded reciprocal y = RN(1/s) once, then per quotient q =
// RN(x*y), the exact residual r = x - s*q (one fused multiply-add) and
// RN(q + r*y), which is the correctly rounded quotient when y is the
// correctly rounded reciprocal and nothing under- or overflows (Markstein's
// correction step).  Here |x| <= 127 |s|; divisors outside [2^-100, 2^100]
// keep the full division.
struct RowDivider {
  float s, y;
  bool fast;
  __device__ __forceinline__ explicit RowDivider(float s_) : s(s_), y(__fdiv_rn(1.0f, s_)) {
    const float as = fabsf(s_);
    fast = as >= 0x1p-100f && as <= 0x1p100f;
  }
  __device__ __forceinline__ float div(float x) const {
    if (!fast) return __fdiv_rn(x, s);
    const float q = x * y;
    return fmaf(fmaf(-s, q, x), y, q);
  }
};

// The int8 code clamp(rint(d), -128, 127) in the low byte of a word: clamp
// first (v_med3; the same integer as clamping after rounding), then t +
// 1.5 * 2^23, which for |t| < 2^22 rounds t to the nearest integer, ties to
// even as rint does, and leaves it as the two's-complement low bits of the
// sum's encoding.
__device__ __forceinline__ uint32_t int8_code_bits(float d) {
  const float t = __builtin_amdgcn_fmed3f(d, -128.0f, 127.0f);
  return __float_as_uint(t + 12582912.0f);
}
// the low bytes of a, b, c, d as the bytes 0..3 of one word
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a0, b0, 0, 0
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);  // c0, d0, 0, 0
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);              // a0, b0, c0, d0
}

// ------------------------------------------------ affine n-bit code streams
// A row's codes form one LSB-first bit stream (code k at stream bits
// BITS*k .. BITS*k + BITS - 1, stream bit i = bit i % 32 of word i / 32), so
// 32 codes always fill exactly BITS words: a unit.  With j known at compile
// time the offsets fold away; a code that straddles two words (3, 5, 6 bits)
// is one funnel shift.
template <int BITS>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w, int j) {
  constexpr uint32_t mask = (1u << BITS) - 1u;
  const int p = BITS * j, i = p >> 5, o = p & 31;
  if (o + BITS <= 32) return (w[i] >> o) & mask;
  return ((w[i] >> o) | (w[i + 1] << (32 - o))) & mask;
}
template <int BITS>
__device__ __forceinline__ void unit_put(uint32_t* w, int j, uint32_t q) {
  const int p = BITS * j, i = p >> 5, o = p & 31;
  w[i] |= q << o;
  if (o + BITS > 32) w[i + 1] |= q >> (32 - o);
}

}  // namespace qlq
