// Packed int4 weights in the [K/2, N] byte layout ("cider/ops.py",
// pack_weight_int4: byte (kp, n) holds the code of k = 2 kp in its high nibble
// and of k = 2 kp + 1 in its low nibble, value = code - 8).  Helpers shared by
// the kernels that read it: a thread loads one dword (4 columns) from each of
// 8 consecutive k-pair rows, turns the block around so that each column's 8
// bytes (16 k) are together, and unpacks them to int8 values 16 (code - 8):
// (code << 4) ^ 0x80 keeps a high nibble in place, a low nibble is shifted up
// first.  The 16 values of a column come out in the order k = 0 2 4 6 | 1 3 5
// 7 | 8 10 12 14 | 9 11 13 15 (high then low nibbles, four bytes at a time);
// the activation operand is stored in the same order.
#pragma once

#include "common.hpp"

namespace qlq {
namespace int4 {

// element of a 16-value chunk held in slot s of the unpacked order:
// k = 0 2 4 6 1 3 5 7 8 10 12 14 9 11 13 15
__host__ __device__ constexpr int act_slot(int s) { return (s & 8) | ((s & 3) << 1) | ((s >> 2) & 1); }

// o[c] = byte c of each of r0..r3, i.e. column c of a 4-row block
__device__ __forceinline__ void transpose4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t (&o)[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t2 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// 16 int8 values 16 (code - 8) of one column from its packed bytes of k-pair
// rows 0..3 (lo) and 4..7 (hi)
__device__ __forceinline__ u32x4_v unpack16(uint32_t lo, uint32_t hi) {
  u32x4_v v;
  v[0] = (lo & 0xF0F0F0F0u) ^ 0x80808080u;
  v[1] = ((lo << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
  v[2] = (hi & 0xF0F0F0F0u) ^ 0x80808080u;
  v[3] = ((hi << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
  return v;
}

// this thread's 8 k-pair rows srow + vrow + i (i < 8) at columns col .. col+3
// of the matrix behind r (K2 rows of N bytes, r based at a column offset
// that leaves ncols columns to its right); srow is wave-uniform (it rides in
// the scalar offset), vrow per lane.  full: every such row of every lane is
// below K2.  Every address stays inside the matrix: otherwise rows past K2
// repeat the last row (their activations are zero), and columns are clamped
// by the caller (BYTES = false: col <= ncols - 4) or here (BYTES = true, for
// N % 4 != 0: each byte's column clamped to ncols - 1).  AUX: the loads'
// cache-policy operand.
template <bool BYTES, int AUX = 0>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, int srow, int vrow, bool full, int K2, int N,
                                      int ncols, int col, uint32_t (&bw)[8]) {
  if constexpr (!BYTES) {
    if (full) {
      const int vo = vrow * N + col;
#pragma unroll
      for (int i = 0; i < 8; ++i) bw[i] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, (srow + i) * N, AUX);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        bw[i] = __builtin_amdgcn_raw_buffer_load_b32(r, min(srow + vrow + i, K2 - 1) * N + col, 0, AUX);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ro = min(srow + vrow + i, K2 - 1) * N;
      uint32_t v = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, ro + min(col + j, ncols - 1), 0, AUX) << (8 * j);
      bw[i] = v;
    }
  }
}

}  // namespace int4
}  // namespace qlq
