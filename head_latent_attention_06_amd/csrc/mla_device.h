// Device-side helpers shared by the MLA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;     // MFMA A/B operand
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;  // 16-byte move
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;     // 32x32 accumulator
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// --- MFMA -------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16.  Operand layout for lane l (0..63):
//   A: A[m = l%32][k = 8*(l/32) + e], e = 0..7       (8 bf16 per lane)
//   B: B[k = 8*(l/32) + e][n = l%32]
//   D: D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32], i = 0..15
// Only the pairing of A's and B's k slots matters for a contraction, and the
// two operands use the same slot numbering.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// --- bf16 <-> f32 ------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Round two floats to bf16 (nearest, ties to even) and pack lo | hi << 16
// (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// --- 16-byte memory moves --------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// --- 8x8 bf16 transpose in registers --------------------------------------------
// in[r] holds row r (8 bf16: element c in half (c&1) of dword c/2).  On return
// out[c] holds column c: element r of out[c] = element c of in[r].
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c2 = 0; c2 < 4; ++c2) {     // column pair (2*c2, 2*c2+1) = dword c2 of every row
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {   // row pair (2*r2, 2*r2+1) -> dword r2 of the outputs
      uint32_t x0 = in[2 * r2][c2], x1 = in[2 * r2 + 1][c2];
      out[2 * c2][r2] = (x0 & 0xFFFFu) | (x1 << 16);
      out[2 * c2 + 1][r2] = (x0 >> 16) | (x1 & 0xFFFF0000u);
    }
  }
}

// --- cross-lane ----------------------------------------------------------------
// max / sum of a value with the one held by lane (l ^ 32).  v_permlane32_swap
// exchanges the two 32-lane halves of the wave without going through LDS; the
// pair it returns is {own value, partner's value} in some order, so a
// symmetric combine of the pair is the same in every lane.
__device__ __forceinline__ float pair_max32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over a full 64-lane wave (butterfly of lane shuffles).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// blockIdx -> logical work id such that consecutive ids run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2),
// so block b lands on XCD b % 8.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8;
  const int xcd = bid % 8, local = bid / 8;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

}  // namespace mla
