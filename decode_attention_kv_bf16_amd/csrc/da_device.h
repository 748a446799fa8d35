// Device-side helpers shared by the decode-attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

// v_exp_f32 / v_log_f32: hardware base-2 exponential and logarithm.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Data-parallel-primitive lane moves within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppQuadReverse = 0x1B; // quad_perm [3,2,1,0]: lane i <- 3 - i within 4
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- 15 - i within 16
constexpr int kDppRowRor4 = 0x124;        // rotate by 4 within 16
constexpr int kDppRowRor8 = 0x128;        // rotate by 8 within 16
// Every lane of a row of 16 receives the value of lane n of that row (DPP
// row_newbcast). n must be a compile-time constant after unrolling: the
// switch then folds to one move.
__device__ __forceinline__ float row_bcast(int n, float v) {
  switch (n) {
    case 0: return dpp_mov<0x150>(v);
    case 1: return dpp_mov<0x151>(v);
    case 2: return dpp_mov<0x152>(v);
    case 3: return dpp_mov<0x153>(v);
    case 4: return dpp_mov<0x154>(v);
    case 5: return dpp_mov<0x155>(v);
    case 6: return dpp_mov<0x156>(v);
    case 7: return dpp_mov<0x157>(v);
    case 8: return dpp_mov<0x158>(v);
    case 9: return dpp_mov<0x159>(v);
    case 10: return dpp_mov<0x15A>(v);
    case 11: return dpp_mov<0x15B>(v);
    case 12: return dpp_mov<0x15C>(v);
    case 13: return dpp_mov<0x15D>(v);
    case 14: return dpp_mov<0x15E>(v);
    default: return dpp_mov<0x15F>(v);
  }
}

// Sum over aligned groups of N consecutive lanes (N in 1, 2, 4, 8, 16); every
// lane of the group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v += dpp_mov<kDppQuadSwap1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppQuadSwap2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
  return v;
}

// bf16 bit patterns -> float: the low half of a dword is shifted up, the high
// half masked.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// float -> bf16 with round-to-nearest-even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pair (low half = lo) with the hardware
// round-to-nearest-even conversion (v_cvt_pk_bf16_f32).
typedef float da_f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 da_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(da_f32x2_t{lo, hi}, da_bf16x2_t));
}

// c + a.lo * b.lo + a.hi * b.hi for packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(da_bf16x2_t, a), __builtin_bit_cast(da_bf16x2_t, b), c,
                                         false);
}

// Merge two online-softmax states (m, l, acc) kept in the base-2 domain:
// m is the running max of log2-scaled scores, l = sum 2^(s - m).
// Returns the factors that rescale each side onto the common max.
struct MergeFactors {
  float m, a, b;
};
__device__ __forceinline__ MergeFactors merge_factors(float m1, float m2) {
  float m = fmaxf(m1, m2);
  float mu = (m == kNegInf) ? 0.0f : m;   // both empty: keep factors finite (0)
  return {m, exp2_hw(m1 - mu), exp2_hw(m2 - mu)};
}

}  // namespace da
