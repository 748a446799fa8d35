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

// Buffer resource for raw (unswizzled, stride 0) byte addressing: loads past
// num_records bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One wave-wide 1 KiB copy HBM -> LDS (buffer_load_dwordx4 ... lds): lane l
// reads 16 bytes at rsrc base + voffset and writes them at LDS byte address
// lds_addr + 16 l (lds_addr is wave-uniform). Written in asm so that the compiler does not track
// the copy: tracked, every LDS read after it waits for all outstanding copies
// (vmcnt(0)), because the compiler cannot tell which LDS bytes a copy writes.
// Completion is waited for explicitly with wait_vm<N>() instead. The asm has
// no output register (the data goes to LDS); M0, which holds the LDS address,
// is saved and restored around it. The cache rows are read once, so the copy
// is non-temporal (`nt`): measured 1.7% faster for the attention kernel, which
// runs at the board's power limit, where moving the cache in from HBM takes
// about a quarter of its time.
__device__ __forceinline__ void buffer_load_to_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                                     uint32_t lds_addr) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(voffset), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// The 4-byte form: lane l reads 4 bytes at rsrc base + voffset and writes
// them at LDS byte address lds_addr + 4 l. Same conventions as above.
__device__ __forceinline__ void buffer_load_to_lds4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                                    uint32_t lds_addr) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(voffset), "s"(rsrc), "s"(lds_addr)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The sequence of rank r when the batch is ordered by length, longest first
// (ties by index, so the ranks are a permutation). Workgroups are dispatched
// in id order, so giving the lowest ids the longest sequences lets the short
// ones fill the end of a ragged batch (longest-processing-time-first
// scheduling). B <= 256; every thread of the workgroup takes part.
template <int kThreads>
__device__ __forceinline__ int longest_first(const int32_t* seq_lens, int B, int r) {
  __shared__ int s_len[256];
  __shared__ int s_pick;
  for (int i = threadIdx.x; i < B; i += kThreads) s_len[i] = seq_lens[i];
  __syncthreads();
  for (int c = threadIdx.x; c < B; c += kThreads) {
    const int lc = s_len[c];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int lj = s_len[j];
      rank += (lj > lc) | ((lj == lc) & (j < c));
    }
    if (rank == r) s_pick = c;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_pick);
}

}  // namespace da
