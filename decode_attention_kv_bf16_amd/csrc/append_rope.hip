// Cache append with rotary position embedding: the step that comes right
// before decode attention. Each decode step makes one new k and v row per
// sequence and appends it to the cache ("KV Cache 如何影响了 LLM Inference",
// section 2.2); for MLA the cached row is [c_kv ; RoPE(k_rope)], the rope key
// rotated before it is cached and shared by all heads, and the query's rope
// part is rotated per head ("Attention variants and KV cache", section 4.2).
// RoPE rotates pair i of the first r entries by m * theta_i, theta_i =
// base^(-2i/r), for a token at position m (the rotary form; the pages fix
// only that R_m depends on m alone with R_m^T R_n = R_{n-m}, section 4.4).
//
// One workgroup serves a slice of one sequence's rows. Work items are
// "pieces" of 8 entries of one row: a rotated piece holds 4 pairs (entries
// 4j..4j+3 and r/2+4j.. for the half pairing, 8j..8j+7 for the interleaved
// one); the other pieces are copies. Every thread issues the loads of its
// piece, then the workgroup makes the r/2 (cos, sin) values of its
// sequence's position in LDS (angles reduced in double precision), and each
// piece is rotated in fp32 and stored, rounded once to the row's type.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPairs = 64;   // r <= 128

// Four entries of a row as raw words: bf16 (8 bytes) or fp32 (16 bytes).
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
  using V = uint2;
  static __device__ __forceinline__ void to_f(V w, float* f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  }
  static __device__ __forceinline__ V from_f(const float* f) {
    return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};
template <> struct Quad<float> {
  using V = float4;
  static __device__ __forceinline__ void to_f(V w, float* f) { f[0] = w.x; f[1] = w.y; f[2] = w.z; f[3] = w.w; }
  static __device__ __forceinline__ V from_f(const float* f) { return make_float4(f[0], f[1], f[2], f[3]); }
};

// (a, b) -> (a cos - b sin, a sin + b cos)
__device__ __forceinline__ void rotate(float& a, float& b, float2 cs) {
  const float na = fmaf(a, cs.x, -b * cs.y);
  const float nb = fmaf(a, cs.y, b * cs.x);
  a = na;
  b = nb;
}

// One thread's piece: 8 entries of a row, read as two quads before the angle
// table is built (so the loads are in flight meanwhile), then rotated or
// copied. Rotated piece j: entries 4j.. and r/2 + 4j.. (half pairing) or
// 8j.. and 8j + 4.. (interleaved); copied piece j: 8j.. and 8j + 4...
template <typename T>
struct Piece {
  using V = typename Quad<T>::V;
  T* dst = nullptr;
  int off_lo = 0, off_hi = 0, j = 0;
  bool rotated = false;
  V lo{}, hi{};

  __device__ __forceinline__ void load(const T* src, T* d, int jj, bool rot, int r, int style) {
    dst = d;
    j = jj;
    rotated = rot;
    off_lo = rot && style == 0 ? 4 * jj : 8 * jj;
    off_hi = rot && style == 0 ? r / 2 + 4 * jj : 8 * jj + 4;
    lo = *reinterpret_cast<const V*>(src + off_lo);
    hi = *reinterpret_cast<const V*>(src + off_hi);
  }

  __device__ __forceinline__ void finish(int style, const float2* cs) {
    if (rotated) {
      float l[4], h[4];
      Quad<T>::to_f(lo, l);
      Quad<T>::to_f(hi, h);
      if (style == 0) {            // half: pair 4j + k is (l[k], h[k])
#pragma unroll
        for (int k = 0; k < 4; ++k) rotate(l[k], h[k], cs[4 * j + k]);
      } else {                     // interleaved: (l0, l1), (l2, l3), (h0, h1), (h2, h3)
        rotate(l[0], l[1], cs[4 * j + 0]);
        rotate(l[2], l[3], cs[4 * j + 1]);
        rotate(h[0], h[1], cs[4 * j + 2]);
        rotate(h[2], h[3], cs[4 * j + 3]);
      }
      lo = Quad<T>::from_f(l);
      hi = Quad<T>::from_f(h);
    }
    *reinterpret_cast<V*>(dst + off_lo) = lo;
    *reinterpret_cast<V*>(dst + off_hi) = hi;
  }
};

// cos and sin of pos * theta_i for i < r/2, into LDS. theta and the angle
// are taken in double, the angle is reduced to [-pi, pi] in double (2 pi in
// two parts, Cody-Waite), and the reduced angle's sine and cosine in float:
// the result is within a few float roundings for any int32 position.
__device__ __forceinline__ void make_table(const AppendArgs& a, int pos, float2* cs) {
  const int i = threadIdx.x;
  if (i < a.rot / 2) {
    const double theta = a.inv_freq ? (double)a.inv_freq[i]
                                    : exp2(-(double)(2 * i) / (double)a.rot * a.log2_base);
    const double phi = (double)pos * theta;
    const double k = rint(phi * 0.15915494309189535);              // 1 / (2 pi)
    double r = fma(-k, 6.283185307179586, phi);                    // 2 pi, high part
    r = fma(-k, 2.4492935982947064e-16, r);                        // 2 pi, low part
    float s, c;
    sincosf((float)r, &s, &c);
    cs[i] = make_float2(c, s);
  }
  __syncthreads();
}

// Element offset of cache row (b, pos): contiguous or through the block table.
__device__ __forceinline__ int64_t row_offset(const AppendArgs& a, int b, int pos) {
  if (a.page_shift == 0) return (int64_t)b * a.c_sb + (int64_t)pos * a.c_st;
  const int32_t page = a.block_table[(int64_t)b * a.max_blocks + (pos >> a.page_shift)];
  return (int64_t)page * a.page_stride + (int64_t)(pos & ((1 << a.page_shift) - 1)) * a.c_st;
}

// GQA rows of sequence b: Hq query rows, Hkv key rows (both rotated), Hkv
// value rows (copied); head_dim / 8 pieces each.
template <typename T>
__global__ __launch_bounds__(kThreads) void gqa_append_rope_kernel(AppendArgs a) {
  __shared__ float2 cs[kMaxPairs];
  const int b = blockIdx.y;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.max_seq_len) return;          // uniform: the sequence is skipped
  const int per_row = a.dim / 8;
  const int item = blockIdx.x * kThreads + threadIdx.x;
  const int row = item / per_row, j = item - row * per_row;
  const bool valid = row < a.q_heads + 2 * a.kv_heads;
  const bool rot_piece = j < a.rot / 8;
  Piece<T> pc;
  if (valid) {
    if (row < a.q_heads) {
      const int64_t o = (int64_t)b * a.q_sb + (int64_t)row * a.q_sh;
      pc.load(static_cast<const T*>(a.q) + o, static_cast<T*>(a.q_out) + o, j, rot_piece, a.rot, a.style);
    } else {
      const int kv = row - a.q_heads;
      const bool is_k = kv < a.kv_heads;
      const int h = is_k ? kv : kv - a.kv_heads;
      const T* src = static_cast<const T*>(is_k ? a.k_new : a.v_new) + (int64_t)b * a.new_sb +
                     (int64_t)h * a.new_sh;
      T* dst = static_cast<T*>(is_k ? a.k_cache : a.v_cache) + row_offset(a, b, pos) +
               (int64_t)h * a.c_sh;
      pc.load(src, dst, j, is_k && rot_piece, a.rot, a.style);
    }
  }
  make_table(a, pos, cs);
  if (valid) pc.finish(a.style, cs);
}

// MLA rows of sequence b: H query rope rows (64 entries, rotated), the rope
// key (64, rotated, into entries 512.. of the cached row) and the latent
// (512, copied into entries 0..511).
__global__ __launch_bounds__(kThreads) void mla_append_rope_kernel(AppendArgs a) {
  __shared__ float2 cs[kMaxPairs];
  constexpr int kDc = 512, kRope = 64, kPieces = kRope / 8;
  const int b = blockIdx.y;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.max_seq_len) return;
  const int item = blockIdx.x * kThreads + threadIdx.x;
  const int q_items = a.q_heads * kPieces;
  const uint16_t* kv_new = static_cast<const uint16_t*>(a.k_new) + (int64_t)b * a.new_sb;
  const bool valid = item < q_items + kPieces + kDc / 8;
  Piece<uint16_t> pc;
  if (item < q_items) {
    const int h = item / kPieces, j = item - h * kPieces;
    const int64_t o = (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;
    pc.load(static_cast<const uint16_t*>(a.q) + o, static_cast<uint16_t*>(a.q_out) + o, j,
            j < a.rot / 8, a.rot, a.style);
  } else if (valid) {
    const int r = item - q_items;
    uint16_t* row = static_cast<uint16_t*>(a.k_cache) + row_offset(a, b, pos);
    if (r < kPieces)
      pc.load(kv_new + kDc, row + kDc, r, r < a.rot / 8, a.rot, a.style);
    else
      pc.load(kv_new, row, r - kPieces, false, a.rot, a.style);
  }
  make_table(a, pos, cs);
  if (valid) pc.finish(a.style, cs);
}

// fp32 -> OCP E4M3 code, round to nearest even, magnitudes clamped to the
// largest finite 448 (the format has no infinities). From the format's
// fields: below 2^-6 the code is a multiple of 2^-9 (subnormal), above it
// the float's mantissa is rounded to 3 bits at bit 20.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);        // 0..8 (8 is 2^-6)
  const uint32_t bits = __float_as_uint(a);
  const uint32_t r = bits + 0x7ffffu + ((bits >> 20) & 1u);            // RNE to 3 mantissa bits
  const uint32_t e = ((r >> 23) & 0xffu) - 127u + 7u;                  // biased E4M3 exponent
  return sign | (e << 3) | ((r >> 20) & 7u);
}

// GQA append into an E4M3 cache. Rows are rotated (keys) in fp32 as in the
// bf16 kernel, then each (token, KV head) row of K and of V is quantized:
// dynamic scales (scale token stride != 0): s = amax(|row|) / 448, written;
// static scales (token stride 0): s read. Codes = E4M3(x / s) (0 when s is 0).
// The row's d/8 pieces sit on consecutive lanes, so its amax is a butterfly
// over those lanes; every lane takes part in it.
__global__ __launch_bounds__(kThreads) void gqa_append_rope_fp8_kernel(AppendArgs a) {
  __shared__ float2 cs[kMaxPairs];
  const int b = blockIdx.y;
  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.max_seq_len) return;
  const int per_row = a.dim / 8;
  const int item = blockIdx.x * kThreads + threadIdx.x;
  const int row = item / per_row, j = item - row * per_row;
  const bool valid = row < a.q_heads + 2 * a.kv_heads;
  const bool is_q = row < a.q_heads;
  const bool rot_piece = j < a.rot / 8;
  const int kv = row - a.q_heads;
  const bool is_k = kv < a.kv_heads;
  const int h = is_k ? kv : kv - a.kv_heads;
  Piece<uint16_t> pc;
  if (valid) {
    if (is_q) {
      const int64_t o = (int64_t)b * a.q_sb + (int64_t)row * a.q_sh;
      pc.load(static_cast<const uint16_t*>(a.q) + o, static_cast<uint16_t*>(a.q_out) + o, j, rot_piece,
              a.rot, a.style);
    } else {
      const uint16_t* src = static_cast<const uint16_t*>(is_k ? a.k_new : a.v_new) +
                            (int64_t)b * a.new_sb + (int64_t)h * a.new_sh;
      pc.load(src, nullptr, j, is_k && rot_piece, a.rot, a.style);
    }
  }
  make_table(a, pos, cs);
  if (valid && is_q) pc.finish(a.style, cs);
  // K/V rows: values in fp32 (rotated for keys)
  float l[4] = {0.f, 0.f, 0.f, 0.f}, hv[4] = {0.f, 0.f, 0.f, 0.f};
  const bool kv_row = valid && !is_q;
  if (kv_row) {
    Quad<uint16_t>::to_f(pc.lo, l);
    Quad<uint16_t>::to_f(pc.hi, hv);
    if (pc.rotated) {
      if (a.style == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) rotate(l[k], hv[k], cs[4 * j + k]);
      } else {
        rotate(l[0], l[1], cs[4 * j + 0]);
        rotate(l[2], l[3], cs[4 * j + 1]);
        rotate(hv[0], hv[1], cs[4 * j + 2]);
        rotate(hv[2], hv[3], cs[4 * j + 3]);
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fmaxf(fabsf(l[k]), fabsf(hv[k])));
  for (int m = 1; m < per_row; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  if (!kv_row) return;
  const int64_t sc_idx = (int64_t)b * a.sc_sb + (int64_t)pos * a.sc_st + (int64_t)h * a.sc_sh;
  float* scales = is_k ? a.k_scale : a.v_scale;
  const bool dynamic = a.sc_st != 0;
  const float s = dynamic ? amax / 448.f : scales[sc_idx];
  if (dynamic && j == 0) scales[sc_idx] = s;
  uint32_t lo = 0, hi = 0;
  if (s != 0.f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= e4m3_code(l[k] / s) << (8 * k);
      hi |= e4m3_code(hv[k] / s) << (8 * k);
    }
  }
  uint8_t* dst = static_cast<uint8_t*>(is_k ? a.k_cache : a.v_cache) + row_offset(a, b, pos) +
                 (int64_t)h * a.c_sh;
  *reinterpret_cast<uint32_t*>(dst + pc.off_lo) = lo;
  *reinterpret_cast<uint32_t*>(dst + pc.off_hi) = hi;
}

}  // namespace

hipError_t launch_gqa_append_rope_fp8(const AppendArgs& a, hipStream_t stream) {
  const int items = (a.q_heads + 2 * a.kv_heads) * (a.dim / 8);
  const dim3 grid((items + kThreads - 1) / kThreads, a.batch);
  gqa_append_rope_fp8_kernel<<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gqa_append_rope(const AppendArgs& a, int dtype, hipStream_t stream) {
  const int items = (a.q_heads + 2 * a.kv_heads) * (a.dim / 8);
  const dim3 grid((items + kThreads - 1) / kThreads, a.batch);
  if (dtype == 1)
    gqa_append_rope_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(a);
  else
    gqa_append_rope_kernel<float><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_mla_append_rope(const AppendArgs& a, hipStream_t stream) {
  const int items = a.q_heads * 8 + 8 + 512 / 8;
  const dim3 grid((items + kThreads - 1) / kThreads, a.batch);
  mla_append_rope_kernel<<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace da
