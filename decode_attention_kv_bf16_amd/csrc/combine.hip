// Split-KV merge: combine per-split (o_s, lse_s) into the final (o, lse).
//
// Flash-decoding splits decode attention along the sequence, normalises each
// split locally and merges the normalisers at the end (arganzheng.life,
// section 5.2). With lse_s = log sum_{j in s} exp(score_j):
//   lse = log sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s.
// A split whose lse_s is -inf held no rows: its o_s is never read.
#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

constexpr int kThreads = 256;

// TPR threads serve one output row; each thread handles float4 columns.
template <int TPR>
__global__ __launch_bounds__(kThreads) void splitkv_combine_kernel(
    int num_splits, int rows, int head_dim, const float* __restrict__ part_out,
    const float* __restrict__ part_lse, float* __restrict__ out, float* __restrict__ lse) {
  const int r = blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (r >= rows) return;
  float M = kNegInf;
  for (int s = 0; s < num_splits; ++s) M = fmaxf(M, part_lse[(int64_t)s * rows + r]);
  if (M == kNegInf) {
    for (int d = t * 4; d < head_dim; d += TPR * 4)
      *reinterpret_cast<float4*>(out + (int64_t)r * head_dim + d) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t == 0 && lse) lse[r] = kNegInf;
    return;
  }
  const float m2 = M * kLog2e;
  float z = 0.f;
  for (int s = 0; s < num_splits; ++s) {
    const float v = part_lse[(int64_t)s * rows + r];
    if (v != kNegInf) z += exp2_hw(fmaf(v, kLog2e, -m2));
  }
  const float inv_z = 1.0f / z;
  for (int d = t * 4; d < head_dim; d += TPR * 4) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < num_splits; ++s) {
      const float v = part_lse[(int64_t)s * rows + r];
      if (v == kNegInf) continue;
      const float w = exp2_hw(fmaf(v, kLog2e, -m2)) * inv_z;
      const float4 x = *reinterpret_cast<const float4*>(part_out + ((int64_t)s * rows + r) * head_dim + d);
      o.x = fmaf(w, x.x, o.x);
      o.y = fmaf(w, x.y, o.y);
      o.z = fmaf(w, x.z, o.z);
      o.w = fmaf(w, x.w, o.w);
    }
    *reinterpret_cast<float4*>(out + (int64_t)r * head_dim + d) = o;
  }
  if (t == 0 && lse) lse[r] = M + log2_hw(z) * kLn2;
}

template <int TPR>
hipError_t launch_t(int S, int rows, int D, const float* po, const float* pl, float* out,
                    float* lse, hipStream_t st) {
  constexpr int rows_per_block = kThreads / TPR;
  const int blocks = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((splitkv_combine_kernel<TPR>), dim3(blocks), dim3(kThreads), 0, st, S, rows,
                     D, po, pl, out, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitkv_combine(int32_t S, int32_t rows, int32_t D, const float* po,
                                  const float* pl, float* out, float* lse, hipStream_t st) {
  const int vec = D / 4;
  if (vec <= 8) return launch_t<8>(S, rows, D, po, pl, out, lse, st);
  if (vec <= 16) return launch_t<16>(S, rows, D, po, pl, out, lse, st);
  if (vec <= 32) return launch_t<32>(S, rows, D, po, pl, out, lse, st);
  if (vec <= 64) return launch_t<64>(S, rows, D, po, pl, out, lse, st);
  if (vec <= 128) return launch_t<128>(S, rows, D, po, pl, out, lse, st);
  return launch_t<256>(S, rows, D, po, pl, out, lse, st);
}

}  // namespace da
