// GQA / MQA / MHA single-token decode, split-KV pass, for gfx950.
//
// What it computes: for each sequence b and query head h,
//   s_j = scale * q[b,h,:] . k[b, j, h / g, :],  p = softmax_j(s),  o = sum_j p_j v[b, j, h / g, :]
// over the cached rows j of one split of the sequence ("Attention variants and
// KV cache", arganzheng.life, sections 3.2-3.3 for the grouping; section 5.2
// for splitting decode attention along the sequence). Query head h reads KV
// head h / g directly from the cache, with no expanded copy (shippingwang.com
// chapter 7, section 7.3).
//
// Work decomposition (MI355X: 256 CUs, wave64):
//   grid  = (split, KV head x head sub-group, batch); block = kWaves waves
//   (4; 8 when the workgroups fill the CUs exactly once; 16 when there are
//   too few work units to give every CU two 4-wave workgroups, so that one
//   workgroup per CU still keeps 16 waves streaming).
//   A workgroup serves GH query heads that share one KV head, so each K/V byte
//   is fetched from HBM once and used GH times from registers.
//   A cache row of D elements is spread over D/8 consecutive lanes (8 elements,
//   16 or 32 bytes per lane), so one wave-wide load covers 4 (D=128) or 8 (D=64)
//   whole rows: fully used 64-byte segments on every load instruction.
//   Each group of lanes that owns a row keeps its own online-softmax state
//   (running max m, sum l, accumulator) in registers. The per-row dot products
//   are combined across the D/8 lanes with DPP row moves: for bf16 rows of 128
//   by a reduce-scatter that leaves each lane with whole scores of its own (one
//   exponential per score), otherwise by a plain all-reduce. States are merged
//   across the lanes of a wave at the end (cross-lane shuffles), then across
//   the waves through LDS.
//   Scores live in the base-2 domain: q is pre-multiplied by scale*log2(e) so
//   each softmax weight is one v_exp_f32.
#include <type_traits>

#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

constexpr int kEPL = 8;  // elements of a cache row owned by one lane

// Cache rows are read once per launch: non-temporal loads (the `nt` cache
// policy) stream them without displacing reusable lines, and measured faster
// on MI355X (about 7.0 vs 6.2 TB/s for a plain streaming read of 512 MiB).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

template <typename T>
struct Row8;

template <>
struct Row8<uint16_t> {  // bfloat16 stored as bit patterns
  struct Raw {
    uint4 w;
  };
  static __device__ __forceinline__ Raw load(const uint16_t* p) {
    return {load_stream(reinterpret_cast<const uint4*>(p))};
  }
  static __device__ __forceinline__ Raw load_plain(const uint16_t* p) {
    return {*reinterpret_cast<const uint4*>(p)};
  }
  static __device__ __forceinline__ Raw zero() { return {make_uint4(0u, 0u, 0u, 0u)}; }
  static __device__ __forceinline__ void cvt(const Raw& r, float* f) { unpack_bf16x8(r.w, f); }
};

template <>
struct Row8<float> {
  struct Raw {
    float4 a, b;
  };
  static __device__ __forceinline__ Raw load(const float* p) {
    return {load_stream(reinterpret_cast<const float4*>(p)), load_stream(reinterpret_cast<const float4*>(p) + 1)};
  }
  static __device__ __forceinline__ Raw load_plain(const float* p) {
    return {reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  static __device__ __forceinline__ Raw zero() {
    return {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
  }
  static __device__ __forceinline__ void cvt(const Raw& r, float* f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
    f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
};

// E4M3 codes, one byte each (the OCP 8-bit floating-point format; FP8 caches,
// "Attention variants and KV cache", arganzheng.life, section 6.3): 8
// elements in 8 bytes. Every E4M3 value is exactly a bf16 value, so key words
// become bf16 pairs for the dot2 score path (the conversion's scale operand is
// 1.0: it only applies a power of two), and values are converted to fp32.
template <>
struct Row8<uint8_t> {
  struct Raw {
    uint2 w;
  };
  static __device__ __forceinline__ Raw load(const uint8_t* p) {
    return {load_stream(reinterpret_cast<const uint2*>(p))};
  }
  static __device__ __forceinline__ Raw load_plain(const uint8_t* p) {
    return {*reinterpret_cast<const uint2*>(p)};
  }
  static __device__ __forceinline__ Raw zero() { return {make_uint2(0u, 0u)}; }
  static __device__ __forceinline__ void cvt(const Raw& r, float* f) {
    const uint32_t w[2] = {r.w.x, r.w.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[j], true);
      f[4 * j + 0] = lo[0];
      f[4 * j + 1] = lo[1];
      f[4 * j + 2] = hi[0];
      f[4 * j + 3] = hi[1];
    }
  }
  // the 8 elements as 4 words of bf16 pairs, in element order
  static __device__ __forceinline__ uint4 bf16x8(const Raw& r) {
    const uint32_t w[2] = {r.w.x, r.w.y};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, false));
      o[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, true));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
};

// One stage of a reduce-scatter over the 16 lanes of a row: lanes are paired
// by the DPP pattern CTRL (each pair has one "high" lane); of the n values
// of a lane, the low lane keeps the sums of the first n/2 and the high lane
// those of the last n/2. With n = 1 the stage is a plain pairwise sum.
template <int CTRL, int N>
__device__ __forceinline__ void reduce_scatter_stage(float* v, bool high) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const float lo = v[j], hi = v[j + N / 2];
      const float keep = high ? hi : lo;
      const float send = high ? lo : hi;
      v[j] = keep + dpp_mov<CTRL>(send);
    }
  } else {
    v[0] += dpp_mov<CTRL>(v[0]);
  }
}

// Lane (of a row of 16) that holds, after the reduce-scatter, the score of
// token u (of the 4 a row group handles per step) for head h, and the index
// of that score among the lane's values.
template <int GH>
__device__ __forceinline__ constexpr int rs_src_lane(int u, int h) {
  return 4 * u + (GH >= 4 ? h / (GH / 4) : h * (4 / GH));
}
template <int GH>
__device__ __forceinline__ constexpr int rs_src_reg(int h) {
  return GH >= 4 ? h % (GH / 4) : 0;
}

template <typename T, int D, int GH, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void gqa_decode_kernel(GqaArgs a) {
  constexpr int kThreads = kWaves * 64;
  constexpr int LPT = D / kEPL;   // lanes per cache row
  constexpr int RPW = 64 / LPT;   // rows covered by one wave-wide load
  constexpr int U = 16 / RPW;     // rows per lane per step
  constexpr int TOK = RPW * U;    // tokens per wave per step (16)
  using R = Row8<T>;

  const int split = blockIdx.x;
  const int b = a.order_by_length ? longest_first<kThreads>(a.seq_lens, a.batch, blockIdx.z) : blockIdx.z;
  const int n_sub = a.group / GH;
  const int kvh = blockIdx.y / n_sub;
  const int h0 = kvh * a.group + (blockIdx.y % n_sub) * GH;
  // clamped to [0, max_seq_len]: no read past the cache or the block table
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), a.max_seq_len) : a.max_seq_len;
  // sliding window: rows before w0 are neither read nor weighted; splits
  // start at w0 (paged: at the 16-row boundary below it, so steps stay
  // inside pages)
  const int w0 = a.window > 0 ? max(L - a.window, 0) : 0;
  const int t_begin = (a.page_shift > 0 ? (w0 & ~15) : w0) + split * a.chunk;
  const int t_end = min(L, t_begin + a.chunk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / LPT;
  const int col = lane % LPT;
  const bool direct = a.num_splits == 1;
  const int64_t rows = (int64_t)a.batch * a.num_q_heads;
  const int64_t r0 = (int64_t)b * a.num_q_heads + h0;

  if (t_begin >= t_end) {  // this split holds no rows of the sequence
    if (direct) {
      for (int i = threadIdx.x; i < GH * D; i += kThreads) a.out[r0 * D + i] = 0.f;
      if (threadIdx.x < GH && a.lse) a.lse[r0 + threadIdx.x] = kNegInf;
    } else if (threadIdx.x < GH) {
      a.part_lse[split * rows + r0 + threadIdx.x] = kNegInf;
    }
    return;
  }

  // Queries. bf16 (and fp8 caches, whose queries are bf16): kept as packed
  // pairs, scores by v_dot2c_f32_bf16 straight from the raw bf16 cache words
  // (or the fp8 words converted to bf16 pairs, exactly); products of bf16
  // values are exact in fp32, and the scale is applied to the reduced score.
  // fp32: converted, pre-scaled.
  constexpr bool kFp8 = sizeof(T) == 1;
  constexpr bool kBf16 = sizeof(T) <= 2;
  using TQ = typename std::conditional<kFp8, uint16_t, T>::type;
  using RQ = Row8<TQ>;
  uint32_t qp[GH][kEPL / 2];
  float qf[kBf16 ? 1 : GH][kEPL];
  {
    const TQ* qsrc = reinterpret_cast<const TQ*>(a.q) + b * a.q_sb + col * kEPL;
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const typename RQ::Raw r = RQ::load_plain(qsrc + (int64_t)(h0 + i) * a.q_sh);  // re-read by every split
      if constexpr (kBf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(&r);
        qp[i][0] = w.x; qp[i][1] = w.y; qp[i][2] = w.z; qp[i][3] = w.w;
      } else {
        RQ::cvt(r, qf[i]);
#pragma unroll
        for (int e = 0; e < kEPL; ++e) qf[i][e] *= a.scale_log2;
      }
    }
  }
  (void)qp;
  (void)qf;

  float m[GH], l[GH], acc[GH][kEPL];
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < kEPL; ++e) acc[i][e] = 0.f;
  }

  // bf16 rows of 128 with 1, 2, 4 or 8 heads per workgroup: the U x GH
  // partial dot products of a lane are reduce-scattered over the 16 lanes of
  // its row group, so each lane finishes kRsV (token, head) scores itself and
  // takes one exponential per score instead of the whole row group repeating
  // all of them. Lane c of a group then holds token u = c / 4 of the step.
  // The running max and sum live with those scores; weights and rescale
  // factors reach the lanes that hold the values by row broadcasts.
  constexpr bool kRS = kBf16 && D == 128 && (GH == 1 || GH == 2 || GH == 4 || GH == 8);
  constexpr int kRsN = U * GH;
  constexpr int kRsV = kRsN >= 16 ? kRsN / 16 : 1;
  float ms[kRsV], ls[kRsV];
#pragma unroll
  for (int k = 0; k < kRsV; ++k) {
    ms[k] = kNegInf;
    ls[k] = 0.f;
  }
  (void)ms;
  (void)ls;

  // Paged pools (arganzheng.life section 6.1): the 16 rows of a step lie in
  // one page (steps start on multiples of 16 and pages hold a power of two
  // >= 16 rows), found in the block table. A step's entry is read one step
  // before its rows are loaded and carried as the loaded value; its offset
  // is computed before the next entry is read, so the wait for it falls on a
  // load that completed with the previous step's rows. The index is clamped
  // to the last row (t_end > 0 wherever this runs), so every read is valid
  // and unconditional.
  const bool paged = a.page_shift > 0;
  const int64_t tab0 = (int64_t)b * a.max_blocks;
  const int64_t kv_b = paged ? 0 : (int64_t)b * a.kv_sb;
  const T* kp = reinterpret_cast<const T*>(a.k) + kv_b + kvh * a.kv_sh + col * kEPL;
  const T* vp = reinterpret_cast<const T*>(a.v) + kv_b + kvh * a.kv_sh + col * kEPL;
  auto step_page = [&](int base) -> int {
    return paged ? table_entry(a.block_table, tab0 + (min(base, t_end - 1) >> a.page_shift)) : 0;
  };
  // element offset of the first row of the step at `base` (page: its entry)
  auto step_off = [&](int base, int page) -> int64_t {
    if (!paged) return (int64_t)base * a.kv_st;
    return (int64_t)page * a.page_stride + (int64_t)(base & ((1 << a.page_shift) - 1)) * a.kv_st;
  };

  // key words as bf16 pairs (fp8: converted exactly)
  auto key_words = [](const typename R::Raw& r) -> uint4 {
    if constexpr (kFp8) {
      return R::bf16x8(r);
    } else {
      return *reinterpret_cast<const uint4*>(&r);
    }
  };
  (void)key_words;
  // FP8 caches: one fp32 scale per (token, KV head) for K and for V, read
  // with the step's rows. A lane needs the scales of its own rows (kSc = U),
  // or in the reduce-scatter path only of the token whose scores it finishes
  // (token (col / 4) of its row group: kSc = 1).
  constexpr int kSc = kFp8 ? (kRS ? 1 : U) : 1;
  const float* ksc = kFp8 ? a.k_scale + b * a.sc_sb + kvh * a.sc_sh : nullptr;
  const float* vsc = kFp8 ? a.v_scale + b * a.sc_sb + kvh * a.sc_sh : nullptr;
  float ksl[kSc], vsl[kSc];
  (void)ksl;
  (void)vsl;

  auto load_step = [&](int base, int64_t off, typename R::Raw (&kk)[U], typename R::Raw (&vv)[U],
                       float (&ks)[kSc], float (&vs)[kSc]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * RPW + row;
      if (base < t_end && (uint32_t)(t - w0) < (uint32_t)(t_end - w0)) {
        kk[u] = R::load(kp + off + (int64_t)(t - base) * a.kv_st);
        vv[u] = R::load(vp + off + (int64_t)(t - base) * a.kv_st);
      } else {
        kk[u] = R::zero();
        vv[u] = R::zero();
      }
    }
    if constexpr (kFp8) {
#pragma unroll
      for (int j = 0; j < kSc; ++j) {
        const int t = base + (kRS ? (col >> 2) : j) * RPW + row;
        const bool ok = (uint32_t)(t - w0) < (uint32_t)(t_end - w0);
        ks[j] = ok ? ksc[(int64_t)t * a.sc_st] : 0.f;
        vs[j] = ok ? vsc[(int64_t)t * a.sc_st] : 0.f;
      }
    }
  };
  // The rows of the next step are loaded before the math of this one, two
  // steps in flight per wave: for one bf16 head per workgroup (MHA; ragged
  // B = 64: 688 -> 680 us; with more heads it measured slower) and for fp8
  // caches, whose steps carry half the bytes, so that a wave's load latency
  // is no longer hidden by the other waves alone.
  constexpr bool kPrefetch = (sizeof(T) == 2 && GH == 1) || kFp8;
  constexpr int kStep = kWaves * TOK;
  typename R::Raw kw[U], vw[U];
  // page_n: table entry of the next step whose rows are loaded
  int page_n = step_page(t_begin + wave * TOK);
  if constexpr (kPrefetch) {
    load_step(t_begin + wave * TOK, step_off(t_begin + wave * TOK, page_n), kw, vw, ksl, vsl);
    page_n = step_page(t_begin + wave * TOK + kStep);
  }
  for (int base = t_begin + wave * TOK; base < t_end; base += kStep) {
    typename R::Raw kn[U], vn[U];
    float ksn[kSc], vsn[kSc];
    if constexpr (kPrefetch) {
      const int64_t off = step_off(base + kStep, page_n);
      page_n = step_page(base + 2 * kStep);
      load_step(base + kStep, off, kn, vn, ksn, vsn);
    } else {
      const int64_t off = step_off(base, page_n);
      page_n = step_page(base + kStep);
      load_step(base, off, kw, vw, ksl, vsl);
    }
    if constexpr (kRS) {
      float v[kRsN];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint4 w = key_words(kw[u]);
        const uint32_t kk[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < GH; ++i) {
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) d = dot2_bf16(qp[i][j], kk[j], d);
          v[u * GH + i] = d;
        }
      }
      reduce_scatter_stage<kDppRowMirror, kRsN>(v, col >= 8);
      reduce_scatter_stage<kDppRowHalfMirror, (kRsN >= 2 ? kRsN / 2 : 1)>(v, (col & 4) != 0);
      reduce_scatter_stage<kDppQuadReverse, (kRsN >= 4 ? kRsN / 4 : 1)>(v, (col & 2) != 0);
      reduce_scatter_stage<kDppQuadSwap1, (kRsN >= 8 ? kRsN / 8 : 1)>(v, (col & 1) != 0);
      const int tv = base + (col >> 2) * RPW + row;
      const bool valid = (uint32_t)(tv - w0) < (uint32_t)(t_end - w0);
      float p[kRsV], alpha[kRsV];
      bool moved = false;
#pragma unroll
      for (int k = 0; k < kRsV; ++k) {
        const float sc = valid ? v[k] * (kFp8 ? a.scale_log2 * ksl[0] : a.scale_log2) : kNegInf;
        float mx = fmaxf(sc, dpp_mov<kDppRowRor4>(sc));   // the group's 4 tokens of this head
        mx = fmaxf(mx, dpp_mov<kDppRowRor8>(mx));
        const float mn = fmaxf(ms[k], mx);
        const float mu = (mn == kNegInf) ? 0.f : mn;
        alpha[k] = exp2_hw(ms[k] - mu);
        p[k] = exp2_hw(sc - mu);
        ls[k] = ls[k] * alpha[k] + p[k];
        if constexpr (kFp8) p[k] *= vsl[0];   // the value scale rides on the weight
        moved |= mn != ms[k];
        ms[k] = mn;
      }
      if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
        for (int i = 0; i < GH; ++i) {
          const float al = row_bcast(rs_src_lane<GH>(0, i), alpha[rs_src_reg<GH>(i)]);
#pragma unroll
          for (int e = 0; e < kEPL; ++e) acc[i][e] *= al;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[kEPL];
        R::cvt(vw[u], vf);
#pragma unroll
        for (int i = 0; i < GH; ++i) {
          const float pb = row_bcast(rs_src_lane<GH>(u, i), p[rs_src_reg<GH>(i)]);
#pragma unroll
          for (int e = 0; e < kEPL; ++e) acc[i][e] = fmaf(pb, vf[e], acc[i][e]);
        }
      }
    } else {
    // scores (base-2 domain), one per (head, row of this lane group)
    float s[GH][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tv = base + u * RPW + row;
      const bool valid = (uint32_t)(tv - w0) < (uint32_t)(t_end - w0);
      if constexpr (kBf16) {
        const uint4 w = key_words(kw[u]);
        const uint32_t kk[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < GH; ++i) {
          float d = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) d = dot2_bf16(qp[i][j], kk[j], d);
          d = group_sum<LPT>(d) * (kFp8 ? a.scale_log2 * ksl[u] : a.scale_log2);
          s[i][u] = valid ? d : kNegInf;
        }
      } else {
        float kf[kEPL];
        R::cvt(kw[u], kf);
#pragma unroll
        for (int i = 0; i < GH; ++i) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < kEPL; ++e) d = fmaf(qf[i][e], kf[e], d);
          d = group_sum<LPT>(d);
          s[i][u] = valid ? d : kNegInf;
        }
      }
    }
    // online softmax: new running max, rescale, weights (s becomes p)
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      float mx = m[i];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[i][u]);
      const float mu = (mx == kNegInf) ? 0.f : mx;
      const float alpha = exp2_hw(m[i] - mu);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < kEPL; ++e) acc[i][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[i][u] = exp2_hw(s[i][u] - mu);
        l[i] += s[i][u];
        if constexpr (kFp8) s[i][u] *= vsl[u];   // the value scale rides on the weight
      }
      m[i] = mx;
    }
    // values, one row at a time
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[kEPL];
      R::cvt(vw[u], vf);
#pragma unroll
      for (int i = 0; i < GH; ++i)
#pragma unroll
        for (int e = 0; e < kEPL; ++e) acc[i][e] = fmaf(s[i][u], vf[e], acc[i][e]);
    }
    }
    if constexpr (kPrefetch) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kw[u] = kn[u];
        vw[u] = vn[u];
      }
#pragma unroll
      for (int j = 0; j < kSc; ++j) {
        ksl[j] = ksn[j];
        vsl[j] = vsn[j];
      }
    }
  }

  if constexpr (kRS) {
    // per-head running max and sum of this row group, in every lane: the sum
    // over the group's 4 token lanes, then broadcast from the head's lane
#pragma unroll
    for (int k = 0; k < kRsV; ++k) {
      ls[k] += dpp_mov<kDppRowRor4>(ls[k]);
      ls[k] += dpp_mov<kDppRowRor8>(ls[k]);
    }
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      m[i] = row_bcast(rs_src_lane<GH>(0, i), ms[rs_src_reg<GH>(i)]);
      l[i] = row_bcast(rs_src_lane<GH>(0, i), ls[rs_src_reg<GH>(i)]);
    }
  }

  // Merge the row groups of this wave: lanes with the same `col`.
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const float mo = __shfl_xor(m[i], off);
      const float lo = __shfl_xor(l[i], off);
      const MergeFactors f = merge_factors(m[i], mo);
      l[i] = l[i] * f.a + lo * f.b;
#pragma unroll
      for (int e = 0; e < kEPL; ++e) acc[i][e] = acc[i][e] * f.a + __shfl_xor(acc[i][e], off) * f.b;
      m[i] = f.m;
    }
  }

  // Merge the waves through LDS and write the result.
  __shared__ float sm_m[kWaves][GH];
  __shared__ float sm_l[kWaves][GH];
  __shared__ float sm_acc[kWaves][GH][D];
  if (row == 0) {
#pragma unroll
    for (int i = 0; i < GH; ++i) {
#pragma unroll
      for (int e = 0; e < kEPL; ++e) sm_acc[wave][i][col * kEPL + e] = acc[i][e];
      if (col == 0) {
        sm_m[wave][i] = m[i];
        sm_l[wave][i] = l[i];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GH * D; idx += kThreads) {
    const int i = idx / D;
    const int d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][i]);
    const float mu = (M == kNegInf) ? 0.f : M;
    float lsum = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_hw(sm_m[w][i] - mu);
      lsum += sm_l[w][i] * f;
      o += sm_acc[w][i][d] * f;
    }
    // lsum >= 1: the row holding the running max contributes 2^0.
    o = o / lsum;
    const float lse_v = (M + log2_hw(lsum)) * kLn2;
    const int64_t r = r0 + i;
    if (direct) {
      a.out[r * D + d] = o;
      if (d == 0 && a.lse) a.lse[r] = lse_v;
    } else {
      a.part_out[(split * rows + r) * D + d] = o;
      if (d == 0) a.part_lse[split * rows + r] = lse_v;
    }
  }
}

// 16-wave workgroups hold at most 128 registers per lane: built only for the
// instantiations that fit without spilling.
template <typename T, int GH>
constexpr bool wide_fits() {
  return sizeof(T) <= 2 ? GH <= 4 : GH <= 2;
}

template <typename T, int D, int GH>
hipError_t launch_t(const GqaArgs& a, hipStream_t st) {
  const dim3 grid(a.num_splits, a.num_kv_heads * (a.group / GH), a.batch);
  if constexpr (wide_fits<T, GH>()) {
    if (a.waves_per_block == 16) {
      hipLaunchKernelGGL((gqa_decode_kernel<T, D, GH, 16>), grid, dim3(16 * 64), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.waves_per_block == 8) {
    hipLaunchKernelGGL((gqa_decode_kernel<T, D, GH, 8>), grid, dim3(8 * 64), 0, st, a);
    return hipGetLastError();
  }
  if (a.waves_per_block != 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gqa_decode_kernel<T, D, GH, 4>), grid, dim3(4 * 64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_gh(const GqaArgs& a, hipStream_t st) {
  switch (a.heads_per_block) {
    case 1: return launch_t<T, D, 1>(a, st);
    case 2: return launch_t<T, D, 2>(a, st);
    case 3: return launch_t<T, D, 3>(a, st);
    case 4: return launch_t<T, D, 4>(a, st);
    case 5: return launch_t<T, D, 5>(a, st);
    case 6: return launch_t<T, D, 6>(a, st);
    case 7: return launch_t<T, D, 7>(a, st);
    case 8: return launch_t<T, D, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gqa_wide_supported(int dtype, int heads_per_block) {
  return dtype != 0 ? heads_per_block <= 4 : heads_per_block <= 2;
}

hipError_t launch_gqa_decode(const GqaArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (gqa_mfma_supported(a, dtype, head_dim)) return launch_gqa_mfma(a, dtype, head_dim, st);
  if (dtype == 1) {
    if (head_dim == 128) return launch_gh<uint16_t, 128>(a, st);
    if (head_dim == 64) return launch_gh<uint16_t, 64>(a, st);
  } else if (dtype == 0) {
    if (head_dim == 128) return launch_gh<float, 128>(a, st);
    if (head_dim == 64) return launch_gh<float, 64>(a, st);
  } else if (dtype == 2) {
    if (head_dim == 128) return launch_gh<uint8_t, 128>(a, st);
    if (head_dim == 64) return launch_gh<uint8_t, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace da
