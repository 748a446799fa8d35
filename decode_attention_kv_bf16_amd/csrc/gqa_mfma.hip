// GQA / MQA / MHA single-token decode on the matrix cores, for bf16 and FP8
// (E4M3) caches, gfx950.
//
// What it computes is what gqa_decode.hip computes (query head h attends KV
// head h / g over the rows of one split; "Attention variants and KV cache",
// arganzheng.life, sections 3.2-3.3 and 5.2; FP8 caches, section 6.3). The
// difference is where the arithmetic runs. A workgroup serves the GH <= 16
// query heads of one KV head; each wave takes steps of 16 tokens (bf16) or
// 32 (fp8), whose K and V rows are copied HBM -> LDS by whole rows
// (load-to-LDS, a per-wave double buffer, one step in flight):
//   S^T = K Q^T   [16 tokens x 16 heads] per D/32 MFMAs 16x16x32, the A
//                 operand (8 consecutive d of one token per lane) read from
//                 LDS with 16-byte reads;
//   P = 2^(S^T * scale * log2(e) - m_ref) per head, in the C layout of S^T,
//                 which is the B operand layout of the value product;
//   O^T += V^T P^T [D x 16 heads] from D/16 MFMAs (16x16x16 for bf16,
//                 16x16x32 for fp8): the A operand holds 4 (8) tokens of one
//                 d column per lane, read transposed (ds_read_b64_tr_b16,
//                 or _tr_b8 for fp8).
// For fp8, the contraction index of the value product runs over the 32
// tokens in the order tau(g, j) of the scores' C layout (lane group g holds
// tokens 4g..4g+3 of each 16-token half), and the _tr_b8 read takes 8
// consecutive rows, so fp8 V rows are written to LDS in tau order. Loading
// K by whole rows matters: read straight into the A layout, each load takes
// 64 bytes of 16 rows, and the keys alone streamed at 5.1 TB/s.
//
// Softmax: each head keeps a reference max m_ref; weights are
// 2^(z - m_ref) <= 2^kHeadroom. Only when some score exceeds its reference by
// more than kHeadroom (always on a wave's first step) does the wave take the
// head-wide max across its lane groups and rescale its accumulators, so the
// common step has no cross-lane work. Weights enter the value product in
// bf16 (relative error <= 2^-8 each); the normaliser sums the fp32 weights.
// FP8 codes are converted to bf16 exactly (every E4M3 value is a bf16
// value); the per-(token, KV head) key scale multiplies the score, the value
// scale the weight.
#include <type_traits>

#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

__device__ __forceinline__ u32x4_t lds_read16(const LDS uint8_t* p) { return *(const LDS u32x4_t*)p; }

constexpr float kHeadroom = 64.0f;   // log2 units a score may exceed its head's reference

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (two words) -> 8 bf16 values, exactly
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  uint4 o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, o);
}

// fp8 steps of 32 tokens: token of contraction element j of lane group g.
__device__ __forceinline__ constexpr int tau(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

template <typename T, int D, int kWaves, int kSlots>
__global__ __launch_bounds__(kWaves * 64) void gqa_mfma_kernel(GqaArgs a) {
  constexpr bool kFp8 = sizeof(T) == 1;
  constexpr int kEsz = (int)sizeof(T);
  constexpr int kTok = kFp8 ? 32 : 16;     // tokens per wave step
  constexpr int kHalves = kTok / 16;       // 16-token row blocks of the score product
  constexpr int kJ = kTok / 4;             // weights per lane per step (contraction elements)
  constexpr int kRowB = D * kEsz;          // bytes of one (token, KV head) row
  constexpr int kChunks = kRowB / 16;      // 16-byte chunks per row (a power of two)
  constexpr int kKS = D / 32;              // k-steps of the score product
  constexpr int kDB = D / 16;              // d-blocks of the value product
  constexpr int kPartB = kTok * kRowB;     // LDS bytes of one step of K (or of V)
  constexpr int kCopies = kPartB / 1024;   // wave-wide 1 KiB copies per step, each of K and V
  static_assert(kPartB % 1024 == 0, "a step of K is whole 1 KiB copies");
  constexpr int kScaleB = kFp8 ? 512 : 0;  // fp8: 64 key scales, then 64 value scales (32 used)
  constexpr int kSlotB = 2 * kPartB + kScaleB;   // [K | V | scales] of one step
  constexpr int kOps = 2 * kCopies + (kFp8 ? 2 : 0);   // vector-memory operations per step
                                                         // (per-step scale copies are issued
                                                         // even when skipped, see issue_step)
  static_assert((kSlots - 1) * kOps <= 63, "waits fit the vmcnt range");
  constexpr int kThreads = kWaves * 64;
  constexpr int kLdsB = kWaves * kSlots * kSlotB;
  constexpr int kMergeB = kWaves * 16 * (D + 2) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsB > kMergeB ? kLdsB : kMergeB];

  const int GH = a.heads_per_block;
  const int split = blockIdx.x;
  // Per-(token, KV head) fp8 scales stored token-major put the scales of a
  // token's KV heads in one 32-byte sector. Workgroups are dealt to the 8
  // XCDs round-robin by linear id, so with the natural order a sequence's KV
  // heads land on 8 different XCDs and each fetches the whole sector for its
  // 4 bytes. With one split per sequence and a multiple of 8 sequences, the
  // (head, sequence) pairs are renumbered so that all workgroups of a
  // sequence share an XCD (linear id mod 8) and its L2 serves the sector to
  // the others.
  int gy = blockIdx.y, gz = blockIdx.z;
  if (kFp8 && a.sc_st != 0 && a.sc_sh != 0 && gridDim.x == 1 && !a.order_by_length &&
      (gridDim.z & 7) == 0) {
    const int lin = blockIdx.y + gridDim.y * blockIdx.z;
    const int q = lin >> 3;
    gy = q % gridDim.y;
    gz = (lin & 7) + 8 * (q / gridDim.y);
  }
  const int b = a.order_by_length ? longest_first<kThreads>(a.seq_lens, a.batch, gz) : gz;
  const int n_sub = a.group / GH;
  const int kvh = gy / n_sub;
  const int h0 = kvh * a.group + (gy % n_sub) * GH;
  const int L = a.seq_lens ? min(max(a.seq_lens[b], 0), a.max_seq_len) : a.max_seq_len;
  // sliding window: rows before w0 are masked; splits start at w0 (paged: at
  // the 16-row boundary below it, so steps stay inside pages)
  const int w0 = a.window > 0 ? max(L - a.window, 0) : 0;
  const int t_begin = (a.page_shift > 0 ? (w0 & ~(kTok - 1)) : w0) + split * a.chunk;
  const int t_end = min(L, t_begin + a.chunk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
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

  // 16-byte chunk c of LDS row R sits at chunk c ^ swz(R): the 16 rows that
  // the 16 lanes of a group read at one logical chunk land in 16 (or all)
  // distinct chunks, so the operand reads are free of bank conflicts.
  auto swz = [](int row) { return row & (kChunks - 1); };
  // logical chunk lane group g reads at score k-step c (8 elements of d):
  // bf16 chunk 4c + g (d = 32c + 8g); fp8 chunk 4(c/2) + g holds 16 codes,
  // d = 64(c/2) + 16g, of which k-step c takes half c % 2
  auto kchunk = [&](int c) { return kFp8 ? 4 * (c >> 1) + g : 4 * c + g; };
  auto dmap = [&](int c) { return kFp8 ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g; };

  // queries: the B operand of S^T, head r of the group (zero past GH)
  bf16x8_t qb[kKS];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + b * a.q_sb + (int64_t)(h0 + min(r, GH - 1)) * a.q_sh;
#pragma unroll
    for (int c = 0; c < kKS; ++c) {
      const uint4 w = r < GH ? *reinterpret_cast<const uint4*>(qrow + dmap(c)) : make_uint4(0u, 0u, 0u, 0u);
      qb[c] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  const int64_t pitch = a.kv_st * kEsz;   // bytes from one token's row to the next
  // Paged pools (arganzheng.life section 6.1): a step of 16 tokens (bf16) or
  // 32 (fp8) starts on a multiple of its size and lies in one page of at
  // least that many rows; its page comes from the block table (step_page).
  const bool paged = a.page_shift > 0;
  const int64_t tab0 = (int64_t)b * a.max_blocks;
  const int64_t kv_b = paged ? 0 : (int64_t)b * a.kv_sb;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (kv_b + kvh * a.kv_sh) * kEsz;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + (kv_b + kvh * a.kv_sh) * kEsz;
  // fp8 scales: (b, t, h) at b sc_sb + t sc_st + h sc_sh; on paged pools the
  // scale arrays are paged like the codes: (page, row, h) at page sc_sb +
  // row sc_st + h sc_sh
  const float* ksc = kFp8 ? a.k_scale + (paged ? 0 : b * a.sc_sb) + kvh * a.sc_sh : nullptr;
  const float* vsc = kFp8 ? a.v_scale + (paged ? 0 : b * a.sc_sb) + kvh * a.sc_sh : nullptr;

  // Both K and V of a step go HBM -> LDS by whole rows (lane l of copy k
  // fills LDS byte k*1024 + 16 l: row R, physical chunk pc, from logical
  // chunk pc ^ swz(R)). K rows are in token order; V rows too for bf16, in
  // tau order for fp8 (the transposed read takes 8 consecutive rows).
  uint32_t koff[kCopies], voff[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) {
    const int o = k * 1024 + 16 * lane;
    const int R = o / kRowB, pc = (o % kRowB) / 16;
    const int lc = pc ^ swz(R);
    const int vtok = kFp8 ? tau(R >> 3, R & 7) : R;
    koff[k] = (uint32_t)(R * pitch + 16 * lc);
    voff[k] = (uint32_t)(vtok * pitch + 16 * lc);
  }
  LDS uint8_t* wlds = (LDS uint8_t*)lds + wave * kSlots * kSlotB;
  const uint32_t wlds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)wlds);
  // Every load of the loop is one of these untracked copies, kOps per step,
  // so a step's completion is an exact vmcnt wait (see wait_steps). FP8: the
  // step's 32 key and 32 value scales go to LDS too (lane l: token l % 32).
  // (Paged pools add one vector load of table entries per 64 steps; the
  // counter counts it as well, so it can only make a wait longer.)
  const uint32_t soff = (uint32_t)((lane & 31) * a.sc_st * 4);
  // one key and one value scale for the whole split (zero token stride)
  const float ks_fixed = kFp8 && a.sc_st == 0 ? ksc[0] : 0.f;
  const float vs_fixed = kFp8 && a.sc_st == 0 ? vsc[0] : 0.f;
  constexpr int kStride = kWaves * kTok;
  const int first = t_begin + wave * kTok;
  const int n = first < t_end ? (t_end - first + kStride - 1) / kStride : 0;
  // Paged pools: each step's table entry is read with a scalar load
  // (table_entry, through the constant address space) one step ahead of its
  // use. A scalar load is counted by lgkmcnt, so its wait never waits for the
  // row copies in flight; a vector load of entries read back with readlane
  // made the compiler wait for every vector load before each use (the fp8
  // path, which reads the entry twice per step, lost 25% to it). Indices are
  // clamped to the wave's last step, so every read is a valid entry.
  int32_t page_next = paged && n > 0 ? table_entry(a.block_table, tab0 + (first >> a.page_shift)) : 0;
  auto step_page = [&](int i) -> int64_t {   // called once per step, in step order
    const int64_t cur = page_next;
    const int nx = i + 1 < n ? i + 1 : n - 1;
    page_next = table_entry(a.block_table, tab0 + ((first + nx * kStride) >> a.page_shift));
    return cur;
  };
  auto issue_step = [&](int i, int slot) {
    const int t0 = first + i * kStride;
    const int valid = min(t_end - t0, kTok);   // rows past it read as zero
    const uint32_t nrec = (uint32_t)(valid * pitch);
    const int64_t page = paged ? step_page(i) : 0;
    const int64_t r0b = paged ? page * a.page_stride * kEsz + (int64_t)(t0 & ((1 << a.page_shift) - 1)) * pitch
                              : (int64_t)t0 * pitch;
    const __amdgpu_buffer_rsrc_t kr = make_raw_rsrc(kbase + r0b, nrec);
    const __amdgpu_buffer_rsrc_t vr = make_raw_rsrc(vbase + r0b, nrec);
    const uint32_t dst = wlds_addr + slot * kSlotB;
#pragma unroll
    for (int k = 0; k < kCopies; ++k) buffer_load_to_lds16(kr, koff[k], dst + k * 1024);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) buffer_load_to_lds16(vr, voff[k], dst + kPartB + k * 1024);
    if constexpr (kFp8) {
      // the scales of tokens [0, valid): ((valid - 1) * stride + 1) floats.
      // With a zero token stride the scales do not change within the split:
      // they are read once (fixed_scales), and these copies read nothing
      // (an empty range reads as zero without a memory access), so that
      // every step still counts kOps operations.
      const uint32_t srec = a.sc_st == 0 ? 0u : (uint32_t)(((valid - 1) * a.sc_st + 1) * 4);
      int64_t s0 = (int64_t)t0 * a.sc_st;
      if (paged) s0 = page * a.sc_sb + (int64_t)(t0 & ((1 << a.page_shift) - 1)) * a.sc_st;
      const __amdgpu_buffer_rsrc_t ks = make_raw_rsrc(ksc + s0, srec);
      const __amdgpu_buffer_rsrc_t vs = make_raw_rsrc(vsc + s0, srec);
      buffer_load_to_lds4(ks, soff, dst + 2 * kPartB);
      buffer_load_to_lds4(vs, soff, dst + 2 * kPartB + 256);
    }
  };
  // wait until step i has landed, when `later` steps were issued after it
  // (s_waitcnt takes an immediate: one branch per possible count)
  auto wait_steps = [](int later) {
    if constexpr (kSlots > 7) if (later >= 7) return wait_vm<7 * kOps>();
    if constexpr (kSlots > 6) if (later == 6) return wait_vm<6 * kOps>();
    if constexpr (kSlots > 5) if (later == 5) return wait_vm<5 * kOps>();
    if constexpr (kSlots > 4) if (later == 4) return wait_vm<4 * kOps>();
    if constexpr (kSlots > 3) if (later == 3) return wait_vm<3 * kOps>();
    if constexpr (kSlots > 2) if (later == 2) return wait_vm<2 * kOps>();
    if (later >= 1) return wait_vm<kOps>();
    wait_vm<0>();
  };
  static_assert(kSlots <= 8, "wait_steps covers up to 7 later steps");

  f32x4_t o[kDB];
#pragma unroll
  for (int m = 0; m < kDB; ++m) o[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_part = 0.f;

  // ---- the pieces of a step ----
  // front_a: scores of step i and their base-2 weights' exponents z (the
  // contraction element j is token 4g + j for bf16, tau(g, j) for fp8)
  struct Front {
    float z[kJ];
    float zmax;
    float vsl[kFp8 ? kJ : 1];
  };
  auto front_a = [&](int i, Front& f) {
    const int t0 = first + i * kStride;
    const LDS uint8_t* kt = wlds + (i % kSlots) * kSlotB;
    float ksl[kFp8 ? kJ : 1];
    if (kFp8 && a.sc_st == 0) {
#pragma unroll
      for (int j = 0; j < (kFp8 ? kJ : 1); ++j) {
        ksl[j] = ks_fixed;
        f.vsl[j] = vs_fixed;
      }
    } else if constexpr (kFp8) {
      // scales of tokens tau(g, 0..7) = 4g..4g+3, 16+4g..16+4g+3
      const LDS uint8_t* sk = kt + 2 * kPartB;
      const u32x4_t k0 = lds_read16(sk + 16 * g), k1 = lds_read16(sk + 64 + 16 * g);
      const u32x4_t v0 = lds_read16(sk + 256 + 16 * g), v1 = lds_read16(sk + 256 + 64 + 16 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ksl[j] = __uint_as_float(k0[j]);
        ksl[4 + j] = __uint_as_float(k1[j]);
        f.vsl[j] = __uint_as_float(v0[j]);
        f.vsl[4 + j] = __uint_as_float(v1[j]);
      }
    }
    (void)ksl;
    // s[hf][e] = S^T[token 16 hf + 4 g + e][head r]
    f32x4_t s[kHalves];
#pragma unroll
    for (int hf = 0; hf < kHalves; ++hf) {
      const int R = 16 * hf + r;
      const LDS uint8_t* krow = kt + R * kRowB;
      s[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kKS; ++c) {
        if constexpr (kFp8) {
          if ((c & 1) == 0) {
            const u32x4_t w = lds_read16(krow + 16 * (kchunk(c) ^ swz(R)));
            s[hf] = mfma32(fp8x8_to_bf16(w.x, w.y), qb[c], s[hf]);
            s[hf] = mfma32(fp8x8_to_bf16(w.z, w.w), qb[c + 1], s[hf]);
          }
        } else {
          const bf16x8_t ak = __builtin_bit_cast(bf16x8_t, lds_read16(krow + 16 * (kchunk(c) ^ swz(R))));
          s[hf] = mfma32(ak, qb[c], s[hf]);
        }
      }
    }
    f.zmax = kNegInf;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int tj = kFp8 ? tau(g, j) : 4 * g + j;
      float scl = a.scale_log2;
      if constexpr (kFp8) scl *= ksl[j];
      // row in [w0, t_end): one unsigned compare
      f.z[j] = (uint32_t)(t0 + tj - w0) < (uint32_t)(t_end - w0)
                   ? (j < 4 ? s[0][j] : s[kHalves - 1][j & 3]) * scl : kNegInf;
      f.zmax = fmaxf(f.zmax, f.z[j]);
    }
  };
  // whether some score exceeds its head's reference by more than kHeadroom
  auto needs_new_ref = [&](const Front& f) {
    return __builtin_amdgcn_ballot_w64(f.zmax > m_ref + kHeadroom) != 0;
  };
  // a new reference for every head (the max over its 4 lane groups); the
  // accumulators are rescaled to it
  auto new_ref = [&](const Front& f) {
    float mg = fmaxf(f.zmax, __shfl_xor(f.zmax, 16));
    mg = fmaxf(mg, __shfl_xor(mg, 32));
    const float m_new = fmaxf(m_ref, mg);
    const float alpha = m_ref == kNegInf ? 0.f : exp2_hw(m_ref - m_new);
#pragma unroll
    for (int m = 0; m < kDB; ++m) o[m] *= alpha;
    l_part *= alpha;
    m_ref = m_new;
  };
  // front_b: the weights as the B operand of the value product
  using PB = typename std::conditional<kFp8, bf16x8_t, i16x4_t>::type;
  auto front_b = [&](const Front& f) -> PB {
    const float mu = m_ref == kNegInf ? 0.f : m_ref;
    float p[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      p[j] = exp2_hw(f.z[j] - mu);
      l_part += p[j];
      if constexpr (kFp8) p[j] *= f.vsl[j];   // p is 0 for masked tokens
    }
    if constexpr (kFp8) {
      uint4 pw;
      pw.x = pack_bf16x2(p[0], p[1]);
      pw.y = pack_bf16x2(p[2], p[3]);
      pw.z = pack_bf16x2(p[4], p[5]);
      pw.w = pack_bf16x2(p[6], p[7]);
      return __builtin_bit_cast(bf16x8_t, pw);
    } else {
      const uint32_t pw[2] = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      return __builtin_bit_cast(i16x4_t, pw);
    }
  };
  // back: O^T[d, h] += sum_t V[t, d] P[h, t]; d-block m: d = 16 m + lane
  // column. The transposed reads do not depend on the weights.
  struct VOps {
    typename std::conditional<kFp8, i32x2_t, i16x4_t>::type av[kDB];
  };
  auto back_reads = [&](int i, VOps& v) {
    const LDS uint8_t* vt = wlds + (i % kSlots) * kSlotB + kPartB;
#pragma unroll
    for (int m = 0; m < kDB; ++m) {
      if constexpr (kFp8) {
        const int R = 8 * g + (r >> 1);
        v.av[m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS i32x2_t*)(vt + R * kRowB + 16 * (m ^ swz(R)) + 8 * (r & 1)));
      } else {
        // 4 bf16 at d = 16 m + 4 (r % 4): byte 32 m + 8 (r % 4) of the row
        const int R = 4 * g + (r >> 2);
        const int lc = 2 * m + ((r & 3) >> 1);
        v.av[m] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS i16x4_t*)(vt + R * kRowB + 16 * (lc ^ swz(R)) + 8 * (r & 1)));
      }
    }
  };
  auto back_mfma = [&](const VOps& v, const PB& pb) {
#pragma unroll
    for (int m = 0; m < kDB; ++m) {
      if constexpr (kFp8) {
        o[m] = mfma32(fp8x8_to_bf16((uint32_t)v.av[m].x, (uint32_t)v.av[m].y), pb, o[m]);
      } else {
        o[m] = mfma16(v.av[m], pb, o[m]);
      }
    }
  };

  // This wave's steps: tokens [t_begin + (i kWaves + wave) kTok, + kTok) for
  // i < n, kSlots - 1 issued ahead. Software pipeline: while the matrix
  // cores run the value product of step i, the wave computes the scores and
  // weights of step i + 1 (one wave per SIMD cannot hide a step's chain of
  // dependent operations otherwise). Only when step i + 1 needs a new
  // reference (the accumulators are rescaled) is the value product of step i
  // run first, since its weights are relative to the old one.
#pragma unroll
  for (int i = 0; i < kSlots - 1; ++i)
    if (i < n) issue_step(i, i);
  PB pb_cur{};
  if (n > 0) {
    wait_steps(min(kSlots - 2, n - 1));   // step 0 has landed
    Front f;
    front_a(0, f);
    if (needs_new_ref(f)) new_ref(f);
    pb_cur = front_b(f);
  }
  for (int i = 0; i < n; ++i) {
    // refill the buffer of step i - 1 (finished in the previous iteration)
    if (i + kSlots - 1 < n) issue_step(i + kSlots - 1, (i + kSlots - 1) % kSlots);
    VOps v;
    back_reads(i, v);
    bool done = false;
    PB pb_next{};
    if (i + 1 < n) {
      // step i + 1 has landed (the memory clobber keeps its LDS reads below)
      wait_steps(min(kSlots - 2, n - 2 - i));
      Front f;
      front_a(i + 1, f);
      if (needs_new_ref(f)) {
        back_mfma(v, pb_cur);
        done = true;
        new_ref(f);
      }
      pb_next = front_b(f);
    }
    if (!done) back_mfma(v, pb_cur);
    pb_cur = pb_next;
  }

  // Per head: the normaliser over the 4 lane groups, then the waves merged
  // through LDS (the step buffers are reused once every wave is done).
  float lsum = l_part + __shfl_xor(l_part, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();
  float* sm_o = reinterpret_cast<float*>(lds);                 // [kWaves][16][D]
  float* sm_m = sm_o + kWaves * 16 * D;                         // [kWaves][16]
  float* sm_l = sm_m + kWaves * 16;                             // [kWaves][16]
#pragma unroll
  for (int m = 0; m < kDB; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm_o[(wave * 16 + r) * D + 16 * m + 4 * g + e] = o[m][e];
  if (g == 0) {
    sm_m[wave * 16 + r] = m_ref;
    sm_l[wave * 16 + r] = lsum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GH * D; idx += kThreads) {
    const int i = idx / D;
    const int d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 16 + i]);
    const float mu = M == kNegInf ? 0.f : M;
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_hw(sm_m[w * 16 + i] - mu);
      l += sm_l[w * 16 + i] * f;
      acc += sm_o[(w * 16 + i) * D + d] * f;
    }
    // l >= 1: the lane holding a head's reference max contributes 2^0
    const float out = acc / l;
    const float lse_v = (M + log2_hw(l)) * kLn2;
    const int64_t rr = r0 + i;
    if (direct) {
      a.out[rr * D + d] = out;
      if (d == 0 && a.lse) a.lse[rr] = lse_v;
    } else {
      a.part_out[(split * rows + rr) * D + d] = out;
      if (d == 0) a.part_lse[split * rows + rr] = lse_v;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const GqaArgs& a, hipStream_t st) {
  const dim3 grid(a.num_splits, a.num_kv_heads * (a.group / a.heads_per_block), a.batch);
  // bf16: 4 waves, each with 3 steps in flight (the LDS holds 4 per wave).
  // fp8: 6 waves with one step in flight each (2 slots): six waves per CU
  // measured 6% faster than four (51.8 against 55.2 us, Llama-3-8B GQA at B
  // 32, L 4096), a wave's step work overlapping another's wait, and two
  // slots per wave about 1% faster than three, over token-major, head-major
  // and paged caches alike (A/B in one process: 52.3 against 53.3 us
  // token-major, 44.7 against 45.2 us head-major). The planner's 8-wave
  // workgroups run as these shapes with the same grid.
  if (a.waves_per_block == 8 || a.waves_per_block == 4) {
    if constexpr (sizeof(T) == 1)
      hipLaunchKernelGGL((gqa_mfma_kernel<T, D, 6, 2>), grid, dim3(6 * 64), 0, st, a);
    else
      hipLaunchKernelGGL((gqa_mfma_kernel<T, D, 4, 4>), grid, dim3(4 * 64), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gqa_mfma_supported(const GqaArgs& a, int dtype, int head_dim) {
  // paged pools: each step inside one page (bf16 16-token steps; fp8
  // 32-token steps need pages of at least 32 rows)
  return (dtype == 1 || (dtype == 2 && (a.page_shift == 0 || a.page_shift >= 5))) &&
         (head_dim == 64 || head_dim == 128) &&
         (a.waves_per_block == 4 || a.waves_per_block == 8) && a.heads_per_block <= 16;
}

hipError_t launch_gqa_mfma(const GqaArgs& a, int dtype, int head_dim, hipStream_t st) {
  if (dtype == 1) return head_dim == 128 ? launch_t<uint16_t, 128>(a, st) : launch_t<uint16_t, 64>(a, st);
  return head_dim == 128 ? launch_t<uint8_t, 128>(a, st) : launch_t<uint8_t, 64>(a, st);
}

}  // namespace da
