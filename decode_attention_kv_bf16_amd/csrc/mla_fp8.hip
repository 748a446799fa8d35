// Absorbed-MLA decode attention over an E4M3 latent cache, gfx950 (CDNA4).
//
// What it computes is the attention stage of mla_decode.hip over rows that
// are stored as 576 one-byte E4M3 codes plus two fp32 scales per (sequence,
// token): row_j = [decode(code_j[:512]) * sn_j ; decode(code_j[512:]) * sr_j]
// ("Attention variants and KV cache", arganzheng.life: section 6.3 for the
// one-byte format and the halved bytes per token, section 4.8 for the c_kv
// and k_rope ranges of a latent row being quantized apart). Scores are
//   s_j = sn_j (q~ . code_j[:512]) + sr_j (q_rope . code_j[512:]),
// and the value sum is sum_j p_j sn_j code_j[:512]; query absorption and the
// split merge with the W_UV projection are the bf16 path's kernels.
//
// Design (the 32x32x16 form of mla_decode.hip, with one-byte tiles):
//  - A 32-row tile is 18 KiB of codes (18 wave-wide 1 KiB load-to-LDS
//    copies) plus its 32 + 32 scales (two 4-byte-per-lane copies): 20 copies,
//    spread evenly over the waves (20 / NW each), issued in the shadow of the
//    score product of an earlier tile.
//  - Codes are converted to bf16 in registers after each LDS read
//    (v_cvt_scalef32_pk_bf16_fp8 with scale 1: every E4M3 value is a bf16
//    value, so the conversion is exact) and enter the same bf16 matrix ops as
//    the bf16 cache. The scales never touch the codes: the score product runs
//    as two chains, c_kv columns and k_rope columns, each multiplied by its
//    token's scale in fp32 afterwards; the nope scale is folded into the
//    weight that enters the value product (p_j sn_j, rounded to bf16 as p_j
//    is for a bf16 cache), while the normaliser sums the unscaled p_j.
//  - The value operand (8 consecutive tokens of one latent column per lane)
//    comes from ds_read_b64_tr_b8, one read per matrix op. That read takes 8
//    consecutive tile rows, so the score product's row index i is mapped to
//    tile row sigma(i) (bits 2 and 3 swapped): then the 8 rows a lane group
//    reads for value step m are exactly the tokens of its score registers
//    8 m .. 8 m + 7, as in the bf16 kernel.
//  - Head counts that are not a multiple of 32 run on the next one up, with
//    zero queries for the missing heads, whose outputs are not stored.
#include "mla_common.h"

namespace da {
namespace {

constexpr int kRowB8 = kRowE;                    // 576 bytes of codes per row
constexpr int kChunks8 = kRowB8 / 16;            // 36 chunks of 16 bytes
constexpr int kTileB8 = kTok * kRowB8;           // 18432 bytes
constexpr int kTileCopies8 = kTileB8 / 1024;     // 18 wave-wide copies
// Scales of a tile after its codes, in 256-byte blocks, one per 4-byte copy.
// Contiguous caches: two copies, nope then rope, each the tile's 32 tokens
// (lanes 0-31; lanes 32-63 repeat them). Paged pools: the tile's two 16-row
// halves may lie in different pages, so four copies, nope half 0, nope half
// 1, rope half 0, rope half 1, each 16 tokens (lanes 0-15).
constexpr int kSlotB8 = kTileB8 + 1024;
static_assert(kTileB8 % 1024 == 0 && kChunks8 % 4 == 0, "tile geometry");

typedef int i32x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (two words, code k in byte k % 4 of word k / 4) -> 8 bf16
// values, exactly.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4_t o;
  o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, o);
}

// XOR swizzle of the 16-byte chunk index inside a 576-byte tile row: only the
// low 2 bits change (36 chunks = 9 aligned groups of 4). Rows r and r + 4
// differ in it, so the 8 consecutive rows of a transposing read land in 8
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 3; }

// Score row index -> tile row (swap bits 2 and 3 of the index).
__device__ __forceinline__ int sigma(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Token (tile row) of score register 4 a + r of a lane in lane group g.
__device__ __forceinline__ int reg_token(int reg, int g) {
  return 16 * (reg >> 3) + 8 * g + 4 * ((reg >> 2) & 1) + (reg & 3);
}

// The score chain of the 32x32x16 form (see qk_first in mla_common.h), with
// its A operand written by vector ALU conversions just before: a matrix op
// reading a register that a vector ALU op wrote needs 2 wait states, which
// the compiler does not insert in front of asm, so each step carries them.
__device__ __forceinline__ void qk8_first(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_next(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk8_last(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(s)
      : "v"(a), "v"(b));
}

// Where a tile's rows come from. Contiguous: one range of codes and the two
// scale ranges. Paged: each 16-row half has its own page (codes resource and
// page index, from which the scale resources are made when they are copied).
template <bool kPaged>
struct TileSrc8 {
  __amdgpu_buffer_rsrc_t codes[kPaged ? 2 : 1];
  __amdgpu_buffer_rsrc_t nope, rope;   // contiguous only
  int page[2], row0[2], rows[2];       // paged only: page, first row in it, valid rows
};

// grid (split, sequence) or (slot) as mla_attend32_kernel; NW waves of 32
// heads (NW in 1, 2, 4).
template <int NW, bool kPaged>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attend_fp8_kernel(MlaArgs a) {
  constexpr int kScaleOps = kPaged ? 4 : 2;
  constexpr int kTileOps = kTileCopies8 + kScaleOps;  // copies per tile
  constexpr int kOps = (kTileOps + NW - 1) / NW;       // copies of the busiest wave per tile
  // scale block of range r (0 nope, 1 rope) for tokens 16 hf .. 16 hf + 15
  constexpr int kRangeStride = kPaged ? 512 : 256;
  constexpr int kHalfStride = kPaged ? 256 : 64;
  constexpr int kAhead = NW == 4 ? 4 : 2;        // tiles issued ahead of the score product
  constexpr int kDepth = kAhead + 2;             // + the tile being scored and the one in the value product
  static_assert((kAhead - 1) * kOps <= 63, "vmcnt range");
  static_assert(kSlotB8 % 256 == 0 && kTileCopies8 % 2 == 0, "slot geometry");
  constexpr int kRingB = kDepth * kSlotB8;
  constexpr int kStageB = NW * 32 * kOutRowB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRingB > kStageB ? kRingB : kStageB];
  LDS uint8_t* lds = (LDS uint8_t*)smem;

  const int H = a.num_heads;    // <= 32 NW; heads past H are padding
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int j16 = lane & 15, q16 = lane >> 4;
  const SplitWork work = assign_split(a, lane, blockIdx.x == 0 && w == 0);
  if (!work.valid) return;
  const int b = work.b;
  const int64_t slot = work.slot;
  int t_begin = work.t_begin;   // re-read per pass of the restart loop (see there)
  const int t_end = work.t_end;
  const int h = 32 * w + l32;

  if (t_begin >= t_end) {  // fixed splits only: a split past the sequence's end
    for (int i = tid; i < H; i += NW * 64) a.part_lse[slot * H + i] = kNegInf;
    return;
  }
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;

  // Copy k of this wave is tile copy j = w + NW k (k < n_ops): j < 18 is
  // 1 KiB of codes (lane l fills tile byte 1024 j + 16 l: row R, physical
  // chunk pc, from logical chunk pc ^ swz8(R); paged: copies 0-8 are rows
  // 0-15, the first half, 9-17 the second); j >= 18 is scale copy e = j - 18
  // into scale block e.
  // this wave's copies per tile (paged, 4 waves: 6 for waves 0-1, 5 for 2-3)
  const int n_ops = (kTileOps - w + NW - 1) / NW;
  const uint32_t row_bytes = (uint32_t)a.cache_st;
  const uint32_t sc_off = (uint32_t)((kPaged ? (lane & 15) : l32) * a.sc_st * 4);
  // The code copy (0..17) that this wave's copy k makes, or -1 for a scale
  // copy; the same assignment as issue_op below.
  auto copy_index = [&](int k) {
    if (NW == 1) return k < kTileCopies8 ? k : -1;
    if (NW * (k + 1) <= kTileCopies8) return w + NW * k;
    if (kPaged) {
      if (NW == 2) return -1;                      // k = 9, 10: scales
      return k == 4 ? -1 : 16 + min(w, 1);         // k = 5: copies 16 and 17 (waves 0 and 1)
    }
    const int j = w + NW * k;
    return j < kTileCopies8 ? j : -1;
  };
  uint32_t voff[kOps];
#pragma unroll
  for (int k = 0; k < kOps; ++k) {
    const int j = copy_index(k);
    const int o = 1024 * max(j, 0) + 16 * lane;
    const int R = o / kRowB8, pc = (o - R * kRowB8) / 16;
    voff[k] = j >= 0 ? (uint32_t)(kPaged ? R & 15 : R) * row_bytes + 16u * (uint32_t)(pc ^ swz8(R)) : sc_off;
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  const int64_t tab0 = (int64_t)b * a.max_blocks;
  const int page_mask = (1 << a.page_shift) - 1;
  auto tile_src = [&](int it) {
    const int t0 = t_begin + it * kTok;
    TileSrc8<kPaged> s;
    if constexpr (kPaged) {
      int32_t pg[2];
      load_two_entries(a.block_table + tab0 + (min(t0, t_end - 1) >> a.page_shift),
                       a.block_table + tab0 + (min(t0 + 16, t_end - 1) >> a.page_shift), pg[0], pg[1]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int th = t0 + 16 * hf;
        s.page[hf] = __builtin_amdgcn_readfirstlane(pg[hf]);
        s.row0[hf] = __builtin_amdgcn_readfirstlane(th & page_mask);
        s.rows[hf] = __builtin_amdgcn_readfirstlane(min(max(t_end - th, 0), 16));
        s.codes[hf] = make_raw_rsrc(a.cache8 + (int64_t)pg[hf] * a.page_stride + (int64_t)s.row0[hf] * a.cache_st,
                                    (uint32_t)s.rows[hf] * row_bytes);
      }
    } else {
      // rows past `valid` read as zero (wave-uniform; said so for the buffer resources)
      const int valid = __builtin_amdgcn_readfirstlane(max(min(t_end - t0, kTok), 0));
      const uint32_t sbytes = valid > 0 ? (uint32_t)(((int64_t)(valid - 1) * a.sc_st + 1) * 4) : 0u;
      const int64_t sc0 = (int64_t)b * a.sc_sb + (int64_t)t0 * a.sc_st;
      s.codes[0] = make_raw_rsrc(a.cache8 + (int64_t)b * a.cache_sb + (int64_t)t0 * a.cache_st,
                                 (uint32_t)valid * row_bytes);
      s.nope = make_raw_rsrc(a.sc_nope + sc0, sbytes);
      s.rope = make_raw_rsrc(a.sc_rope + sc0, sbytes);
    }
    return s;
  };
  auto settle = [&](const TileSrc8<kPaged>& src) {
    if constexpr (kPaged) asm volatile("" ::"s"(src.codes[0]), "s"(src.codes[1]));
  };
  // scale copy e of a tile into scale block e
  auto issue_scale = [&](const TileSrc8<kPaged>& src, int e, uint32_t base) {
    const uint32_t dst = base + kTileB8 + 256u * (uint32_t)e;
    if constexpr (kPaged) {
      // (e is wave-uniform; the selects keep every operand in scalar registers)
      const bool hf = (e & 1) != 0;
      const int n = __builtin_amdgcn_readfirstlane(hf ? src.rows[1] : src.rows[0]);
      const int pgv = __builtin_amdgcn_readfirstlane(hf ? src.page[1] : src.page[0]);
      const int r0v = __builtin_amdgcn_readfirstlane(hf ? src.row0[1] : src.row0[0]);
      const float* sc = (e >> 1) ? a.sc_rope : a.sc_nope;
      const uint32_t sbytes = n > 0 ? (uint32_t)(((int64_t)(n - 1) * a.sc_st + 1) * 4) : 0u;
      copy4(make_raw_rsrc(sc + (int64_t)pgv * a.sc_sb + (int64_t)r0v * a.sc_st, sbytes), sc_off, dst);
    } else {
      copy4(e ? src.rope : src.nope, sc_off, dst);
    }
  };
  // Copy k of this wave. Which kind of copy a k is must not depend on the
  // wave at run time beyond one plain branch: a per-copy test of the copy
  // index inside the unrolled score loop multiplied the code and pushed the
  // absorbed queries into scratch memory (whose loads wait for every copy in
  // flight). Scale copy e of a wave is chosen by selects.
  auto issue_op = [&](const TileSrc8<kPaged>& src, int k, int buf) {
    const uint32_t base = lds0 + (uint32_t)(buf * kSlotB8);
    auto codes = [&](int j) {   // j < 18, wave-uniform
      const bool hf = kPaged && j >= kTileCopies8 / 2;
      copy16(hf ? src.codes[kPaged ? 1 : 0] : src.codes[0], voff[k], base + 1024u * (uint32_t)j);
    };
    if (NW == 1) {              // one wave: every index is known here
      if (k < kTileCopies8)
        codes(k);
      else
        issue_scale(src, k - kTileCopies8, base);
    } else if (NW * (k + 1) <= kTileCopies8) {   // codes for every wave
      codes(w + NW * k);
    } else if constexpr (kPaged) {
      if (NW == 2) {
        issue_scale(src, 2 * (k - 9) + w, base);      // k = 9: nope of half w; k = 10: rope of half w
      } else if (k == 4) {
        issue_scale(src, w, base);                    // wave w: scale copy w
      } else if (w < 2) {
        codes(16 + w);                                // k = 5: copies 16 and 17 (n_ops 6 and 5)
      }
    } else {
      // contiguous, last copy: codes for w + NW k < 18, else scale copy w + NW k - 18
      const int j = w + NW * k;
      if (j < kTileCopies8)
        codes(j);
      else
        issue_scale(src, j - kTileCopies8, base);
    }
  };
  auto issue_tile = [&](int it, int buf) {
    const TileSrc8<kPaged> src = tile_src(it);
    settle(src);
#pragma unroll
    for (int k = 0; k < kOps; ++k) issue_op(src, k, buf);
  };
  // wait until this wave's copies of the oldest tile in flight have landed
  auto wait_tile = [&]() {
    if (n_ops == kOps)
      wait_vm<(kAhead - 1) * kOps>();
    else
      wait_vm<(kAhead - 1) * (kOps - 1)>();
  };

  // absorbed query of the lane's head as B operands (zero for padding heads)
  bf16x8_t qb[36];
  {
    // operand order when H is a multiple of 32 (one contiguous KiB per step;
    // a wave past the last head block reads its block's first one), rows
    // otherwise
    const bool blocks = H % 32 == 0;
    const uint16_t* qp = blocks ? a.q_hat + qhat_index(a, b, min(32 * w, H - 32), 0) + 8 * lane
                                : a.q_hat + ((int64_t)b * H + min(h, H - 1)) * kRowE + 8 * g;
    const int step = blocks ? 512 : 16;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qp + step * ks);
      qb[ks] = as_bf16x8(h < H ? v : u32x4_t{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) asm volatile("" ::"v"(qb[ks]));
  }

  float m_ref = kNegInf;  // reference max (log2 units) of the lane's head, fixed by the first tile
  float thr = kNegInf;    // score above which the reference must be raised
  // score operand reads: tile row sigma(l32), logical chunk ks, half g
  const int rs = sigma(l32);
  int s_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) s_off[m] = rs * kRowB8 + 16 * (m ^ swz8(rs)) + 8 * g;
  // transposed reads of value step m, column block cb: lane j16 of group q16
  // names row 16 m + 8 (q16 / 2) + j16 / 2, logical chunk 2 cb + q16 % 2,
  // half j16 % 2, and receives column j16 of that chunk for the 8 rows
  const int r_t = 8 * (q16 >> 1) + (j16 >> 1);
  int t_off[2];
#pragma unroll
  for (int cbl = 0; cbl < 2; ++cbl) t_off[cbl] = r_t * kRowB8 + 16 * ((2 * cbl + (q16 & 1)) ^ swz8(r_t)) + 8 * (j16 & 1);
  // scales of the lane's score registers 4 a .. 4 a + 3: tokens
  // 16 (a / 2) + 8 g + 4 (a % 2) + 0..3, in range r's block of half a / 2 at
  // kRangeStride r + kHalfStride (a / 2) + 4 (8 g + 4 (a % 2))
  const int sc_lds = kTileB8 + 4 * 8 * g;

  __shared__ int restart_flag;
  if (tid == 0) restart_flag = 0;

  f32x16_t o[16];
  float l_part;  // this lane's share of sum_j 2^(s_j - m_ref) (the other tokens are in lane l ^ 32)

  constexpr int kSRing = 5;
  auto score_tile = [&](int it, int refill_it, const TileSrc8<kPaged>& refill_src, f32x16_t& sn, f32x16_t& sr) {
    const int refill_buf = refill_it % kDepth;
    const LDS uint8_t* tile = lds + (it % kDepth) * kSlotB8;
    u32x2_t ra[kSRing];
#pragma unroll
    for (int ks = 0; ks < kSRing - 1; ++ks)
      ra[ks] = *reinterpret_cast<const LDS u32x2_t*>(tile + s_off[ks & 3] + 64 * (ks >> 2));
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
#pragma unroll
      for (int k = ks * kOps / 36; k < (ks + 1) * kOps / 36; ++k) issue_op(refill_src, k, refill_buf);
      const int kn = ks + kSRing - 1;
      if (kn < 36) ra[kn % kSRing] = *reinterpret_cast<const LDS u32x2_t*>(tile + s_off[kn & 3] + 64 * (kn >> 2));
      const bf16x8_t av = fp8x8_to_bf16(ra[ks % kSRing].x, ra[ks % kSRing].y);
      if (ks == 0)
        qk8_first(sn, av, qb[0]);
      else if (ks < 32)
        qk8_next(sn, av, qb[ks]);
      else if (ks == 32)
        qk8_first(sr, av, qb[ks]);
      else if (ks < 35)
        qk8_next(sr, av, qb[ks]);
      else
        qk8_last(sr, av, qb[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // s = sn_j * (nope chain) + sr_j * (rope chain), token by token
  auto apply_scales = [&](int it, f32x16_t& sn, const f32x16_t& sr) {
    const LDS uint8_t* sc = lds + (it % kDepth) * kSlotB8 + sc_lds;
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int off = kHalfStride * (a4 >> 1) + 16 * (a4 & 1);
      const f32x4_t fn = *reinterpret_cast<const LDS f32x4_t*>(sc + off);
      const f32x4_t fr = *reinterpret_cast<const LDS f32x4_t*>(sc + kRangeStride + off);
#pragma unroll
      for (int r = 0; r < 4; ++r) sn[4 * a4 + r] = fmaf(fn[r], sn[4 * a4 + r], fr[r] * sr[4 * a4 + r]);
    }
  };
  // softmax reference of tile `it`, as in mla_attend32_kernel (rows past the
  // split end get score -inf)
  auto softmax_ref = [&](int it, f32x16_t& s) {
    const int nv = t_end - (t_begin + it * kTok);
    if (nv < kTok) {
      const int nvg = nv - 8 * g;   // register r is past the end when reg_token(r, 0) >= nvg
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (reg_token(r, 0) >= nvg) s[r] = kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
    mx = fmaxf(mx, s[15]);
    if (__builtin_amdgcn_ballot_w64(mx > thr) != 0) {
      float m2 = mx * a.scale_log2;
      m2 = fmaxf(m2, __shfl_xor(m2, 32));
      if (m_ref == kNegInf) {
        m_ref = m2;                              // first tile of the split
      } else if (m2 > m_ref + kRefHeadroom) {   // rare: restart with a raised reference
        m_ref = m2;
        restart_flag = 1;
      }
      thr = (m_ref + kRefHeadroom) / a.scale_log2;
    }
  };
  auto weight = [&](const f32x16_t& s, int r) { return exp2_hw(fmaf(s[r], a.scale_log2, -m_ref)); };
  // value-product weights p_j sn_j in bf16; the normaliser takes p_j
  auto pack = [&](int it, const float (&p)[16], bf16x8_t (&pb)[2]) {
    l_part += (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
              (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
    const LDS uint8_t* sc = lds + (it % kDepth) * kSlotB8 + sc_lds;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const f32x4_t f0 = *reinterpret_cast<const LDS f32x4_t*>(sc + kHalfStride * m);
      const f32x4_t f1 = *reinterpret_cast<const LDS f32x4_t*>(sc + kHalfStride * m + 16);
      u32x4_t pw;
      pw.x = cvt_bf16x2(p[8 * m + 0] * f0[0], p[8 * m + 1] * f0[1]);
      pw.y = cvt_bf16x2(p[8 * m + 2] * f0[2], p[8 * m + 3] * f0[3]);
      pw.z = cvt_bf16x2(p[8 * m + 4] * f1[0], p[8 * m + 5] * f1[1]);
      pw.w = cvt_bf16x2(p[8 * m + 6] * f1[2], p[8 * m + 7] * f1[3]);
      pb[m] = as_bf16x8(pw);
    }
  };
  // O^T += C^T P^T for the tile in ring buffer `buf`, matrix op k = 16 m + cb
  constexpr int kTRing = 4;
  i32x2_t tv[kTRing];
  auto read_tv = [&](const LDS uint8_t* tile, int k) {
    const int m = k >> 4, cb = k & 15;
    // chunk 2 cb + q16 % 2 = 4 (cb / 2) + (2 (cb % 2) + q16 % 2): the aligned
    // group of 4 moves by 64 bytes, the swizzled position inside it is t_off
    tv[k % kTRing] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (LDS i32x2_t*)(tile + t_off[cb & 1] + 16 * m * kRowB8 + 64 * (cb >> 1)));
  };
  auto pv_start = [&](int buf) {
    const LDS uint8_t* tile = lds + buf * kSlotB8;
#pragma unroll
    for (int k = 0; k < kTRing - 1; ++k) read_tv(tile, k);
  };
  auto pv_run = [&](int buf, const bf16x8_t (&pb)[2], auto&& extra) {
    const LDS uint8_t* tile = lds + buf * kSlotB8;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k + kTRing - 1 < 32) read_tv(tile, k + kTRing - 1);
      const int m = k >> 4, cb = k & 15;
      const i32x2_t v = tv[k % kTRing];
      o[cb] = mfma32x32x16(fp8x8_to_bf16((uint32_t)v.x, (uint32_t)v.y), pb[m], o[cb]);
      extra(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (;;) {
    // Opaque to the compiler: otherwise it hoists the first tiles' copy
    // sources out of this loop, and their scalar registers stay live (and
    // spill) through all of it.
    asm volatile("" : "+s"(t_begin));
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) o[cb] = f32x16_t{};
    l_part = 0.f;
    f32x16_t sn, sr;   // after apply_scales, sn holds the scores
    bf16x8_t pb[2];
    // the weights of tile `it` are computed in the shadow of the value
    // product of tile it - 1; tiles it + 1 .. it + kAhead - 1 are in flight
#pragma unroll
    for (int j = 0; j < kAhead; ++j) issue_tile(j, j);
    {
      const TileSrc8<kPaged> refill = tile_src(kAhead);
      wait_tile();
      tile_barrier();
      score_tile(0, kAhead, refill, sn, sr);
      apply_scales(0, sn, sr);
      softmax_ref(0, sn);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = weight(sn, r);
      pack(0, p, pb);
    }
    for (int it = 1; it < ntiles; ++it) {
      const TileSrc8<kPaged> refill = tile_src(it + kAhead);
      wait_tile();
      tile_barrier();
      score_tile(it, it + kAhead, refill, sn, sr);
      pv_start((it - 1) % kDepth);
      apply_scales(it, sn, sr);
      softmax_ref(it, sn);
      float p[16];
      pv_run((it - 1) % kDepth, pb, [&](int k) {
        if ((k & 1) == 0) p[k >> 1] = weight(sn, k >> 1);
      });
      pack(it, p, pb);
    }
    pv_start((ntiles - 1) % kDepth);
    pv_run((ntiles - 1) % kDepth, pb, [](int) {});
    wait_vm_all();
    __syncthreads();
    if (!restart_flag) break;
    __syncthreads();  // every thread has seen the flag before it is cleared
    if (tid == 0) restart_flag = 0;
  }

  // o~_s = O / l (bf16) through LDS, whole 16-byte pieces of each head's row
  // (as mla_attend32_kernel); padding heads are not stored
  float l_tot = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l_tot;
  LDS uint8_t* stage = lds + w * 32 * kOutRowB;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2_t v;
      v.x = cvt_bf16x2(o[cb][4 * i + 0] * inv, o[cb][4 * i + 1] * inv);
      v.y = cvt_bf16x2(o[cb][4 * i + 2] * inv, o[cb][4 * i + 3] * inv);
      *reinterpret_cast<LDS u32x2_t*>(stage + l32 * kOutRowB + 2 * (32 * cb + 8 * i + 4 * g)) = v;
    }
  __syncthreads();
  const int nh = min(32, H - 32 * w);   // heads of this wave that exist
  uint16_t* po = a.part_out + (slot * H + 32 * w) * kDc;
  for (int r = 0; r < nh; ++r)
    *reinterpret_cast<u32x4_t*>(po + r * kDc + 8 * lane) =
        *reinterpret_cast<const LDS u32x4_t*>(stage + r * kOutRowB + 16 * lane);
  if (g == 0 && h < H) a.part_lse[slot * H + h] = (m_ref + log2_hw(l_tot)) * kLn2;
}

template <bool kPaged, typename F>
bool with_fp8_shape(int num_heads, F&& f) {
  switch (num_heads) {
    case 16: case 32: f(mla_attend_fp8_kernel<1, kPaged>, 1); return true;
    case 48: case 64: f(mla_attend_fp8_kernel<2, kPaged>, 2); return true;
    case 96: case 128: f(mla_attend_fp8_kernel<4, kPaged>, 4); return true;
    default: return false;
  }
}

}  // namespace

hipError_t launch_mla_attend_fp8(const MlaArgs& a, hipStream_t st) {
  const dim3 grid = a.num_splits > 0 ? dim3(a.num_splits, a.batch) : dim3(a.slots, 1);
  auto launch = [&](auto kernel, int nw) { hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, st, a); };
  const bool ok = a.page_shift > 0 ? with_fp8_shape<true>(a.num_heads, launch)
                                   : with_fp8_shape<false>(a.num_heads, launch);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

int mla_attend_fp8_blocks_per_cu(int num_heads) {
  int n = 0;
  const bool ok = with_fp8_shape<false>(num_heads, [&](auto kernel, int nw) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel), 64 * nw,
                                                     0) != hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
  });
  return ok ? n : 0;
}

hipError_t launch_mla_decode_fp8(const MlaArgs& a, hipStream_t st) {
  hipError_t e = launch_mla_absorb(a, st);
  if (e != hipSuccess) return e;
  e = launch_mla_attend_fp8(a, st);
  if (e != hipSuccess) return e;
  return launch_mla_merge_project(a, st);
}

}  // namespace da
