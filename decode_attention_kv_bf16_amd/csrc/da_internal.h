// Host-side interfaces between the C ABI layer (api.hip) and the kernel
// launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace da {

// One GQA decode launch (split-KV pass). Everything the kernel reads.
struct GqaArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;   // may be null: every sequence has max_seq_len rows
  float* out;                // [B, Hq, D] final output (used when num_splits == 1)
  float* lse;                // [B, Hq] or null
  float* part_out;           // [S, B, Hq, D] split partials (num_splits > 1)
  float* part_lse;           // [S, B, Hq]
  int64_t q_sb, q_sh;        // element strides
  int64_t kv_sb, kv_st, kv_sh;
  int32_t batch, num_q_heads, num_kv_heads, group;   // group = Hq / Hkv
  int32_t heads_per_block;   // query heads one workgroup serves (divides group)
  int32_t waves_per_block;   // 4, 8 or 16
  int32_t order_by_length;   // 1: workgroups take sequences longest first (needs batch <= 256)
  int32_t max_seq_len, num_splits, chunk;            // chunk = tokens per split
  // Sliding window w > 0: sequence b attends rows [w0, L_b), w0 = max(0, L_b - w).
  // Splits cover rows from w0 (contiguous caches) or from w0 rounded down to a
  // multiple of 16 (paged pools, so that steps stay inside pages), and rows
  // before w0 are masked. 0: every row.
  int32_t window;
  float scale_log2;          // softmax_scale * log2(e)
  // Paged K/V pools (page_shift > 0): token t of sequence b is row
  // t & (2^page_shift - 1) of page block_table[b * max_blocks + (t >> page_shift)]
  // of each pool, pages page_stride elements apart; kv_sb is then unused.
  // chunk is a multiple of 16, so each 16-token step lies in one page.
  const int32_t* block_table;
  int32_t page_shift, max_blocks;
  int64_t page_stride;
  // FP8 (E4M3) caches (dtype 2): element (b, t, h, :) of K stands for its
  // code times k_scale[b * sc_sb + t * sc_st + h * sc_sh] (V likewise).
  const float* k_scale;
  const float* v_scale;
  int64_t sc_sb, sc_st, sc_sh;
};

// dtype: 0 = f32, 1 = bf16, 2 = fp8 E4M3 cache with bf16 queries (matches da_dtype_t).
hipError_t launch_gqa_decode(const GqaArgs& a, int dtype, int head_dim, hipStream_t stream);

// Whether 16-wave workgroups exist for this dtype and heads per workgroup.
bool gqa_wide_supported(int dtype, int heads_per_block);

// The matrix-core GQA kernel (gqa_mfma.hip): bf16 and fp8 caches, contiguous,
// 4- or 8-wave workgroups, up to 16 heads per workgroup.
bool gqa_mfma_supported(const GqaArgs& a, int dtype, int head_dim);
hipError_t launch_gqa_mfma(const GqaArgs& a, int dtype, int head_dim, hipStream_t stream);

// Log-sum-exp merge of split partials: rows = B * H.
// Streaming probes (hbm_probe.hip): bytes is a positive multiple of 16,
// depth (16-byte loads in flight per thread) is 4, 8 or 16.
hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t blocks, int32_t depth,
                              uint32_t* sink, hipStream_t st);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks,
                              int32_t depth, hipStream_t st);

hipError_t launch_splitkv_combine(int32_t num_splits, int32_t rows, int32_t head_dim,
                                  const float* part_out, const float* part_lse,
                                  float* out, float* lse, hipStream_t stream);

// Absorbed-MLA decode: three launches (query absorption, split-KV latent
// attention, merge + W_UV up-projection).
struct MlaArgs {
  const uint16_t* q_nope;    // [B, H, 128]
  const uint16_t* q_rope;    // [B, H, 64]
  const uint16_t* cache;     // row stride cache_st, batch stride cache_sb
  const int32_t* seq_lens;
  const uint16_t* w_uk;      // [H, 512, 128]
  const uint16_t* w_uv;      // [H, 512, 128]
  float* out;                // [B, H, 128]
  float* lse;                // [B, H] or null
  uint16_t* q_hat;           // [B, H, 576] bf16: [bf16(q~) | q_rope], in operand order
                             // when H is a multiple of 32 (qhat_index, mla_common.h)
  // [B, H, 512] bf16: the part of q~ that bf16(q~) leaves out, q~ - bf16(q~)
  // rounded to bf16. The scores use bf16(q~) (the matrix-core operand); the
  // merge adds scale * q~_lo . o~ to each lse, the first-order change of the
  // log-sum-exp when the scores move by scale * q~_lo . c_j.
  uint16_t* q_lo;
  // Split partials, slot-major: part_out [slots, H, 512] bf16 (each split's
  // normalised o~_s), part_lse [slots, H]. Fixed splits: slot = s * B + b
  // (num_splits per sequence, chunk rows each). Balanced splits
  // (num_splits == 0): the attention workgroups size every sequence's splits
  // from seq_lens so that all carry about the same number of tiles, give
  // sequence b the slots P_b .. P_b + S_b - 1, and record P_b, S_b in
  // split_table (2 B int32) for the merge.
  uint16_t* part_out;
  float* part_lse;
  int32_t* split_table;
  int64_t cache_sb, cache_st;
  int32_t batch, num_heads, max_seq_len, num_splits, chunk;
  int32_t wg_budget;         // balanced: tiles are spread over this many workgroups
  int32_t slots;             // rows of part_out / H
  float scale_log2;          // softmax_scale * log2(e)
  float scale;               // softmax_scale
  // Paged latent pool (page_shift > 0): token t of sequence b is row
  // t & (2^page_shift - 1) of page block_table[b * max_blocks + (t >> page_shift)],
  // pages page_stride elements apart; cache_sb is then unused. Splits start
  // on 32-row tiles, so a tile spans at most two pages.
  const int32_t* block_table;
  int32_t page_shift, max_blocks;
  int64_t page_stride;
  // E4M3 latent cache (launch_mla_attend_fp8): cache8 holds one-byte codes,
  // cache_sb and cache_st then count bytes; row (b, t) stands for
  // [decode(code[:512]) * sc_nope[b sc_sb + t sc_st] ; decode(code[512:]) * sc_rope[...]].
  const uint8_t* cache8;
  const float* sc_nope;
  const float* sc_rope;
  int64_t sc_sb, sc_st;
};

hipError_t launch_mla_absorb(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_attend(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_merge_project(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream);  // all three
// The attention stage over an E4M3 latent cache (mla_fp8.hip); absorb and
// merge are the bf16 path's. Head counts 16, 32, 48, 64, 96, 128.
hipError_t launch_mla_attend_fp8(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_decode_fp8(const MlaArgs& a, hipStream_t stream);  // absorb, attend_fp8, merge

// Cache append with rotary embedding (append_rope.hip): one launch.
struct AppendArgs {
  const void* q;             // queries to rotate: GQA q [B, Hq, D]; MLA q_rope [B, H, 64]
  void* q_out;               // same strides as q (may be q)
  int64_t q_sb, q_sh;        // element strides
  const void* k_new;         // GQA: new keys [B, Hkv, D]; MLA: new rows [B, 576] = [c_kv | k_rope]
  const void* v_new;         // GQA: new values [B, Hkv, D]; MLA: unused
  int64_t new_sb, new_sh;    // strides of k_new and v_new (MLA: new_sb only)
  const int32_t* positions;  // [B]: cache row and rotation position; outside [0, max_seq_len): skipped
  void* k_cache;             // GQA K cache / MLA latent cache
  void* v_cache;             // GQA V cache
  int64_t c_sb, c_st, c_sh;  // cache strides (c_sb unused when paged)
  const int32_t* block_table;  // paged when page_shift > 0 (as GqaArgs)
  int32_t page_shift, max_blocks;
  int64_t page_stride;
  const float* inv_freq;     // [r/2] or null: theta_i = 2^(-(2i/r) * log2_base)
  double log2_base;
  int32_t batch, q_heads, kv_heads, dim;   // dim: GQA head_dim (MLA: unused)
  int32_t rot, style, max_seq_len;         // style 0 half, 1 interleaved
  // E4M3 caches: scales of K and V rows, (b, t, h) at b*sc_sb + t*sc_st + h*sc_sh;
  // sc_st != 0: computed per (token, head) and written; sc_st == 0: read
  float* k_scale;
  float* v_scale;
  int64_t sc_sb, sc_st, sc_sh;
};

// dtype 0 f32, 1 bf16
hipError_t launch_gqa_append_rope(const AppendArgs& a, int dtype, hipStream_t stream);
hipError_t launch_mla_append_rope(const AppendArgs& a, hipStream_t stream);
hipError_t launch_gqa_append_rope_fp8(const AppendArgs& a, hipStream_t stream);

// Entry i of a paged cache's block table, read through the constant address
// space: the table is not written while a kernel runs, and so read, a load at
// a wave-uniform index becomes a scalar load (s_load). That load is counted
// by the scalar/LDS counter, not by the vector-memory counter that waits for
// cache rows, so waiting for it does not wait for rows in flight. The
// compiler makes a wave-uniform load from global memory a vector load when
// it cannot prove the memory unwritten, with exactly that wait.
__device__ __forceinline__ int32_t table_entry(const int32_t* table, int64_t i) {
  typedef const __attribute__((address_space(4))) int32_t ConstI32;
  return ((ConstI32*)table)[i];
}

// Workgroups of the MLA attention kernel for `num_heads` that one CU holds at
// once on the current device; 0 if the device cannot be queried.
int mla_attend_blocks_per_cu(int num_heads);
int mla_attend_fp8_blocks_per_cu(int num_heads);

}  // namespace da
