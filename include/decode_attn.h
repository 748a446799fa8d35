/*
 * decode_attn.h -- C ABI of libdecode_attn.so: single-token decode attention
 * over a KV cache on AMD Instinct MI355X (gfx950).
 *
 * Two operations, both one layer and one new query token per sequence:
 *
 *  1. GQA / MQA / MHA decode. g = Hq / Hkv query heads share one cached K/V
 *     head; query head h reads KV head h / g (integer division), read in place
 *     with no copy of the cache. Semantics: "Attention variants and KV cache"
 *     (arganzheng.life), sections 3.1-3.3; kakack.github.io KV-cache page,
 *     section 4 (UnifiedAttention, with its Hq % Hkv == 0 requirement);
 *     shippingwang.com chapter 7, section 7.3 (the q_head // g mapping).
 *
 *  2. DeepSeek-style MLA decode with matrix absorption. Per head,
 *     q~ = q_nope W_UK^T (512-d); all heads attend one shared cached row
 *     [c_kv (512) ; k_rope (64)] with scale 1/sqrt(192); the first 512 columns
 *     of that row are the value; the 512-d result is multiplied by W_UV.
 *     arganzheng.life sections 4.2, 4.5 and 4.6; jianzhnie.github.io
 *     "Multi-head Latent Attention", sections 2 and 4.
 *
 *  Plus the split-KV merge (flash-decoding: split the cache along the
 *  sequence, softmax per split, merge the normalisers; arganzheng.life
 *  section 5.2), paged and FP8 (E4M3) caches (section 6), sliding-window
 *  GQA (section 5.3), and the step before decode: appending the new token's
 *  rows to the cache with rotary position embedding (kakack.github.io
 *  section 2.2; arganzheng.life sections 4.2 and 4.4).
 *
 * Conventions shared by every entry point
 *  - All pointers to tensors are DEVICE pointers on the current HIP device;
 *    the caller allocates and owns every buffer, including workspace. The
 *    library never allocates or frees device memory and keeps no state
 *    between calls apart from cached device properties.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *    stream). Outputs are valid once that stream has been synchronised.
 *    Calls are thread-safe. Calls that share a workspace buffer race unless
 *    they are ordered on one stream.
 *  - lse is the natural-log log-sum-exp of the scaled scores,
 *    lse = log(sum_j exp(s_j)); a sequence of length 0 yields out = 0 and
 *    lse = -inf.
 *  - Strides are in elements. The innermost (head_dim / row) axis must be
 *    contiguous; every pointer must be 16-byte aligned and every stride a
 *    multiple of 16 bytes.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns a non-zero status synchronously and launches nothing.
 *    Device-resident seq_lens are not read on the host (that would need a
 *    synchronising copy); the caller guarantees 0 <= seq_lens[b] <= max_seq_len.
 *    A launch failure returns DA_ERR_HIP. No C++ exception crosses this ABI.
 *  - The cache holds the current token already: all seq_lens[b] rows are
 *    attended and no causal mask applies at decode (kakack.github.io
 *    section 2.2; arganzheng.life section 2.2).
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define DA_EXPORT __attribute__((visibility("default")))
#else
#define DA_EXPORT
#endif

typedef enum {
  DA_OK = 0,
  DA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, stride or alignment */
  DA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim 96) */
  DA_ERR_WORKSPACE_TOO_SMALL = 3,
  DA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} da_status_t;

typedef enum {
  DA_DTYPE_F32 = 0,
  DA_DTYPE_BF16 = 1,
  DA_DTYPE_FP8_E4M3 = 2   /* GQA only, da_gqa_decode_fp8: cache in E4M3, queries in bf16 */
} da_dtype_t;

/* ------------------------------------------------------------------------ */
/* GQA / MQA / MHA decode                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t num_q_heads;     /* Hq >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;        /* D: 64 or 128 */
  int32_t max_seq_len;     /* L_max >= 1: rows allocated per sequence */
  da_dtype_t dtype;        /* element type of q, k_cache and v_cache (FP8_E4M3: see da_gqa_decode_fp8) */
  float softmax_scale;     /* usually 1/sqrt(head_dim) */
  int64_t q_stride_b;      /* q[b, h, d] at q + b*q_stride_b + h*q_stride_h + d */
  int64_t q_stride_h;
  int64_t kv_stride_b;     /* k[b, t, kh, d] at k + b*kv_stride_b + t*kv_stride_t + kh*kv_stride_h + d;
                              all strides in elements of their own array */
  int64_t kv_stride_t;     /* default layout [B, L_max, Hkv, D]: */
  int64_t kv_stride_h;     /*   kv_stride_b = L_max*Hkv*D, kv_stride_t = Hkv*D, kv_stride_h = D */
  int32_t num_splits;      /* S >= 1 forces a split count; 0 lets the library choose */
  int32_t sliding_window;  /* w >= 1: attend only rows [max(0, L_b - w), L_b) (sliding-window
                              attention, arganzheng.life section 5.3); 0: all rows */
} da_gqa_params_t;

/* Bytes of workspace da_gqa_decode needs for these parameters (0 when the
 * planned split count is 1). Returns 0 for invalid parameters as well. */
DA_EXPORT size_t da_gqa_decode_workspace_size(const da_gqa_params_t* params);

/* Split count da_gqa_decode will use for these parameters (>= 1), or 0 for
 * invalid parameters. */
DA_EXPORT int32_t da_gqa_decode_num_splits(const da_gqa_params_t* params);

/*
 * out[b, h, :] = sum_j p_j v[b, j, h/g, :] with p = softmax_j(scale * q[b,h,:] . k[b, j, h/g, :]),
 * j over [0, seq_lens[b]).
 *   q        [B, Hq, D] (strides q_stride_b, q_stride_h), dtype
 *   k_cache  [B, L_max, Hkv, D] (kv strides), dtype
 *   v_cache  same shape and strides as k_cache, dtype
 *   seq_lens [B] int32, device; NULL means every sequence has max_seq_len rows
 *   out      [B, Hq, D] float32, contiguous
 *   lse      [B, Hq] float32, contiguous; may be NULL
 *   workspace  device buffer of at least da_gqa_decode_workspace_size() bytes
 *              (may be NULL when that size is 0); its contents are scratch.
 * Rows past seq_lens[b] are never read, so they may hold anything.
 * With a sliding window w, rows before max(0, L_b - w) take no part: on a
 * contiguous cache they are not read; on paged pools the rows of the window's
 * first page from the 16-row boundary at or below L_b - w are read and given
 * weight 0 (so they must be finite), and the table entries of earlier blocks
 * are never read (their pages may be released).
 */
DA_EXPORT da_status_t da_gqa_decode(const da_gqa_params_t* params,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens,
                          float* out, float* lse,
                          void* workspace, size_t workspace_bytes,
                          void* hip_stream);

/*
 * The split pass of da_gqa_decode on its own (flash-decoding: each split of a
 * sequence is normalised locally; arganzheng.life section 5.2). With
 * S = da_gqa_decode_num_splits(params), it writes for every split s:
 *   part_out [S, B, Hq, D] float32: that split's normalised output o_s
 *   part_lse [S, B, Hq] float32:    that split's lse_s (-inf if it holds no rows)
 * Feeding them to da_splitkv_combine gives exactly what da_gqa_decode returns.
 * When S == 1 the partials are already the final out and lse.
 * Needs no workspace. Other arguments as for da_gqa_decode.
 */
DA_EXPORT da_status_t da_gqa_decode_split_pass(const da_gqa_params_t* params,
                                               const void* q, const void* k_cache,
                                               const void* v_cache, const int32_t* seq_lens,
                                               float* part_out, float* part_lse,
                                               void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Absorbed MLA decode (one shared latent KV head)                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t batch;           /* B >= 1 */
  int32_t num_heads;       /* n_h: 16, 32, 48, 64, 96 or 128 (else UNSUPPORTED) */
  int32_t kv_lora_rank;    /* d_c: must be 512 */
  int32_t qk_rope_dim;     /* d_rope: must be 64 */
  int32_t qk_nope_dim;     /* d_nope: must be 128 */
  int32_t v_head_dim;      /* d_v: must be 128 */
  int32_t max_seq_len;     /* L_max >= 1 */
  float softmax_scale;     /* 1/sqrt(qk_nope_dim + qk_rope_dim) = 1/sqrt(192) for DeepSeek-V3;
                              must be finite and > 0 (else UNSUPPORTED) */
  int64_t cache_stride_b;  /* row [b, t] at kv_cache + b*cache_stride_b + t*cache_stride_t */
  int64_t cache_stride_t;  /* default layout [B, L_max, 576]: 576*L_max and 576 */
  int32_t num_splits;      /* S >= 1 forces S splits per sequence; 0 lets the library choose */
} da_mla_params_t;

/* Splitting (flash-decoding, arganzheng.life section 5.2). The attention of a
 * sequence is split along its rows; each split leaves a partial o~_s and
 * lse_s in a "slot", and the merge combines the slots of each sequence.
 *  - Fixed splits (num_splits = S >= 1, or chosen by the library when the
 *    batch alone fills the GPU): splits of ceil(L_max / S) rows rounded up
 *    to a multiple of 32 (so at most S) per
 *    sequence, split s of sequence b in slot s*B + b.
 *  - Balanced splits (num_splits = 0 and a batch smaller than the number of
 *    resident workgroups): the split sizes are decided on the device from
 *    seq_lens so that every split carries about the same number of rows,
 *    whatever the spread of lengths; the slots of each sequence are recorded
 *    in a small table after the lse values (see da_mla_partials_size).
 * Slots hold part_out [slots, H, d_c] bf16 (normalised o~_s) and part_lse
 * [slots, H] float32 (lse_s; -inf for a split with no rows). */

/* Bytes of workspace da_mla_decode_absorbed needs (never 0 for valid
 * parameters): the absorbed-query buffer of da_mla_absorb_query (B*H*1088
 * bf16), then the two partial buffers of da_mla_partials_size, each
 * starting on a 256-byte boundary in that order. */
DA_EXPORT size_t da_mla_decode_workspace_size(const da_mla_params_t* params);

/* Fixed split count per sequence (>= 1); 0 when the splits are balanced on
 * the device; -1 if the parameters are invalid. */
DA_EXPORT int32_t da_mla_decode_num_splits(const da_mla_params_t* params);

/* Sizes in bytes of the two partial buffers that da_mla_attend_split_pass
 * writes and da_mla_merge_project reads: part_out (the o~_s of every slot)
 * and part_lse (the lse_s of every slot, followed with balanced splits by
 * the table of each sequence's slots). Their layout inside is the
 * library's. Errors: as da_mla_decode_absorbed's parameter checks, or
 * INVALID_ARGUMENT for a NULL output. */
DA_EXPORT da_status_t da_mla_partials_size(const da_mla_params_t* params,
                                           size_t* part_out_bytes, size_t* part_lse_bytes);

/*
 *   q_nope   [B, H, d_nope] bf16, contiguous
 *   q_rope   [B, H, d_rope] bf16, contiguous (RoPE already applied)
 *   kv_cache [B, L_max, d_c + d_rope] bf16; row = [c_kv | k_rope], k_rope already rotated
 *   seq_lens [B] int32, device; NULL means max_seq_len for every sequence
 *   w_uk     [H, d_c, d_nope] bf16, contiguous: per-head slice, k^C_{j,h} = c_kv_j W_UK[h]
 *   w_uv     [H, d_c, d_v] bf16, contiguous:    per-head slice, v^C_{j,h} = c_kv_j W_UV[h]
 *   out      [B, H, d_v] float32, contiguous
 *   lse      [B, H] float32, contiguous; may be NULL
 * Numerics: q~, the softmax weights, each split's o~_s and the merged o~ are
 * rounded to bf16 before they enter the matrix cores or memory; every sum is
 * accumulated in float32. The scores use bf16(q~); the part of q~ that this
 * rounding drops, q~_lo, is kept, and each lse is corrected by
 * scale * q~_lo . o~ (the first-order change of the log-sum-exp when every
 * score moves by scale * q~_lo . c_j), so lse follows the unrounded q~.
 * Equivalent to da_mla_absorb_query, da_mla_attend_split_pass and
 * da_mla_merge_project in sequence on the workspace buffers.
 */
DA_EXPORT da_status_t da_mla_decode_absorbed(const da_mla_params_t* params,
                                   const void* q_nope, const void* q_rope,
                                   const void* kv_cache, const int32_t* seq_lens,
                                   const void* w_uk, const void* w_uv,
                                   float* out, float* lse,
                                   void* workspace, size_t workspace_bytes,
                                   void* hip_stream);

/*
 * da_mla_decode_absorbed without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments, kernels and
 * results as da_mla_decode_absorbed; its workspace is a fixed scratch array
 * built into the library (da_noalloc_scratch_bytes(): 64 MiB), of which
 * every device that loads the library holds its own copy until the process
 * ends. The call allocates and frees nothing.
 * Calls that overlap on one device (other streams, other threads) share that
 * array and race: order them on one stream. Nothing needs clearing between
 * calls: every call writes each scratch byte before reading it.
 * Errors: as da_mla_decode_absorbed; WORKSPACE_TOO_SMALL (before anything is
 * launched) when these parameters need more workspace than the scratch
 * holds (da_mla_decode_workspace_size > da_noalloc_scratch_bytes); HIP when
 * the scratch's device address cannot be obtained.
 */
DA_EXPORT da_status_t da_mla_decode_absorbed_noalloc(const da_mla_params_t* params,
                                                     const void* q_nope, const void* q_rope,
                                                     const void* kv_cache, const int32_t* seq_lens,
                                                     const void* w_uk, const void* w_uv,
                                                     float* out, float* lse, void* hip_stream);

/* Bytes of the built-in scratch that da_mla_decode_absorbed_noalloc uses. */
DA_EXPORT size_t da_noalloc_scratch_bytes(void);

/* Stage 1, query-side absorption (arganzheng.life section 4.5; jianzhnie.github.io
 * section 4, "Absorb"): with q~ = q_nope[b,h] W_UK[h]^T (float32 accumulation),
 * q_hat[b, h, :] = [bf16(q~) | q_rope[b,h]].
 *   q_hat  B*H*(2 d_c + d_rope) bf16 = B*H*1088, contiguous (written): first
 *          the absorbed queries, B*H*(d_c + d_rope) values, then the low parts
 *          q~_lo [B, H, d_c] = bf16(q~ - bf16(q~)), which stage 3 uses to
 *          correct the lse. The absorbed queries are rows [B, H, d_c + d_rope]
 *          when H is not a multiple of 32; when it is, they are in the order
 *          stage 2's matrix ops read them: for each b and block of 32 heads,
 *          36 steps of 512 values, step ks holding for i < 32 and g < 2 the 8
 *          values q_hat[b, 32 blk + i, 16 ks + 8 g .. + 7] at 8 (32 g + i).
 *          Treat the buffer as opaque between the stages. */
DA_EXPORT da_status_t da_mla_absorb_query(const da_mla_params_t* params,
                                          const void* q_nope, const void* q_rope,
                                          const void* w_uk, void* q_hat, void* hip_stream);

/* Stage 2, attention of the absorbed queries over the shared latent rows,
 * split along the sequence (arganzheng.life sections 4.5 and 5.2). Writes,
 * for every split s of every sequence, o~_s = sum_{j in s} softmax_s(score)_j
 * c_kv_j and lse_s into part_out and part_lse, two device buffers of the
 * sizes da_mla_partials_size gives (16- and 4-byte aligned). */
DA_EXPORT da_status_t da_mla_attend_split_pass(const da_mla_params_t* params,
                                               const void* q_hat, const void* kv_cache,
                                               const int32_t* seq_lens,
                                               void* part_out, float* part_lse,
                                               void* hip_stream);

/* Stage 3, merge the splits by log-sum-exp, then project by W_UV
 * (arganzheng.life section 4.5, output side): out[b,h] = o~[b,h] W_UV[h];
 * lse[b,h] = log sum_s exp(lse_s) + scale * q~_lo[b,h] . o~[b,h]. q_hat is
 * stage 1's buffer (its q~_lo part is read), part_out and part_lse as
 * written by stage 2 with the same parameters. */
DA_EXPORT da_status_t da_mla_merge_project(const da_mla_params_t* params, const void* q_hat,
                                           const void* part_out, const float* part_lse,
                                           const void* w_uv, float* out, float* lse,
                                           void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Paged KV caches                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Paging ("Attention variants and KV cache", arganzheng.life, section 6.1):
 * the cache rows of each sequence are cut into blocks of page_size tokens
 * that live anywhere in a shared pool, and a per-sequence block table maps
 * logical block j to a physical page; the kernels look the table up as they
 * read the cache. Token t of sequence b is row t % page_size of page
 * block_table[b * max_blocks_per_seq + t / page_size].
 *
 * The block table is device memory and is not read on the host. The caller
 * guarantees that the entries for the blocks holding rows [0, seq_lens[b])
 * are valid pages of the pool(s); the other entries are never read. Every
 * other parameter keeps its meaning, except that the batch stride of the
 * cache (kv_stride_b, cache_stride_b) is unused: a row's place inside its
 * page is given by the token stride (kv_stride_t, cache_stride_t).
 */
typedef struct {
  const int32_t* block_table; /* [B, max_blocks_per_seq] int32, device */
  int32_t page_size;          /* rows per page: a power of two, 16 .. 2^20 */
  int32_t max_blocks_per_seq; /* row length of block_table, >= ceil(max_seq_len / page_size) */
  int64_t page_stride;        /* elements from one page of a pool to the next (> 0, 16-byte multiple) */
} da_paged_kv_t;

/* da_gqa_decode over paged pools: k_pool, v_pool [num_pages, page_size,
 * Hkv, D] in the params' token and head strides; one block table for both.
 * Splits start on multiples of 16 rows. The workspace that
 * da_gqa_decode_workspace_size reports for the same params is large enough.
 * Errors: as da_gqa_decode, and INVALID_ARGUMENT for a NULL `pages` or block
 * table, a page_size that is not a power of two in [16, 2^20], too few
 * blocks per sequence for max_seq_len, or a bad page_stride. */
DA_EXPORT da_status_t da_gqa_decode_paged(const da_gqa_params_t* params, const da_paged_kv_t* pages,
                                          const void* q, const void* k_pool, const void* v_pool,
                                          const int32_t* seq_lens, float* out, float* lse,
                                          void* workspace, size_t workspace_bytes,
                                          void* hip_stream);

/* da_mla_decode_absorbed over a paged latent pool cache_pool [num_pages,
 * page_size, 576] bf16 (row = [c_kv | k_rope]). Workspace as
 * da_mla_decode_workspace_size. Errors: as da_mla_decode_absorbed, plus the
 * paging checks of da_gqa_decode_paged. */
DA_EXPORT da_status_t da_mla_decode_absorbed_paged(const da_mla_params_t* params,
                                                   const da_paged_kv_t* pages,
                                                   const void* q_nope, const void* q_rope,
                                                   const void* cache_pool, const int32_t* seq_lens,
                                                   const void* w_uk, const void* w_uv,
                                                   float* out, float* lse, void* workspace,
                                                   size_t workspace_bytes, void* hip_stream);

/* Stage 2 (da_mla_attend_split_pass) over a paged latent pool; its partials
 * have the layout that da_mla_merge_project reads for the same params. */
DA_EXPORT da_status_t da_mla_attend_split_pass_paged(const da_mla_params_t* params,
                                                     const da_paged_kv_t* pages, const void* q_hat,
                                                     const void* cache_pool, const int32_t* seq_lens,
                                                     void* part_out, float* part_lse,
                                                     void* hip_stream);

/* ------------------------------------------------------------------------ */
/* FP8 (E4M3) KV caches                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Quantized caches ("Attention variants and KV cache", arganzheng.life,
 * section 6.3): one byte per element in the E4M3 format (read here as the
 * OCP 8-bit floating-point E4M3: bias 7, largest finite 448, no infinities),
 * with fp32 scale factors, so that the bytes read at decode halve. Element
 * (b, t, h, :) of K stands for E4M3(code) * k_scale[b, t, h]; V likewise with
 * v_scale. The scale arrays are indexed through the strides below (in floats),
 * so one scale per (token, KV head), per token (stride_h = 0) or per KV head
 * (stride_b = stride_t = 0) are all the same call.
 */
typedef struct {
  const float* k_scale;   /* device, 4-byte aligned */
  const float* v_scale;   /* device, 4-byte aligned; same strides as k_scale */
  int64_t stride_b;       /* scale of (b, t, h) at b*stride_b + t*stride_t + h*stride_h (>= 0) */
  int64_t stride_t;       /* 0 .. 2^24 for decode */
  int64_t stride_h;
} da_kv_scales_t;

/* da_gqa_decode over an E4M3 cache. params->dtype must be DA_DTYPE_FP8_E4M3:
 * q is bf16 (its strides in bf16 elements), k_cache and v_cache hold one-byte
 * codes (their strides in bytes, multiples of 16). Scales are read only for
 * rows [0, seq_lens[b]). Workspace as da_gqa_decode_workspace_size for the
 * same params. Errors: as da_gqa_decode, and INVALID_ARGUMENT for another
 * dtype, a NULL `scales` or scale pointer, a misaligned scale pointer, a
 * negative scale stride or a token stride above 2^24. da_gqa_decode,
 * da_gqa_decode_split_pass and da_gqa_decode_paged reject DA_DTYPE_FP8_E4M3
 * (they have no scales); paged E4M3 pools go through da_gqa_decode_fp8_paged.
 * Layout: any strides give the same result bit for bit, but the rate differs.
 * With head_dim 128 a KV head's row is 128 bytes; stored token-major
 * ([B, L, Hkv, D]) one head's rows lie Hkv * 128 bytes apart, and the call
 * reads them about 14% slower than when each head's rows are contiguous
 * (head-major storage, [B, Hkv, L, D], passed as kv_stride_t = D and
 * kv_stride_h = L * D). Token-major scales ([B, L, Hkv]) read fastest. */
DA_EXPORT da_status_t da_gqa_decode_fp8(const da_gqa_params_t* params, const da_kv_scales_t* scales,
                                        const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* seq_lens, float* out, float* lse,
                                        void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * An absorbed-MLA latent cache in E4M3: row (b, t) is 576 one-byte codes, and
 * its two ranges carry their own fp32 scales, because the c_kv and k_rope
 * parts of a latent row have different numeric ranges ("Attention variants
 * and KV cache", arganzheng.life, section 4.8; the one-byte format, section
 * 6.3). The row stands for
 *   [E4M3(code[0:512]) * nope_scale[b, t] ; E4M3(code[512:576]) * rope_scale[b, t]].
 */
typedef struct {
  const float* nope_scale;  /* device, 4-byte aligned: scale of the c_kv range of (b, t) */
  const float* rope_scale;  /* device, 4-byte aligned: scale of the k_rope range; same strides */
  int64_t stride_b;         /* scale of (b, t) at b*stride_b + t*stride_t (floats, >= 0) */
  int64_t stride_t;         /* 0 .. 2^24 (0: one scale per sequence) */
} da_mla_scales_t;

/* Workspace of da_mla_decode_absorbed_fp8 for these params (the layout of
 * da_mla_decode_workspace_size; the split plan follows the E4M3 kernel). 0
 * for invalid parameters. */
DA_EXPORT size_t da_mla_decode_fp8_workspace_size(const da_mla_params_t* params);

/* da_mla_decode_absorbed over an E4M3 latent cache kv_codes [B, L_max, 576]
 * uint8, whose strides params->cache_stride_b and cache_stride_t count BYTES
 * here (multiples of 16; cache_stride_t >= 576). q_nope, q_rope, w_uk, w_uv,
 * out and lse as for da_mla_decode_absorbed (bf16 inputs, fp32 outputs).
 * Codes and scales are read only for rows [0, seq_lens[b]) (rows past them
 * may hold anything, NaN codes included). Every head count of
 * da_mla_decode_absorbed is supported. Errors: as da_mla_decode_absorbed,
 * and INVALID_ARGUMENT for a NULL `scales` or scale pointer, a misaligned
 * scale pointer, a negative scale stride or a token stride above 2^24. */
DA_EXPORT da_status_t da_mla_decode_absorbed_fp8(const da_mla_params_t* params,
                                                 const da_mla_scales_t* scales, const void* q_nope,
                                                 const void* q_rope, const void* kv_codes,
                                                 const int32_t* seq_lens, const void* w_uk,
                                                 const void* w_uv, float* out, float* lse,
                                                 void* workspace, size_t workspace_bytes,
                                                 void* hip_stream);

/* da_mla_decode_absorbed_fp8 over a paged E4M3 latent pool code_pool
 * [num_pages, page_size, 576] bytes (params->cache_stride_t in bytes; the
 * batch stride is unused; pages->page_stride in bytes). The scales are paged
 * like the codes: the scales of row r of page P are at P*stride_b + r*stride_t
 * of nope_scale and rope_scale. Splits start on 32-row tiles; each 16-row
 * half of a tile lies in one page. Workspace as da_mla_decode_fp8_workspace_size.
 * Errors: as da_mla_decode_absorbed_fp8, plus the paging checks of
 * da_gqa_decode_paged (a NULL `pages` is INVALID_ARGUMENT). */
DA_EXPORT da_status_t da_mla_decode_absorbed_fp8_paged(const da_mla_params_t* params,
                                                       const da_paged_kv_t* pages,
                                                       const da_mla_scales_t* scales,
                                                       const void* q_nope, const void* q_rope,
                                                       const void* code_pool, const int32_t* seq_lens,
                                                       const void* w_uk, const void* w_uv, float* out,
                                                       float* lse, void* workspace,
                                                       size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Cache append with rotary position embedding                               */
/* ------------------------------------------------------------------------ */

/*
 * The step before decode attention: each decode step computes one new k and
 * v row per sequence and appends it to the cache, where the next steps find
 * it ("KV Cache 如何影响了 LLM Inference", kakack.github.io, section 2.2).
 * Keys and queries are rotated by their position first. For MLA, one
 * projection gives 576 values per token: the first 512 are the latent c_kv
 * (normalised by the caller), the last 64 are rotated and cached as the rope
 * key that every head shares; each head's query rope part is rotated as well
 * ("Attention variants and KV cache", arganzheng.life, section 4.2;
 * jianzhnie.github.io "Multi-head Latent Attention", section 2).
 *
 * Rotation (the rotary form; the pages fix only that R_m depends on the
 * position m alone and that R_m^T R_n = R_{n-m}, arganzheng.life section
 * 4.4): the first r entries of a vector form r/2 pairs (a, b), and pair i
 * becomes (a cos phi - b sin phi, a sin phi + b cos phi), phi = m * theta_i,
 * theta_i = base^(-2i/r) or inv_freq[i]. Entries from r on are unchanged.
 * Angles are formed and reduced to [-pi, pi] in double precision, their sine
 * and cosine taken in float32, the products in float32, and each result is
 * rounded once to the row's type.
 *
 * Sequence b is appended at row m = positions[b] (also its rotation
 * position); a position outside [0, max_seq_len) skips the sequence: nothing
 * of it is written. Every other cache row is left untouched. positions is
 * device memory and not read on the host. New rows must not overlap the
 * cache; q_out may be q itself (in place) but no other overlap.
 */
typedef enum {
  DA_ROPE_HALF = 0,        /* pair i is entries (i, i + r/2) */
  DA_ROPE_INTERLEAVED = 1  /* pair i is entries (2i, 2i + 1) */
} da_rope_style_t;

typedef struct {
  int32_t rotary_dim;      /* r: a multiple of 8, 8 <= r <= head_dim (GQA) or qk_rope_dim (MLA) */
  int32_t rope_style;      /* da_rope_style_t */
  double rope_base;        /* theta_i = rope_base^(-2i/r); finite and > 1 unless inv_freq is set */
  const float* inv_freq;   /* NULL, or device [r/2] float32 theta_i (for frequency-scaled variants) */
  int64_t new_stride_b;    /* new rows: entry (b, h, d) at b*new_stride_b + h*new_stride_h + d */
  int64_t new_stride_h;    /*   (in elements, >= 0, 16-byte multiples; MLA reads new_stride_b only) */
} da_append_t;

/* GQA append: q_out[b, h] = RoPE_m(q[b, h]); k_cache[b, m, kh] = RoPE_m(k_new[b, kh]);
 * v_cache[b, m, kh] = v_new[b, kh], with m = positions[b].
 *   params   as for da_gqa_decode; dtype BF16 or F32 (FP8_E4M3: UNSUPPORTED);
 *            softmax_scale and num_splits are unused
 *   q, q_out [B, Hq, D] in the params' q strides, dtype
 *   k_new, v_new [B, Hkv, D] in the append strides, dtype
 *   positions [B] int32, device
 *   k_cache, v_cache [B, L_max, Hkv, D] in the params' kv strides, or paged
 *            pools [num_pages, page_size, Hkv, D] when `pages` is not NULL
 *            (rows then land on page block_table[b, m / page_size]; that
 *            entry must be a valid page).
 * Errors: as da_gqa_decode's checks, plus INVALID_ARGUMENT for a NULL append
 * descriptor or buffer, a rotary_dim that is not a multiple of 8 in
 * [8, head_dim], an unknown style, a base that is not finite and > 1 without
 * inv_freq, a misaligned pointer or a bad stride, and the paging checks of
 * da_gqa_decode_paged. */
DA_EXPORT da_status_t da_gqa_append_rope(const da_gqa_params_t* params, const da_append_t* append,
                                         const da_paged_kv_t* pages, const void* q, void* q_out,
                                         const void* k_new, const void* v_new,
                                         const int32_t* positions, void* k_cache, void* v_cache,
                                         void* hip_stream);

/* GQA append into an E4M3 cache (params->dtype DA_DTYPE_FP8_E4M3; the
 * quantized cache of arganzheng.life section 6.3, as da_gqa_decode_fp8 reads
 * it). q, q_out, k_new and v_new are bf16; the new key is rotated in float32
 * as by da_gqa_append_rope, then each appended (token, KV head) row x of K
 * and of V is stored as codes E4M3(x / s), rounded to nearest even with
 * magnitudes clamped to 448 (all codes 0 when s is 0), where s is
 *  - per (token, KV head), when scales->stride_t != 0: s = max|x| / 448 in
 *    float32, written to k_scale / v_scale at the row's index (the entry
 *    point writes through these pointers; stride_h must then be nonzero);
 *  - read from the arrays, when stride_t == 0 (per-head or per-tensor scales,
 *    fixed by the caller).
 * k_cache and v_cache hold one-byte codes (strides in bytes), contiguous
 * caches only: `pages` must be NULL (appending into paged E4M3 pools is
 * UNSUPPORTED; da_gqa_decode_fp8_paged reads such pools). Errors: as da_gqa_append_rope, plus those of da_gqa_decode_fp8 for
 * the scales, and UNSUPPORTED for a nonzero token stride with a zero head
 * stride. */
DA_EXPORT da_status_t da_gqa_append_rope_fp8(const da_gqa_params_t* params, const da_append_t* append,
                                             const da_paged_kv_t* pages, const da_kv_scales_t* scales,
                                             const void* q, void* q_out, const void* k_new,
                                             const void* v_new, const int32_t* positions,
                                             void* k_cache, void* v_cache, void* hip_stream);

/* MLA append: q_rope_out[b, h] = RoPE_m(q_rope[b, h]); the cache row (b, m)
 * becomes [kv_new[b, 0:512] ; RoPE_m(kv_new[b, 512:576])].
 *   params   as for da_mla_decode_absorbed (softmax_scale and num_splits unused)
 *   q_rope, q_rope_out [B, H, 64] bf16, contiguous
 *   kv_new   [B, 576] bf16, row stride append->new_stride_b
 *   kv_cache [B, L_max, 576] bf16 in the params' strides, or a paged pool
 *            [num_pages, page_size, 576] when `pages` is not NULL.
 * Errors: as da_gqa_append_rope, with rotary_dim in [8, 64]. */
DA_EXPORT da_status_t da_mla_append_rope(const da_mla_params_t* params, const da_append_t* append,
                                         const da_paged_kv_t* pages, const void* q_rope,
                                         void* q_rope_out, const void* kv_new,
                                         const int32_t* positions, void* kv_cache,
                                         void* hip_stream);

/* da_gqa_decode_fp8 over paged E4M3 pools: k_pool, v_pool [num_pages,
 * page_size, Hkv, D] codes (strides in bytes) and scales paged the same way:
 * the scale of row r of page P for KV head h is at P*stride_b + r*stride_t +
 * h*stride_h (stride_b is the scales' page stride), or one scale per head
 * (stride_b = stride_t = 0). One block table serves codes and scales
 * (arganzheng.life sections 6.1 and 6.3). Pages hold at least 32 rows (the
 * kernel's fp8 steps are 32 tokens inside one page); splits start on
 * multiples of 32 rows. Workspace as da_gqa_decode_workspace_size for the
 * same params. Errors: as da_gqa_decode_fp8 and da_gqa_decode_paged, and
 * UNSUPPORTED for pages of fewer than 32 rows or scales that vary by page
 * only (stride_t = 0 with stride_b != 0). As for da_gqa_decode_fp8, pages
 * whose codes are stored head-major ([num_pages, Hkv, page_size, D] through
 * the strides) read faster than token-major ones. */
DA_EXPORT da_status_t da_gqa_decode_fp8_paged(const da_gqa_params_t* params, const da_paged_kv_t* pages,
                                              const da_kv_scales_t* scales, const void* q,
                                              const void* k_pool, const void* v_pool,
                                              const int32_t* seq_lens, float* out, float* lse,
                                              void* workspace, size_t workspace_bytes,
                                              void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Split-KV merge                                                            */
/* ------------------------------------------------------------------------ */

/*
 * lse[r] = log(sum_s exp(partial_lse[s, r])),
 * out[r, :] = sum_s exp(partial_lse[s, r] - lse[r]) * partial_out[s, r, :]
 * for every row r = (b, h). A split with partial_lse = -inf is empty: its
 * partial_out row is never read. All splits empty gives out = 0, lse = -inf.
 *   partial_out [S, B, H, head_dim] float32, contiguous
 *   partial_lse [S, B, H] float32, contiguous
 *   out [B, H, head_dim] float32; lse [B, H] float32 (may be NULL)
 * head_dim must be a multiple of 4 and at most 1024.
 */
DA_EXPORT da_status_t da_splitkv_combine(int32_t num_splits, int32_t batch, int32_t num_heads,
                               int32_t head_dim,
                               const float* partial_out, const float* partial_lse,
                               float* out, float* lse, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Streaming probes                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Measurement aids, not part of the attention path: the rate at which this
 * device streams a large buffer out of (and back into) HBM. That rate is the
 * ceiling decode attention works against: every decode step reads each
 * sequence's whole K/V history, so at large batch that read sets the step
 * time (arganzheng.life, section 2.4).
 * Time them with events on hip_stream over a buffer well beyond the caches.
 *
 * da_probe_stream_read reads `bytes` bytes at `src` once and XORs the XOR of
 * all its 32-bit words into *sink (device memory, 4-byte aligned; the caller
 * clears it first if it wants that value). Calls sharing a sink on different
 * streams race.
 * da_probe_stream_copy copies `bytes` bytes from src to dst (no overlap).
 * bytes > 0 and a multiple of 16; src and dst 16-byte aligned. blocks is the
 * number of 256-thread workgroups (1 .. 2^20), or 0 for one per compute unit;
 * depth, the 16-byte loads each thread keeps in flight, is 4, 8 or 16.
 * Anything else returns DA_ERR_INVALID_ARGUMENT and launches nothing.
 */
DA_EXPORT da_status_t da_probe_stream_read(const void* src, int64_t bytes, int32_t blocks,
                                           int32_t depth, uint32_t* sink, void* hip_stream);
DA_EXPORT da_status_t da_probe_stream_copy(const void* src, void* dst, int64_t bytes,
                                           int32_t blocks, int32_t depth, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Miscellany                                                                */
/* ------------------------------------------------------------------------ */

/* Static, never NULL. */
DA_EXPORT const char* da_status_string(da_status_t status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
DA_EXPORT int32_t da_version(void);

/* sizeof(da_gqa_params_t), sizeof(da_mla_params_t), sizeof(da_paged_kv_t),
 * sizeof(da_kv_scales_t) and sizeof(da_append_t) as compiled, so that bindings can check their
 * struct mirrors. */
DA_EXPORT size_t da_gqa_params_size(void);
DA_EXPORT size_t da_mla_params_size(void);
DA_EXPORT size_t da_paged_kv_size(void);
DA_EXPORT size_t da_kv_scales_size(void);
DA_EXPORT size_t da_mla_scales_size(void);
DA_EXPORT size_t da_append_size(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
