// C ABI of libdecode_attn.so: argument checks, split planning, workspace
// layout and kernel dispatch. Every check runs on the host before any launch.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "da_internal.h"
#include "decode_attn.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached); 256 (a full MI355X) when no
// device can be queried, so that host-only queries still answer.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides beyond 2^48 elements address nothing a device can hold; rejecting
// them first keeps every later stride product inside int64.
// Streaming probes: at most this many workgroups, 0 picking one per compute
// unit; 4, 8 or 16 loads in flight per thread.
constexpr int32_t kMaxProbeBlocks = 1 << 20;
inline int32_t probe_blocks(int32_t blocks) { return blocks == 0 ? device_cu_count() : blocks; }
inline bool probe_shape_ok(int32_t blocks, int32_t depth) {
  return blocks >= 0 && blocks <= kMaxProbeBlocks && (depth == 4 || depth == 8 || depth == 16);
}

constexpr int64_t kMaxStride = int64_t(1) << 48;
inline bool stride_in_range(int64_t s) { return s >= 0 && s <= kMaxStride; }
inline bool stride_ok(int64_t s, int64_t esz) { return stride_in_range(s) && (s * esz) % 16 == 0; }
// Token stride of fp8 scale arrays: the decode kernels copy a tile's scales
// with 32-bit byte offsets (31 tokens x 4 bytes x stride), so it is bounded.
inline bool scale_stride_t_ok(int64_t s) { return s >= 0 && s <= (int64_t(1) << 24); }

// The dtype field as the caller wrote it. A C caller may store any int32 in
// an enum field; reading one outside the enumerators through the enum type is
// undefined in C++, so the bits are copied out as an int.
inline int32_t dtype_code(const da_gqa_params_t* p) {
  int32_t v;
  static_assert(sizeof(p->dtype) == sizeof(v), "enum field is 32 bits");
  memcpy(&v, &p->dtype, sizeof(v));
  return v;
}
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// GQA
// ---------------------------------------------------------------------------

// Largest divisor of the group size that is at most 8: the number of query
// heads one workgroup serves from one pass over a KV head.
int gqa_heads_per_block(int group) {
  for (int gh = 8; gh >= 1; --gh)
    if (group % gh == 0) return gh;
  return 1;
}

da_status_t check_gqa_params(const da_gqa_params_t* p) {
  if (!p) return DA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->batch > 65535 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->max_seq_len < 1 || p->head_dim < 1 || p->num_splits < 0 || p->sliding_window < 0)
    return DA_ERR_INVALID_ARGUMENT;
  if (p->num_q_heads % p->num_kv_heads != 0) return DA_ERR_INVALID_ARGUMENT;
  if (p->num_q_heads > 65535) return DA_ERR_INVALID_ARGUMENT;
  if (p->max_seq_len > (1 << 30)) return DA_ERR_UNSUPPORTED;   // split arithmetic stays in int32
  if (dtype_code(p) != DA_DTYPE_F32 && dtype_code(p) != DA_DTYPE_BF16 && dtype_code(p) != DA_DTYPE_FP8_E4M3)
    return DA_ERR_INVALID_ARGUMENT;
  if (!isfinite(p->softmax_scale)) return DA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != 64 && p->head_dim != 128) return DA_ERR_UNSUPPORTED;
  // element bytes of q and of the cache (fp8 caches take bf16 queries)
  const int64_t q_esz = dtype_code(p) == DA_DTYPE_F32 ? 4 : 2;
  const int64_t kv_esz = dtype_code(p) == DA_DTYPE_F32 ? 4 : dtype_code(p) == DA_DTYPE_BF16 ? 2 : 1;
  const int64_t q_strides[2] = {p->q_stride_b, p->q_stride_h};
  const int64_t kv_strides[3] = {p->kv_stride_b, p->kv_stride_t, p->kv_stride_h};
  for (int64_t s : q_strides)
    if (!stride_ok(s, q_esz)) return DA_ERR_INVALID_ARGUMENT;
  for (int64_t s : kv_strides)
    if (!stride_ok(s, kv_esz)) return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

// Kernel dtype code (0 f32, 1 bf16, 2 fp8 cache with bf16 queries).
int gqa_kernel_dtype(const da_gqa_params_t* p) {
  return dtype_code(p) == DA_DTYPE_F32 ? 0 : dtype_code(p) == DA_DTYPE_BF16 ? 1 : 2;
}

// Split count for `units` independent work items of `len` rows each when
// `slots` workgroups can be resident at once: the s in [1, s_max] that
// minimises rounds(s) * (ceil(len / s) + overhead_rows), with rounds(s) =
// ceil(units * s / slots) waves of workgroups, each as long as its chunk plus
// a fixed per-workgroup cost. Lengths are taken as len for every item (the
// lengths themselves stay on the device).
int64_t choose_splits(int64_t units, int64_t len, int64_t slots, int64_t min_rows,
                      int64_t overhead_rows) {
  int64_t s_max = ceil_div(len, min_rows);
  s_max = s_max < 1024 ? s_max : 1024;
  int64_t best = 1, best_cost = -1;
  for (int64_t s = 1; s <= s_max; ++s) {
    const int64_t cost = ceil_div(units * s, slots) * (ceil_div(len, s) + overhead_rows);
    if (best_cost < 0 || cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

struct GqaPlan {
  int splits, chunk, heads_per_block, waves_per_block;
  size_t part_out_bytes, part_lse_bytes, workspace;
};

// align: split boundaries on multiples of this many rows (16 for paged
// pools, so that every 16-row step of the kernel lies in one page)
GqaPlan plan_gqa(const da_gqa_params_t* p, int align = 1) {
  GqaPlan pl{};
  const int group = p->num_q_heads / p->num_kv_heads;
  pl.heads_per_block = gqa_heads_per_block(group);
  const int64_t units = (int64_t)p->batch * p->num_kv_heads * (group / pl.heads_per_block);
  // The pass streams the cache once and is bound by HBM. Measured on MI355X:
  // 8-16 waves per CU saturate it; every split beyond that only adds partial
  // rows, a merge and per-workgroup start-up; and with many units the
  // hardware's workgroup dispatch balances ragged lengths better than
  // splitting does. Work units are (sequence, KV head, head group).
  //  * at least 2 units per CU: one split, 4-wave workgroups;
  //  * the units divide the CUs with at most 2 splits (CUs / units in {1, 2}):
  //    8-wave workgroups, CUs / units splits, exactly one per CU (Llama-3-8B
  //    GQA at B 32, 256 units: 85.7 against 87.8 us for two 4-wave splits and a combine);
  //  * otherwise at least half a unit per CU: 4-wave workgroups, splits for 2
  //    per CU (8-wave workgroups that do not fill the CUs evenly measured up
  //    to 13% slower);
  //  * fewer units (small batches, few KV heads): 16-wave workgroups, one per
  //    CU, as many splits as fit in one round (where that shape is built).
  // Chunks stay at least 128 rows.
  const int64_t cus = device_cu_count();
  // (paged fp8 pools run on the matrix-core kernel only: no 16-wave plans)
  const bool wide = da::gqa_wide_supported(gqa_kernel_dtype(p), pl.heads_per_block) && align < 32;
  int64_t s;
  if (p->num_splits > 0) {
    s = p->num_splits;
    pl.waves_per_block = (wide && 2 * units < cus && units * s <= cus) ? 16
                         : (units * s == cus) ? 8 : 4;
  } else if (units >= 2 * cus) {
    pl.waves_per_block = 4;
    s = 1;
  } else if (2 * units >= cus && cus % units == 0) {
    pl.waves_per_block = 8;
    s = cus / units;
  } else if (2 * units >= cus || !wide) {
    pl.waves_per_block = 4;
    s = ceil_div(2 * cus, units);
  } else {
    pl.waves_per_block = 16;
    s = cus / units;
  }
  // Rows a sequence can attend: all L_max, or with a sliding window w the
  // rows [L - w, L), whose start the kernels round down to a multiple of 16
  // (32 for fp8) on paged pools: at most w + 31 rows (the same bound for
  // both, so that the workspace queries, which do not know about paging,
  // cover paged calls).
  const int64_t len = p->sliding_window > 0 && (int64_t)p->sliding_window + 31 < p->max_seq_len
                          ? (int64_t)p->sliding_window + 31 : p->max_seq_len;
  if (p->num_splits == 0) {
    const int64_t s_max = ceil_div(len, 128);
    s = s < s_max ? s : s_max;
  }
  if (s > len) s = len;
  if (s < 1) s = 1;
  pl.chunk = (int)round_up((size_t)ceil_div(len, s), (size_t)align);
  pl.splits = (int)ceil_div(len, pl.chunk);  // drop splits that would be empty
  if (pl.splits > 1) {
    const size_t rows = (size_t)p->batch * p->num_q_heads;
    pl.part_out_bytes = round_up((size_t)pl.splits * rows * p->head_dim * sizeof(float), 256);
    pl.part_lse_bytes = round_up((size_t)pl.splits * rows * sizeof(float), 256);
    pl.workspace = pl.part_out_bytes + pl.part_lse_bytes;
  }
  return pl;
}

// ---------------------------------------------------------------------------
// MLA
// ---------------------------------------------------------------------------

constexpr int kMlaDc = 512, kMlaRope = 64, kMlaNope = 128, kMlaV = 128;

struct MlaPlan;
// fp8: the attention stage reads an E4M3 latent cache (one-byte rows, its
// own kernel's occupancy)
MlaPlan plan_mla(const da_mla_params_t* p, bool fp8 = false);
bool mla_plan_oversize(const da_mla_params_t* p, bool fp8);

// Rows per sequence beyond 2^30 are refused by every entry point: split and
// chunk arithmetic then stays inside int32.
constexpr int32_t kMaxSeqLen = 1 << 30;

// cache strides count elements of the cache: bf16 (fp8 false) or bytes (fp8)
da_status_t check_mla_params(const da_mla_params_t* p, bool fp8 = false) {
  if (!p) return DA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->batch > 65535 || p->num_heads < 1 || p->max_seq_len < 1 ||
      p->num_splits < 0 || p->kv_lora_rank < 1 || p->qk_rope_dim < 0 || p->qk_nope_dim < 1 ||
      p->v_head_dim < 1)
    return DA_ERR_INVALID_ARGUMENT;
  if (!isfinite(p->softmax_scale)) return DA_ERR_INVALID_ARGUMENT;
  // the attention kernel screens raw scores against a threshold, which needs a
  // positive scale (the method's 1/sqrt(d) always is)
  if (!(p->softmax_scale > 0.0f)) return DA_ERR_UNSUPPORTED;
  if (p->kv_lora_rank != kMlaDc || p->qk_rope_dim != kMlaRope || p->qk_nope_dim != kMlaNope ||
      p->v_head_dim != kMlaV)
    return DA_ERR_UNSUPPORTED;
  // head counts with an attention-kernel shape (multiples of 16 whose
  // wave count divides a tile's 36 copies)
  switch (p->num_heads) {
    case 16: case 32: case 48: case 64: case 96: case 128: break;
    default: return DA_ERR_UNSUPPORTED;
  }
  if (p->max_seq_len > kMaxSeqLen) return DA_ERR_UNSUPPORTED;
  const int64_t esz = fp8 ? 1 : 2;
  if (!stride_ok(p->cache_stride_b, esz) || p->cache_stride_t < kMlaDc + kMlaRope ||
      p->cache_stride_t > (1 << 24) || !stride_ok(p->cache_stride_t, esz))
    return DA_ERR_INVALID_ARGUMENT;
  if (mla_plan_oversize(p, fp8)) return DA_ERR_UNSUPPORTED;
  return DA_OK;
}

struct MlaPlan {
  int splits, chunk;   // fixed splits; splits == 0: balanced on the device
  int wg_budget, slots;
  bool oversize;       // the split slots would not fit an int32 (parameters unsupported)
  size_t q_hat_bytes, part_out_bytes, part_lse_bytes, table_bytes, workspace;
};

MlaPlan plan_mla(const da_mla_params_t* p, bool fp8) {
  MlaPlan pl{};
  // One workgroup serves all heads of a split of one sequence; resident
  // workgroups from the kernel's occupancy (1 per CU when no device can be
  // asked).
  int bpc = fp8 ? da::mla_attend_fp8_blocks_per_cu(p->num_heads) : da::mla_attend_blocks_per_cu(p->num_heads);
  if (bpc < 1) bpc = 1;
  const int64_t budget = (int64_t)bpc * device_cu_count();
  const int64_t row_bytes = p->cache_stride_t * (fp8 ? 1 : 2);
  // Balanced splits when the batch alone cannot fill the GPU (and B <= 512,
  // what the device-side assignment handles): the split
  // sizes then follow the actual lengths (device-side), so ragged batches
  // keep every workgroup equally busy. A split's rows are addressed with
  // 32-bit byte offsets: its chunk must stay below 2 GiB of cache.
  const int64_t max_tiles = (int64_t)p->batch * ceil_div(p->max_seq_len, 32);
  const int64_t max_chunk_rows = 32 * ceil_div(max_tiles, budget);
  if (p->num_splits == 0 && p->batch < budget && p->batch <= 512 &&
      max_chunk_rows * row_bytes < ((int64_t)1 << 31)) {
    pl.splits = 0;
    pl.chunk = 0;
    pl.wg_budget = (int)budget;
    pl.slots = (int)(budget + p->batch);
  } else {
    int64_t s;
    if (p->num_splits > 0) {
      s = p->num_splits;
    } else {
      // splits no shorter than 128 rows, and a fixed cost of about 128 rows
      // per workgroup (loading its queries, writing its partials)
      s = choose_splits(p->batch, p->max_seq_len, budget, 128, 128);
    }
    const int64_t s_min = ceil_div((int64_t)p->max_seq_len * row_bytes, (int64_t)1 << 31);
    if (s < s_min) s = s_min;
    if (s > p->max_seq_len) s = p->max_seq_len;
    if (s < 1) s = 1;
    // splits start on 32-row tiles (paged pools then have at most two pages
    // per tile; the contiguous and the paged pass share one layout)
    pl.chunk = (int)round_up((size_t)ceil_div(p->max_seq_len, s), 32);
    pl.splits = (int)ceil_div(p->max_seq_len, pl.chunk);
    pl.wg_budget = 0;
    const int64_t slots = (int64_t)pl.splits * p->batch;
    pl.oversize = slots > INT32_MAX / 128;
    pl.slots = pl.oversize ? 0 : (int)slots;
  }
  const size_t rows = (size_t)p->batch * p->num_heads;
  // q^ [B, H, 576] bf16, then the low parts q~_lo [B, H, 512] bf16
  pl.q_hat_bytes = round_up(rows * (kMlaDc + kMlaRope + kMlaDc) * 2, 256);
  pl.part_out_bytes = round_up((size_t)pl.slots * p->num_heads * kMlaDc * 2, 256);  // bf16
  pl.table_bytes = pl.splits == 0 ? round_up((size_t)p->batch * 2 * sizeof(int32_t), 256) : 0;
  pl.part_lse_bytes = round_up((size_t)pl.slots * p->num_heads * sizeof(float), 256) + pl.table_bytes;
  pl.workspace = pl.q_hat_bytes + pl.part_out_bytes + pl.part_lse_bytes;
  return pl;
}

bool mla_plan_oversize(const da_mla_params_t* p, bool fp8) { return plan_mla(p, fp8).oversize; }

da_status_t from_hip(hipError_t e) { return e == hipSuccess ? DA_OK : DA_ERR_HIP; }

}  // namespace

namespace {

da_status_t check_gqa_buffers(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seq_lens, const float* out, const float* lse) {
  if (!q || !k_cache || !v_cache || !out) return DA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return DA_ERR_INVALID_ARGUMENT;
  if ((seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Every pointer non-null and 16-byte aligned.
da_status_t check_ptrs16(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

da::MlaArgs mla_args(const da_mla_params_t* p, const MlaPlan& pl) {
  da::MlaArgs a{};
  a.cache_sb = p->cache_stride_b;
  a.cache_st = p->cache_stride_t;
  a.batch = p->batch;
  a.num_heads = p->num_heads;
  a.max_seq_len = p->max_seq_len;
  a.num_splits = pl.splits;
  a.chunk = pl.chunk;
  a.wg_budget = pl.wg_budget;
  a.slots = pl.slots;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.scale = p->softmax_scale;
  return a;
}

// The absorbed-query buffer: q^ [B, H, 576] bf16 followed by q~_lo [B, H, 512].
void set_q_hat(da::MlaArgs& a, const void* buf) {
  uint16_t* base = static_cast<uint16_t*>(const_cast<void*>(buf));
  a.q_hat = base;
  a.q_lo = base + (size_t)a.batch * a.num_heads * (kMlaDc + kMlaRope);
}

// part_lse holds slots x H floats, then (balanced splits) the split table
void set_partials(da::MlaArgs& a, const MlaPlan& pl, void* part_out, void* part_lse) {
  a.part_out = static_cast<uint16_t*>(part_out);
  a.part_lse = static_cast<float*>(part_lse);
  a.split_table = pl.splits == 0 ? reinterpret_cast<int32_t*>(static_cast<char*>(part_lse) + pl.part_lse_bytes -
                                                                pl.table_bytes)
                                 : nullptr;
}

da::GqaArgs gqa_args(const da_gqa_params_t* p, const GqaPlan& pl, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* seq_lens) {
  da::GqaArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seq_lens = seq_lens;
  a.q_sb = p->q_stride_b;
  a.q_sh = p->q_stride_h;
  a.kv_sb = p->kv_stride_b;
  a.kv_st = p->kv_stride_t;
  a.kv_sh = p->kv_stride_h;
  a.batch = p->batch;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.heads_per_block = pl.heads_per_block;
  a.waves_per_block = pl.waves_per_block;
  // Longest sequences first, where the order can matter: when there are more
  // workgroups than stay resident at once (about 4 per CU), the last ones to
  // start decide the end of a ragged batch. The ordering is computed by every
  // workgroup, so it is limited to batches of at most 256. (Ragged MHA,
  // B = 64, 2048 workgroups: 740 -> 688 us.)
  const int64_t wgs = (int64_t)pl.splits * p->batch * p->num_kv_heads *
                      ((p->num_q_heads / p->num_kv_heads) / pl.heads_per_block);
  a.order_by_length = (seq_lens != nullptr && p->batch > 1 && p->batch <= 256 && wgs > 4 * device_cu_count()) ? 1 : 0;
  a.max_seq_len = p->max_seq_len;
  a.num_splits = pl.splits;
  a.chunk = pl.chunk;
  a.window = p->sliding_window;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  return a;
}

// Paged pools: a block table in device memory, pages of a power-of-two
// number of rows >= 16, enough table entries per sequence for max_seq_len.
da_status_t check_paged(const da_paged_kv_t* pg, int64_t max_seq_len, int64_t elem_bytes) {
  if (!pg || !pg->block_table || !aligned4(pg->block_table)) return DA_ERR_INVALID_ARGUMENT;
  const int64_t ps = pg->page_size;
  if (ps < 16 || ps > (1 << 20) || (ps & (ps - 1)) != 0) return DA_ERR_INVALID_ARGUMENT;
  if (pg->max_blocks_per_seq < ceil_div(max_seq_len, ps)) return DA_ERR_INVALID_ARGUMENT;
  if (pg->page_stride <= 0 || !stride_ok(pg->page_stride, elem_bytes)) return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

int log2_exact(int64_t x) {
  int k = 0;
  while ((int64_t{1} << k) < x) ++k;
  return k;
}

template <typename Args>
void set_paged(Args& a, const da_paged_kv_t* pg) {
  a.block_table = pg->block_table;
  a.page_shift = log2_exact(pg->page_size);
  a.max_blocks = pg->max_blocks_per_seq;
  a.page_stride = pg->page_stride;
}

// One GQA decode call: split pass (over paged pools when `pages`, over an
// fp8 cache with `scales`), then the combine when there are several splits.
da_status_t gqa_decode_impl(const da_gqa_params_t* p, const da_paged_kv_t* pages,
                            const da_kv_scales_t* scales, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* seq_lens, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  da_status_t st = check_gqa_params(p);
  if (st != DA_OK) return st;
  if (pages) {
    st = check_paged(pages, p->max_seq_len,
                     dtype_code(p) == DA_DTYPE_F32 ? 4 : dtype_code(p) == DA_DTYPE_BF16 ? 2 : 1);
    if (st != DA_OK) return st;
  }
  if (scales) {
    if (!scales->k_scale || !scales->v_scale || !aligned4(scales->k_scale) ||
        !aligned4(scales->v_scale) || !stride_in_range(scales->stride_b) || !scale_stride_t_ok(scales->stride_t) ||
        !stride_in_range(scales->stride_h))
      return DA_ERR_INVALID_ARGUMENT;
  }
  st = check_gqa_buffers(q, k_cache, v_cache, seq_lens, out, lse);
  if (st != DA_OK) return st;
  // paged calls split on multiples of 16 rows (32 for fp8), so that a step
  // never straddles a page
  const bool fp8 = dtype_code(p) == DA_DTYPE_FP8_E4M3;
  const GqaPlan pl = plan_gqa(p, pages ? (fp8 ? 32 : 16) : 1);
  if (pl.workspace > 0) {
    if (!workspace || workspace_bytes < pl.workspace) return DA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(workspace)) return DA_ERR_INVALID_ARGUMENT;
  }
  da::GqaArgs a = gqa_args(p, pl, q, k_cache, v_cache, seq_lens);
  if (pages) set_paged(a, pages);
  if (scales) {
    a.k_scale = scales->k_scale;
    a.v_scale = scales->v_scale;
    a.sc_sb = scales->stride_b;
    a.sc_st = scales->stride_t;
    a.sc_sh = scales->stride_h;
  }
  a.out = out;
  a.lse = lse;
  if (pages && fp8 && !da::gqa_mfma_supported(a, 2, p->head_dim)) return DA_ERR_UNSUPPORTED;
  if (pl.splits > 1) {
    a.part_out = reinterpret_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_out_bytes);
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = da::launch_gqa_decode(a, gqa_kernel_dtype(p), p->head_dim, stream);
  if (e != hipSuccess) return DA_ERR_HIP;
  if (pl.splits > 1) {
    e = da::launch_splitkv_combine(pl.splits, p->batch * p->num_q_heads, p->head_dim, a.part_out,
                                   a.part_lse, out, lse, stream);
  }
  return from_hip(e);
}

// Append descriptor: rotary_dim a multiple of 8 in [8, max_rot], a known
// pairing, a base > 1 or a caller table, new-row strides of 16-byte multiples.
da_status_t check_append(const da_append_t* ap, int max_rot, int64_t esz) {
  if (!ap) return DA_ERR_INVALID_ARGUMENT;
  if (ap->rotary_dim < 8 || ap->rotary_dim > max_rot || ap->rotary_dim % 8 != 0)
    return DA_ERR_INVALID_ARGUMENT;
  if (ap->rope_style != DA_ROPE_HALF && ap->rope_style != DA_ROPE_INTERLEAVED)
    return DA_ERR_INVALID_ARGUMENT;
  if (ap->inv_freq) {
    if (!aligned4(ap->inv_freq)) return DA_ERR_INVALID_ARGUMENT;
  } else if (!(isfinite(ap->rope_base) && ap->rope_base > 1.0)) {
    return DA_ERR_INVALID_ARGUMENT;
  }
  if (!stride_ok(ap->new_stride_b, esz) || !stride_ok(ap->new_stride_h, esz))
    return DA_ERR_INVALID_ARGUMENT;
  return DA_OK;
}

da::AppendArgs append_args(const da_append_t* ap, const da_paged_kv_t* pages,
                           const int32_t* positions, int batch, int max_seq_len) {
  da::AppendArgs a{};
  a.new_sb = ap->new_stride_b;
  a.new_sh = ap->new_stride_h;
  a.positions = positions;
  a.inv_freq = ap->inv_freq;
  a.log2_base = ap->inv_freq ? 0.0 : log2(ap->rope_base);
  a.rot = ap->rotary_dim;
  a.style = ap->rope_style;
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  if (pages) set_paged(a, pages);
  return a;
}

}  // namespace


// ---------------------------------------------------------------------------
// Scratch for the call that allocates nothing
// ---------------------------------------------------------------------------
// A file-scope device array in place of a caller workspace: each device that
// loads the library holds its own copy until the process ends. Host code never
// passes the array's name to a kernel (on the host it stands for a host-side
// shadow, not a device address): its device address is looked up once per
// device and kept here.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch; null if it cannot be had.
void* current_device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_addr[dev] = ptr;
  }
  return g_scratch_addr[dev];
}
}  // namespace

extern "C" {

da_status_t da_gqa_append_rope(const da_gqa_params_t* p, const da_append_t* ap,
                               const da_paged_kv_t* pages, const void* q, void* q_out,
                               const void* k_new, const void* v_new, const int32_t* positions,
                               void* k_cache, void* v_cache, void* hip_stream) {
  da_status_t st = check_gqa_params(p);
  if (st != DA_OK) return st;
  if (dtype_code(p) == DA_DTYPE_FP8_E4M3) return DA_ERR_UNSUPPORTED;
  const int64_t esz = dtype_code(p) == DA_DTYPE_BF16 ? 2 : 4;
  st = check_append(ap, p->head_dim, esz);
  if (st != DA_OK) return st;
  if (pages && (st = check_paged(pages, p->max_seq_len, esz)) != DA_OK) return st;
  st = check_ptrs16({q, q_out, k_new, v_new, k_cache, v_cache});
  if (st != DA_OK) return st;
  if (!positions || !aligned4(positions)) return DA_ERR_INVALID_ARGUMENT;
  da::AppendArgs a = append_args(ap, pages, positions, p->batch, p->max_seq_len);
  a.q = q;
  a.q_out = q_out;
  a.q_sb = p->q_stride_b;
  a.q_sh = p->q_stride_h;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.c_sb = p->kv_stride_b;
  a.c_st = p->kv_stride_t;
  a.c_sh = p->kv_stride_h;
  a.q_heads = p->num_q_heads;
  a.kv_heads = p->num_kv_heads;
  a.dim = p->head_dim;
  return from_hip(da::launch_gqa_append_rope(a, gqa_kernel_dtype(p), static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_gqa_append_rope_fp8(const da_gqa_params_t* p, const da_append_t* ap,
                                   const da_paged_kv_t* pages, const da_kv_scales_t* sc,
                                   const void* q, void* q_out, const void* k_new, const void* v_new,
                                   const int32_t* positions, void* k_cache, void* v_cache,
                                   void* hip_stream) {
  da_status_t st = check_gqa_params(p);
  if (st != DA_OK) return st;
  if (dtype_code(p) != DA_DTYPE_FP8_E4M3) return DA_ERR_INVALID_ARGUMENT;
  st = check_append(ap, p->head_dim, 2);     // new rows are bf16
  if (st != DA_OK) return st;
  if (pages) return DA_ERR_UNSUPPORTED;      // no paged E4M3 caches (decode has none either)
  if (!sc || !sc->k_scale || !sc->v_scale || !aligned4(sc->k_scale) || !aligned4(sc->v_scale) ||
      !stride_in_range(sc->stride_b) || !stride_in_range(sc->stride_t) || !stride_in_range(sc->stride_h))
    return DA_ERR_INVALID_ARGUMENT;
  if (sc->stride_t != 0 && sc->stride_h == 0) return DA_ERR_UNSUPPORTED;
  st = check_ptrs16({q, q_out, k_new, v_new, k_cache, v_cache});
  if (st != DA_OK) return st;
  if (!positions || !aligned4(positions)) return DA_ERR_INVALID_ARGUMENT;
  da::AppendArgs a = append_args(ap, pages, positions, p->batch, p->max_seq_len);
  a.q = q;
  a.q_out = q_out;
  a.q_sb = p->q_stride_b;
  a.q_sh = p->q_stride_h;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.c_sb = p->kv_stride_b;
  a.c_st = p->kv_stride_t;
  a.c_sh = p->kv_stride_h;
  a.q_heads = p->num_q_heads;
  a.kv_heads = p->num_kv_heads;
  a.dim = p->head_dim;
  a.k_scale = const_cast<float*>(sc->k_scale);
  a.v_scale = const_cast<float*>(sc->v_scale);
  a.sc_sb = sc->stride_b;
  a.sc_st = sc->stride_t;
  a.sc_sh = sc->stride_h;
  return from_hip(da::launch_gqa_append_rope_fp8(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_mla_append_rope(const da_mla_params_t* p, const da_append_t* ap,
                               const da_paged_kv_t* pages, const void* q_rope, void* q_rope_out,
                               const void* kv_new, const int32_t* positions, void* kv_cache,
                               void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_append(ap, kMlaRope, 2);
  if (st != DA_OK) return st;
  if (pages && (st = check_paged(pages, p->max_seq_len, 2)) != DA_OK) return st;
  st = check_ptrs16({q_rope, q_rope_out, kv_new, kv_cache});
  if (st != DA_OK) return st;
  if (!positions || !aligned4(positions)) return DA_ERR_INVALID_ARGUMENT;
  da::AppendArgs a = append_args(ap, pages, positions, p->batch, p->max_seq_len);
  a.q = q_rope;
  a.q_out = q_rope_out;
  a.q_sb = (int64_t)p->num_heads * kMlaRope;
  a.q_sh = kMlaRope;
  a.k_new = kv_new;
  a.k_cache = kv_cache;
  a.c_sb = p->cache_stride_b;
  a.c_st = p->cache_stride_t;
  a.q_heads = p->num_heads;
  a.dim = kMlaRope;
  return from_hip(da::launch_mla_append_rope(a, static_cast<hipStream_t>(hip_stream)));
}

size_t da_gqa_decode_workspace_size(const da_gqa_params_t* p) {
  if (check_gqa_params(p) != DA_OK) return 0;
  size_t ws = plan_gqa(p).workspace;
  if (dtype_code(p) == DA_DTYPE_FP8_E4M3) {   // paged fp8 pools plan without 16-wave shapes
    const size_t paged = plan_gqa(p, 32).workspace;
    ws = paged > ws ? paged : ws;
  }
  return ws;
}

int32_t da_gqa_decode_num_splits(const da_gqa_params_t* p) {
  if (check_gqa_params(p) != DA_OK) return 0;
  return plan_gqa(p).splits;
}

da_status_t da_gqa_decode_split_pass(const da_gqa_params_t* p, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* seq_lens, float* part_out, float* part_lse,
                                     void* hip_stream) {
  da_status_t st = check_gqa_params(p);
  if (st != DA_OK) return st;
  if (dtype_code(p) == DA_DTYPE_FP8_E4M3) return DA_ERR_INVALID_ARGUMENT;   // needs scales
  st = check_gqa_buffers(q, k_cache, v_cache, seq_lens, part_out, part_lse);
  if (st != DA_OK) return st;
  if (!part_lse) return DA_ERR_INVALID_ARGUMENT;
  const GqaPlan pl = plan_gqa(p);
  da::GqaArgs a = gqa_args(p, pl, q, k_cache, v_cache, seq_lens);
  if (pl.splits == 1) {
    a.out = part_out;
    a.lse = part_lse;
  } else {
    a.part_out = part_out;
    a.part_lse = part_lse;
  }
  return from_hip(da::launch_gqa_decode(a, gqa_kernel_dtype(p), p->head_dim,
                                        static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_gqa_decode(const da_gqa_params_t* p, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* seq_lens, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (p && dtype_code(p) == DA_DTYPE_FP8_E4M3) return DA_ERR_INVALID_ARGUMENT;   // needs scales
  return gqa_decode_impl(p, nullptr, nullptr, q, k_cache, v_cache, seq_lens, out, lse, workspace,
                         workspace_bytes, hip_stream);
}

da_status_t da_gqa_decode_paged(const da_gqa_params_t* p, const da_paged_kv_t* pages, const void* q,
                                const void* k_pool, const void* v_pool, const int32_t* seq_lens,
                                float* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* hip_stream) {
  if (!pages) return DA_ERR_INVALID_ARGUMENT;
  if (p && dtype_code(p) == DA_DTYPE_FP8_E4M3) return DA_ERR_INVALID_ARGUMENT;
  return gqa_decode_impl(p, pages, nullptr, q, k_pool, v_pool, seq_lens, out, lse, workspace,
                         workspace_bytes, hip_stream);
}

da_status_t da_gqa_decode_fp8(const da_gqa_params_t* p, const da_kv_scales_t* scales, const void* q,
                              const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                              float* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
  if (!p || dtype_code(p) != DA_DTYPE_FP8_E4M3 || !scales) return DA_ERR_INVALID_ARGUMENT;
  return gqa_decode_impl(p, nullptr, scales, q, k_cache, v_cache, seq_lens, out, lse, workspace,
                         workspace_bytes, hip_stream);
}

da_status_t da_gqa_decode_fp8_paged(const da_gqa_params_t* p, const da_paged_kv_t* pages,
                                    const da_kv_scales_t* scales, const void* q, const void* k_pool,
                                    const void* v_pool, const int32_t* seq_lens, float* out,
                                    float* lse, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  if (!p || dtype_code(p) != DA_DTYPE_FP8_E4M3 || !scales || !pages) return DA_ERR_INVALID_ARGUMENT;
  // 32-token steps inside one page; scales that do not vary with the row are
  // per head (a per-page scale has no meaning for the method)
  if (pages->page_size < 32) return DA_ERR_UNSUPPORTED;
  if (scales->stride_t == 0 && scales->stride_b != 0) return DA_ERR_UNSUPPORTED;
  return gqa_decode_impl(p, pages, scales, q, k_pool, v_pool, seq_lens, out, lse, workspace,
                         workspace_bytes, hip_stream);
}

size_t da_mla_decode_workspace_size(const da_mla_params_t* p) {
  if (check_mla_params(p) != DA_OK) return 0;
  return plan_mla(p).workspace;
}

int32_t da_mla_decode_num_splits(const da_mla_params_t* p) {
  if (check_mla_params(p) != DA_OK) return -1;
  return plan_mla(p).splits;
}

da_status_t da_mla_partials_size(const da_mla_params_t* p, size_t* part_out_bytes, size_t* part_lse_bytes) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  if (!part_out_bytes || !part_lse_bytes) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  *part_out_bytes = pl.part_out_bytes;
  *part_lse_bytes = pl.part_lse_bytes;
  return DA_OK;
}

da_status_t da_mla_decode_absorbed(const da_mla_params_t* p, const void* q_nope,
                                   const void* q_rope, const void* kv_cache,
                                   const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                                   float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_nope, q_rope, kv_cache, w_uk, w_uv, out});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens) || !aligned4(lse)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  if (!workspace || workspace_bytes < pl.workspace) return DA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return DA_ERR_INVALID_ARGUMENT;
  char* ws = static_cast<char*>(workspace);
  da::MlaArgs a = mla_args(p, pl);
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.cache = static_cast<const uint16_t*>(kv_cache);
  a.seq_lens = seq_lens;
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.out = out;
  a.lse = lse;
  set_q_hat(a, ws);
  set_partials(a, pl, ws + pl.q_hat_bytes, ws + pl.q_hat_bytes + pl.part_out_bytes);
  return from_hip(da::launch_mla_decode(a, static_cast<hipStream_t>(hip_stream)));
}

size_t da_mla_decode_fp8_workspace_size(const da_mla_params_t* p) {
  if (check_mla_params(p, true) != DA_OK) return 0;
  return plan_mla(p, true).workspace;
}

namespace {

// One E4M3 MLA call: absorb, the E4M3 attention (over paged pools when
// `pages`), merge + project.
da_status_t mla_fp8_impl(const da_mla_params_t* p, const da_paged_kv_t* pages, const da_mla_scales_t* scales,
                         const void* q_nope, const void* q_rope, const void* kv_codes, const int32_t* seq_lens,
                         const void* w_uk, const void* w_uv, float* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  da_status_t st = check_mla_params(p, true);
  if (st != DA_OK) return st;
  if (pages) {
    st = check_paged(pages, p->max_seq_len, 1);
    if (st != DA_OK) return st;
  }
  if (!scales || !scales->nope_scale || !scales->rope_scale || !aligned4(scales->nope_scale) ||
      !aligned4(scales->rope_scale) || !stride_in_range(scales->stride_b) ||
      !scale_stride_t_ok(scales->stride_t))
    return DA_ERR_INVALID_ARGUMENT;
  st = check_ptrs16({q_nope, q_rope, kv_codes, w_uk, w_uv, out});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens) || !aligned4(lse)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p, true);
  if (!workspace || workspace_bytes < pl.workspace) return DA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return DA_ERR_INVALID_ARGUMENT;
  char* ws = static_cast<char*>(workspace);
  da::MlaArgs a = mla_args(p, pl);
  if (pages) set_paged(a, pages);
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.cache8 = static_cast<const uint8_t*>(kv_codes);
  a.sc_nope = scales->nope_scale;
  a.sc_rope = scales->rope_scale;
  a.sc_sb = scales->stride_b;
  a.sc_st = scales->stride_t;
  a.seq_lens = seq_lens;
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.out = out;
  a.lse = lse;
  set_q_hat(a, ws);
  set_partials(a, pl, ws + pl.q_hat_bytes, ws + pl.q_hat_bytes + pl.part_out_bytes);
  return from_hip(da::launch_mla_decode_fp8(a, static_cast<hipStream_t>(hip_stream)));
}

}  // namespace

da_status_t da_mla_decode_absorbed_fp8(const da_mla_params_t* p, const da_mla_scales_t* scales,
                                       const void* q_nope, const void* q_rope, const void* kv_codes,
                                       const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                                       float* out, float* lse, void* workspace, size_t workspace_bytes,
                                       void* hip_stream) {
  return mla_fp8_impl(p, nullptr, scales, q_nope, q_rope, kv_codes, seq_lens, w_uk, w_uv, out, lse, workspace,
                      workspace_bytes, hip_stream);
}

da_status_t da_mla_decode_absorbed_fp8_paged(const da_mla_params_t* p, const da_paged_kv_t* pages,
                                             const da_mla_scales_t* scales, const void* q_nope,
                                             const void* q_rope, const void* code_pool, const int32_t* seq_lens,
                                             const void* w_uk, const void* w_uv, float* out, float* lse,
                                             void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!pages) return DA_ERR_INVALID_ARGUMENT;
  return mla_fp8_impl(p, pages, scales, q_nope, q_rope, code_pool, seq_lens, w_uk, w_uv, out, lse, workspace,
                      workspace_bytes, hip_stream);
}

size_t da_noalloc_scratch_bytes(void) { return kScratchBytes; }

da_status_t da_mla_decode_absorbed_noalloc(const da_mla_params_t* p, const void* q_nope,
                                           const void* q_rope, const void* kv_cache,
                                           const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                                           float* out, float* lse, void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  const size_t need = plan_mla(p).workspace;
  if (need > kScratchBytes) return DA_ERR_WORKSPACE_TOO_SMALL;
  st = check_ptrs16({q_nope, q_rope, kv_cache, w_uk, w_uv, out});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens) || !aligned4(lse)) return DA_ERR_INVALID_ARGUMENT;
  void* ws = current_device_scratch();
  if (!ws) return DA_ERR_HIP;
  // the scratch needs no clearing: every call writes each byte it reads first
  return da_mla_decode_absorbed(p, q_nope, q_rope, kv_cache, seq_lens, w_uk, w_uv, out, lse, ws,
                                kScratchBytes, hip_stream);
}

da_status_t da_mla_absorb_query(const da_mla_params_t* p, const void* q_nope, const void* q_rope,
                                const void* w_uk, void* q_hat, void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_nope, q_rope, w_uk, q_hat});
  if (st != DA_OK) return st;
  da::MlaArgs a = mla_args(p, plan_mla(p));
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  set_q_hat(a, q_hat);
  return from_hip(da::launch_mla_absorb(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_mla_attend_split_pass(const da_mla_params_t* p, const void* q_hat,
                                     const void* kv_cache, const int32_t* seq_lens,
                                     void* part_out, float* part_lse, void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_hat, kv_cache, part_out, part_lse});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  da::MlaArgs a = mla_args(p, pl);
  set_q_hat(a, q_hat);
  a.cache = static_cast<const uint16_t*>(kv_cache);
  a.seq_lens = seq_lens;
  set_partials(a, pl, part_out, part_lse);
  return from_hip(da::launch_mla_attend(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_mla_decode_absorbed_paged(const da_mla_params_t* p, const da_paged_kv_t* pages,
                                         const void* q_nope, const void* q_rope, const void* cache_pool,
                                         const int32_t* seq_lens, const void* w_uk, const void* w_uv,
                                         float* out, float* lse, void* workspace, size_t workspace_bytes,
                                         void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_paged(pages, p->max_seq_len, 2);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_nope, q_rope, cache_pool, w_uk, w_uv, out});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens) || !aligned4(lse)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  if (!workspace || workspace_bytes < pl.workspace) return DA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return DA_ERR_INVALID_ARGUMENT;
  char* ws = static_cast<char*>(workspace);
  da::MlaArgs a = mla_args(p, pl);
  set_paged(a, pages);
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_rope = static_cast<const uint16_t*>(q_rope);
  a.cache = static_cast<const uint16_t*>(cache_pool);
  a.seq_lens = seq_lens;
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.out = out;
  a.lse = lse;
  set_q_hat(a, ws);
  set_partials(a, pl, ws + pl.q_hat_bytes, ws + pl.q_hat_bytes + pl.part_out_bytes);
  return from_hip(da::launch_mla_decode(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_mla_attend_split_pass_paged(const da_mla_params_t* p, const da_paged_kv_t* pages,
                                           const void* q_hat, const void* cache_pool,
                                           const int32_t* seq_lens, void* part_out, float* part_lse,
                                           void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_paged(pages, p->max_seq_len, 2);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_hat, cache_pool, part_out, part_lse});
  if (st != DA_OK) return st;
  if (!aligned4(seq_lens)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  da::MlaArgs a = mla_args(p, pl);
  set_paged(a, pages);
  set_q_hat(a, q_hat);
  a.cache = static_cast<const uint16_t*>(cache_pool);
  a.seq_lens = seq_lens;
  set_partials(a, pl, part_out, part_lse);
  return from_hip(da::launch_mla_attend(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_mla_merge_project(const da_mla_params_t* p, const void* q_hat, const void* part_out,
                                 const float* part_lse, const void* w_uv, float* out, float* lse,
                                 void* hip_stream) {
  da_status_t st = check_mla_params(p);
  if (st != DA_OK) return st;
  st = check_ptrs16({q_hat, part_out, w_uv, out});
  if (st != DA_OK) return st;
  if (!part_lse || !aligned4(part_lse) || !aligned4(lse)) return DA_ERR_INVALID_ARGUMENT;
  const MlaPlan pl = plan_mla(p);
  da::MlaArgs a = mla_args(p, pl);
  set_partials(a, pl, const_cast<void*>(part_out), const_cast<float*>(part_lse));
  set_q_hat(a, q_hat);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.out = out;
  a.lse = lse;
  return from_hip(da::launch_mla_merge_project(a, static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_splitkv_combine(int32_t num_splits, int32_t batch, int32_t num_heads,
                               int32_t head_dim, const float* partial_out,
                               const float* partial_lse, float* out, float* lse,
                               void* hip_stream) {
  if (num_splits < 1 || batch < 1 || num_heads < 1 || head_dim < 4 || head_dim % 4 != 0 ||
      head_dim > 1024)
    return DA_ERR_INVALID_ARGUMENT;
  if ((int64_t)batch * num_heads > INT32_MAX) return DA_ERR_INVALID_ARGUMENT;
  if (!partial_out || !partial_lse || !out) return DA_ERR_INVALID_ARGUMENT;
  if (!aligned16(partial_out) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(partial_lse) & 3u) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return DA_ERR_INVALID_ARGUMENT;
  return from_hip(da::launch_splitkv_combine(num_splits, batch * num_heads, head_dim, partial_out,
                                             partial_lse, out, lse,
                                             static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_probe_stream_read(const void* src, int64_t bytes, int32_t blocks, int32_t depth,
                                 uint32_t* sink, void* hip_stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || !probe_shape_ok(blocks, depth))
    return DA_ERR_INVALID_ARGUMENT;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return DA_ERR_INVALID_ARGUMENT;
  return from_hip(da::launch_stream_read(src, bytes, probe_blocks(blocks), depth, sink,
                                         static_cast<hipStream_t>(hip_stream)));
}

da_status_t da_probe_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks,
                                 int32_t depth, void* hip_stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || !probe_shape_ok(blocks, depth))
    return DA_ERR_INVALID_ARGUMENT;
  if (!aligned16(src) || !aligned16(dst)) return DA_ERR_INVALID_ARGUMENT;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return DA_ERR_INVALID_ARGUMENT;
  return from_hip(da::launch_stream_copy(src, dst, bytes, probe_blocks(blocks), depth,
                                         static_cast<hipStream_t>(hip_stream)));
}

const char* da_status_string(da_status_t status) {
  int32_t s;   // the caller's value, which may lie outside the enumerators
  static_assert(sizeof(status) == sizeof(s), "enum is 32 bits");
  memcpy(&s, &status, sizeof(s));
  switch (s) {
    case DA_OK: return "ok";
    case DA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t da_version(void) { return 100; }

size_t da_gqa_params_size(void) { return sizeof(da_gqa_params_t); }
size_t da_mla_params_size(void) { return sizeof(da_mla_params_t); }
size_t da_mla_scales_size(void) { return sizeof(da_mla_scales_t); }
size_t da_paged_kv_size(void) { return sizeof(da_paged_kv_t); }
size_t da_kv_scales_size(void) { return sizeof(da_kv_scales_t); }
size_t da_append_size(void) { return sizeof(da_append_t); }

}  // extern "C"
