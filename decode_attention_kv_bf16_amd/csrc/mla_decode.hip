// DeepSeek-style absorbed-MLA decode for gfx950 (CDNA4): three launches.
//
// The method ("Attention variants and KV cache", arganzheng.life, sections
// 4.5-4.6; jianzhnie.github.io "Multi-head Latent Attention", section 4):
//   q~_h = q_nope_h W_UK,h^T (512), q^_h = [q~_h ; q_rope_h] (576),
//   s_j  = q^_h . row_j / sqrt(192) with row_j = [c_kv_j ; k_rope_j] shared by all heads,
//   o~_h = sum_j softmax(s)_j c_kv_j (the value is the first 512 columns of the same row),
//   o_h  = o~_h W_UV,h.
// After absorption every head attends the same 576-wide row, so decode is one
// dense contraction per sequence: S^T = C Q^^T ([T x 576] x [576 x H]) and
// O^T += C[:, :512]^T P^T, which runs on the matrix cores.
//
// Kernels
//  1. mla_absorb_kernel   q^ = [q_nope W_UK^T | q_rope] (bf16) for all (b, h).
//  2. mla_attend_kernel   one workgroup per (split, sequence); for 128 heads,
//     4 waves of 32 heads each (one wave per SIMD, accumulators in AGPRs).
//     32-row latent tiles are copied HBM -> LDS by the load-to-LDS path
//     (global_load_lds_dwordx4, no register staging), double-buffered; each
//     tile is read from LDS as the A operand of S^T (row-major 16-byte reads)
//     and, transposed by ds_read_b64_tr_b16, as the A operand of O^T. Each
//     head's softmax reference max is fixed by its first tile, so the
//     accumulators are never rescaled in the loop (see kRefHeadroom). Each
//     split writes its normalised o~_s (bf16) and lse_s.
//  3. mla_merge_project_kernel  merges the splits by log-sum-exp and multiplies
//     by W_UV,h on the matrix cores (W_UV,h staged in LDS, read transposed).
#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

constexpr int kDc = 512;            // latent (value) width
constexpr int kRowE = 576;          // cached row: c_kv (512) | k_rope (64)
constexpr int kRowB = kRowE * 2;    // 1152 bytes
constexpr int kChunks = kRowB / 16; // 72 16-byte chunks per row
constexpr int kTok = 32;            // rows per tile
constexpr int kTileB = kTok * kRowB;          // 36864 bytes, a multiple of 1 KiB
constexpr int kTileDma = kTileB / 1024;       // wave-wide 1 KiB copies per tile (36)
// A head's reference max is fixed by its first tile; later scores may exceed
// it by up to 2^64 (fp32 and bf16 share an exponent range up to 2^127, so the
// weights and sums stay finite). A tile that exceeds it by more restarts the
// split with a raised reference instead of rescaling the accumulators, which
// live in AGPRs where arithmetic cannot touch them.
constexpr float kRefHeadroom = 64.0f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane j names an 8-byte
// piece (row j/4, piece j%4) of a 4x16 bf16 block; lane i gets column i.
__device__ __forceinline__ i16x4_t lds_read_tr(const LDS uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4_t*)p);
}

__device__ __forceinline__ bf16x8_t join_tr(i16x4_t lo, i16x4_t hi) {
  i16x4_t v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ void load_to_lds16(const void* src, LDS uint8_t* dst_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (LDS void*)dst_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without the release fence of __syncthreads(): that fence
// makes the compiler wait for every outstanding load-to-LDS copy (vmcnt(0)),
// including the tiles meant to stay in flight, which empties the copy ring on
// every tile. Ordering here is explicit instead: each wave waits for its own
// copies of the tile with wait_vm<N>() before the barrier, and every LDS read
// of the buffer being refilled has returned (its value was consumed) before
// the wave reaches the barrier. The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }


__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  return pack_bf16x2(lo, hi);
}

// XOR swizzle of the 16-byte chunk index inside a tile row (rows are 1152
// bytes = 72 chunks; only the low 3 bits of a chunk index change, so a chunk
// stays inside its aligned group of 8 and inside its row): f(r) = r mod 8.
// Both read patterns of the tile are free of LDS bank conflicts with it, as
// measured with the SQ_LDS_BANK_CONFLICT counter: (a) 16-byte reads of 16
// consecutive rows at one logical chunk (the S^T operand) and (b) the
// transposing 8-byte reads of 4 consecutive rows x 32 bytes (the O^T operand).
// Rows r and r + 16 share f, so one lane offset serves both halves of a tile.
__device__ __forceinline__ int row_swizzle(int row) { return row & 7; }

// Two block-table entries of a paged pool, read with scalar loads that are
// issued together and waited for once, inside this block (so no load is left
// in flight when it ends). Written by hand because the compiler, short of
// scalar registers here, uses the first entry before issuing the second
// load, and so waits twice.
__device__ __forceinline__ void load_two_entries(const int32_t* p0, const int32_t* p1, int32_t& e0,
                                                 int32_t& e1) {
  asm volatile(
      "s_load_dword %0, %2, 0x0\n\t"
      "s_load_dword %1, %3, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(e0), "=&s"(e1)
      : "s"(p0), "s"(p1)
      : "memory");
}

// Where the rows of one tile come from in a paged pool: a 32-row tile that
// starts on a multiple of 32 is two halves of 16 rows, each inside one page
// of >= 16 rows, and 16 rows (18 KiB) are exactly 18 of the tile's 1 KiB
// copies, so each copy reads from one half, through that half's buffer
// resource (its page, sized to its valid rows).
struct PagedTile {
  __amdgpu_buffer_rsrc_t half[2];
};

// ---------------------------------------------------------------------------
// 1. query absorption
// ---------------------------------------------------------------------------
// 8 slices of 64 latent columns per head; one wave each. Computes the transpose
// q~^T[c, b] = sum_e W_UK[h, c, e] q_nope[b, h, e] so that each lane ends up
// with 4 consecutive latent columns of one batch row (one 8-byte store).
// Both operands are read in their stored layout (e contiguous).
constexpr int kAbsorbBatch = 64;   // batch rows per pass (4 blocks of 16)

__global__ __launch_bounds__(64) void mla_absorb_kernel(MlaArgs a) {
  // Workgroups are dealt to the 8 XCDs round-robin by linear id; this mapping
  // puts the 8 slices of a head on one XCD, so its q_nope column is fetched
  // from HBM once and then served by that XCD's L2.
  const int id = blockIdx.x;
  const int slice = (id >> 3) & 7;
  const int h = (id & 7) + 8 * (id >> 6);
  const int H = a.num_heads;
  const int B = a.batch;
  const int lane = threadIdx.x;
  const int q4 = lane >> 4, l16 = lane & 15;
  const int c0 = 64 * slice;

  bf16x8_t wa[4][4];   // A: W_UK[h, c0 + 16cb + l16, 32ks + 8q4 .. +8]
  const uint16_t* wp = a.w_uk + ((int64_t)h * kDc + c0 + l16) * 128 + 8 * q4;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      wa[cb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(wp + cb * 16 * 128 + 32 * ks));

  for (int b0 = 0; b0 < B; b0 += kAbsorbBatch) {
    bf16x8_t qb[4][4];  // B: q_nope[b0 + 16bb + l16, h, 32ks + 8q4 .. +8]
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int b = b0 + 16 * bb + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (b < B) v = *reinterpret_cast<const uint4*>(a.q_nope + ((int64_t)b * H + h) * 128 + 32 * ks + 8 * q4);
        qb[bb][ks] = as_bf16x8(v);
      }
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int b = b0 + 16 * bb + l16;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(wa[cb][ks], qb[bb][ks], acc);
        // lane holds q~[b][c0 + 16cb + 4q4 + i], i = 0..3
        if (b < B) {
          uint2 v;
          v.x = cvt_bf16x2(acc[0], acc[1]);
          v.y = cvt_bf16x2(acc[2], acc[3]);
          *reinterpret_cast<uint2*>(a.q_hat + ((int64_t)b * H + h) * kRowE + c0 + 16 * cb + 4 * q4) = v;
        }
      }
    }
  }
  // append q_rope (already rotated) unchanged: B x 8 16-byte chunks per head,
  // spread over the 8 slice workgroups (one chunk per lane up to B = 64)
  for (int i = slice * 64 + lane; i < B * 8; i += 8 * 64) {
    const int b = i >> 3, ch = i & 7;
    *reinterpret_cast<uint4*>(a.q_hat + ((int64_t)b * H + h) * kRowE + kDc + 8 * ch) =
        *reinterpret_cast<const uint4*>(a.q_rope + ((int64_t)b * H + h) * 64 + 8 * ch);
  }
}

// ---------------------------------------------------------------------------
// split assignment
// ---------------------------------------------------------------------------
struct SplitWork {
  int b, slot, t_begin, t_end;  // wave-uniform
  bool valid;
};

// Inclusive prefix sum over the 64 lanes of a wave by DPP (no LDS round
// trips): shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes with no
// source add 0), then the last lane of row 0 is added to row 1 and of row 2
// to row 3 (row_bcast:15), then the last lane of row 1 to rows 2 and 3
// (row_bcast:31). Lanes that a step leaves out add 0.
__device__ __forceinline__ int wave_inclusive_scan_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); // row_bcast:31, rows 2, 3
  return x;
}

// The work of a workgroup. Fixed splits: grid (S, B), chunk rows per split.
// Balanced splits: every sequence b gets S_b = ceil(tiles_b / q) splits of q
// tiles (32 rows) with q = ceil(total tiles / wg_budget), so that all splits
// carry about the same work whatever the lengths; the splits of b take the
// slots P_b .. P_b + S_b - 1 (P = exclusive prefix sum of S) and work item wg
// (a permutation of the workgroup id) serves slot wg. Every wave computes this from seq_lens on its own (its
// results are wave-uniform); wave 0 of workgroup 0 publishes P and S for the
// merge. A split is never empty; workgroups past the last slot get none.
__device__ SplitWork assign_split(const MlaArgs& a, int lane, bool publish) {
  SplitWork r{0, 0, 0, 0, false};
  if (a.num_splits > 0) {
    r.b = blockIdx.y;
    r.slot = blockIdx.x * a.batch + blockIdx.y;
    // clamped to [0, max_seq_len]: no read past the cache or the block table
    const int L = a.seq_lens ? min(max(a.seq_lens[r.b], 0), a.max_seq_len) : a.max_seq_len;
    r.t_begin = blockIdx.x * a.chunk;
    r.t_end = min(L, r.t_begin + a.chunk);
    r.valid = true;
    return r;
  }
  const int B = a.batch;
  // Work item of this workgroup. The first wg_budget items (the ones that run
  // in the first round) go in consecutive runs of wg_budget / 8 to the XCDs,
  // which take workgroups id = x (mod 8): the splits of one sequence, which
  // share its absorbed queries, then mostly share an XCD and its L2. Items
  // past wg_budget keep their id.
  const int wg = (blockIdx.x < a.wg_budget && (a.wg_budget & 7) == 0)
                     ? (blockIdx.x & 7) * (a.wg_budget >> 3) + (blockIdx.x >> 3)
                     : blockIdx.x;
  constexpr int kMaxChunks = 8;  // balanced splits are planned for B <= 512
  const int n_chunks = (B + 63) >> 6;
  // lengths of sequences c * 64 + lane, clamped to [0, max_seq_len] (rows past
  // max_seq_len are never read, as with fixed splits); all loads are issued
  // before the first use (clamped indexes, so no branch separates them)
  int len[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int b = min(c * 64 + lane, B - 1);
    len[c] = a.seq_lens ? a.seq_lens[b] : a.max_seq_len;
  }
  int tiles_lane = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    len[c] = c * 64 + lane < B ? min(max(len[c], 0), a.max_seq_len) : 0;
    tiles_lane += (len[c] + kTok - 1) / kTok;
  }
  const int total = __builtin_amdgcn_readlane(wave_inclusive_scan_i(tiles_lane), 63);
  const int q = max(1, (total + a.wg_budget - 1) / a.wg_budget);
  int carry = 0;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c >= n_chunks) break;
    const int b = c * 64 + lane;
    const int S = ((len[c] + kTok - 1) / kTok + q - 1) / q;
    const int incl = wave_inclusive_scan_i(S);
    const int P = carry + incl - S;
    if (publish && b < B) {
      a.split_table[2 * b] = P;
      a.split_table[2 * b + 1] = S;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(b < B && wg >= P && wg < P + S);
    if (hit != 0) {
      const int src = __builtin_ctzll(hit);
      r.b = __builtin_amdgcn_readlane(b, src);
      const int s = wg - __builtin_amdgcn_readlane(P, src);
      const int L = __builtin_amdgcn_readlane(len[c], src);
      r.slot = wg;
      r.t_begin = s * q * kTok;
      r.t_end = min(L, r.t_begin + q * kTok);
      r.valid = true;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  // the values are wave-uniform; say so, so that they stay in scalar registers
  r.b = __builtin_amdgcn_readfirstlane(r.b);
  r.slot = __builtin_amdgcn_readfirstlane(r.slot);
  r.t_begin = __builtin_amdgcn_readfirstlane(r.t_begin);
  r.t_end = __builtin_amdgcn_readfirstlane(r.t_end);
  return r;
}

// ---------------------------------------------------------------------------
// 2. split-KV latent attention
// ---------------------------------------------------------------------------
// grid (split, sequence); NW waves, each owning HB blocks of 16 heads
// (H = 16 * NW * HB; 128 heads: 4 waves x 32 heads, one wave per SIMD, so a
// wave may hold its 256 accumulator registers plus the 144 registers of its
// absorbed queries). Every wave reads each 32-row tile from LDS once and
// feeds both of its head blocks from that read.
template <int NW, int HB, bool kPaged>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attend_kernel(MlaArgs a) {
  // LDS ring of kDepth tiles: up to kDepth - 1 tiles in flight from HBM while
  // one is consumed. Each wave issues kCopies 1 KiB copies per tile, and a
  // wave may have at most 63 vector-memory operations outstanding.
  constexpr int kCopies = kTileDma / NW;
  static_assert(kTileDma % NW == 0, "copies split evenly over the waves");
  constexpr int kDepth = (3 * kCopies <= 63) ? 4 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDepth * kTileB];
  LDS uint8_t* lds = (LDS uint8_t*)smem;

  constexpr int H = NW * 16 * HB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  const SplitWork work = assign_split(a, lane, blockIdx.x == 0 && w == 0);
  if (!work.valid) return;
  const int b = work.b;
  const int64_t slot = work.slot;
  const int t_begin = work.t_begin;
  const int t_end = work.t_end;

  if (t_begin >= t_end) {  // fixed splits only: a split past the sequence's end
    for (int i = tid; i < H; i += NW * 64) a.part_lse[slot * H + i] = kNegInf;
    return;
  }

  const uint16_t* cache_b = a.cache + (int64_t)b * a.cache_sb;
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;

  // HBM -> LDS copy of one tile: wave w issues 1 KiB copies k = w, w+NW, ...
  // Lane l of copy k fills tile chunk p = 64k + l with the logical chunk that
  // the swizzle stores there; its byte offset inside a tile is fixed, so it is
  // computed once. Each tile gets a buffer resource that ends at the split's
  // last row, so rows past it read as zeros (their weights are zero anyway).
  const uint32_t row_bytes = (uint32_t)a.cache_st * 2u;
  // byte offset of the lane's chunk in the tile (paged: in its half-tile)
  uint32_t voff[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int p = (w + NW * i) * 64 + lane;
    const int row = p / kChunks;
    const int c = (p - row * kChunks) ^ row_swizzle(row);
    voff[i] = (uint32_t)(kPaged ? row & 15 : row) * row_bytes + 16u * (uint32_t)c;
  }
  // LDS destinations are computed in scalar registers: this wave's first copy
  // slot of ring buffer 0, as a byte address
  const uint32_t lds_w0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds + (uint32_t)w * 1024u);
  // Tiles past the split's end get an empty range: their copies read nothing
  // and fill the (unused) ring buffer with zeros, which keeps the number of
  // copies in flight, and so every wait below, the same on every tile.
  //
  // Paged pools (arganzheng.life section 6.1): each half-tile's page is
  // looked up in the block table with a scalar load. Both lookups are
  // unconditional, at rows clamped to the split's last row (t_end > t_begin
  // here, so the entry is always one of the sequence's), so they are issued
  // together and waited for once; a half with no valid rows gets an empty
  // resource.
  const int64_t tab0 = (int64_t)b * a.max_blocks;
  auto tile_src = [&](int it) {
    const int t0 = t_begin + it * kTok;
    if constexpr (kPaged) {
      int32_t page[2];
      load_two_entries(a.block_table + tab0 + (min(t0, t_end - 1) >> a.page_shift),
                       a.block_table + tab0 + (min(t0 + 16, t_end - 1) >> a.page_shift), page[0], page[1]);
      PagedTile pt;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int th = t0 + 16 * hf;
        // (the clamp is a vector instruction: made scalar again for the resource)
        const int rows = __builtin_amdgcn_readfirstlane(min(max(t_end - th, 0), 16));
        const uint16_t* base = a.cache + (int64_t)page[hf] * a.page_stride +
                               (int64_t)(th & ((1 << a.page_shift) - 1)) * a.cache_st;
        pt.half[hf] = make_raw_rsrc(base, (uint32_t)rows * row_bytes);
      }
      return pt;
    } else {
      return make_raw_rsrc(cache_b + (int64_t)t0 * a.cache_st, (uint32_t)max(t_end - t0, 0) * row_bytes);
    }
  };
  using TileSrc = decltype(tile_src(0));
  // the compiler waits for a tile's table lookups where this is called, when
  // no LDS read is in flight (LDS reads and scalar loads share one counter)
  auto settle = [&](const TileSrc& src) {
    if constexpr (kPaged) asm volatile("" ::"s"(src.half[0]), "s"(src.half[1]));
  };
  auto issue_copy = [&](const TileSrc& src, int i, int buf) {
    const uint32_t dst = lds_w0 + (uint32_t)(buf * kTileB + NW * i * 1024);
    if constexpr (kPaged) {
      // copy w + NW i reads the second half-tile iff it is >= kTileDma / 2;
      // known at compile time (for an unrolled i) unless the copies of step i
      // straddle it; wave-uniform in any case
      constexpr int kHalf = kTileDma / 2;
      const int second = NW * i >= kHalf ? 1 : NW * i + NW <= kHalf ? 0 : (w + NW * i >= kHalf);
      buffer_load_to_lds16(__builtin_amdgcn_readfirstlane(second) ? src.half[1] : src.half[0], voff[i], dst);
    } else {
      buffer_load_to_lds16(src, voff[i], dst);
    }
  };
  auto issue_tile = [&](int it, int buf) {
    const TileSrc src = tile_src(it);
    settle(src);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) issue_copy(src, i, buf);
  };

  // absorbed queries of this lane's heads, as B operands: q^[h][32ks + 8q4 .. +8]
  bf16x8_t qb[HB][18];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = (w * HB + hb) * 16 + l16;
    const uint16_t* qp = a.q_hat + ((int64_t)b * H + h) * kRowE + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qb[hb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 32 * ks));
  }
  // The compiler does not see the tile copies, so its wait for these loads
  // would be a vmcnt(0) at their first use, after the copies are in flight:
  // take the wait here, before any copy is issued.
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) asm volatile("" ::"v"(qb[hb][ks]));

  float m_ref[HB];  // reference max (log2 units) of this lane's heads; fixed by the first tile
  float thr[HB];    // raw score above which a head's reference must be raised
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) m_ref[hb] = thr[hb] = kNegInf;
  // lane-constant pieces of the LDS addresses
  const int f_s = row_swizzle(l16);                         // rows l16 and l16 + 16
  const int s_off0 = l16 * kRowB + 16 * ((0 + q4) ^ f_s);   // logical chunk 4ks + q4, ks even
  const int s_off1 = l16 * kRowB + 16 * ((4 + q4) ^ f_s);   // ks odd
  const int r1 = 4 * q4 + (l16 >> 2);                       // transposed reads: rows r1, r1 + 16
  const int f_t = row_swizzle(r1);
  const int hbit = (l16 & 3) >> 1;
  int t_off[4];
#pragma unroll
  for (int cbl = 0; cbl < 4; ++cbl) t_off[cbl] = r1 * kRowB + 16 * ((2 * cbl + hbit) ^ f_t) + 8 * (l16 & 1);

  __shared__ int restart_flag;
  if (tid == 0) restart_flag = 0;

  f32x4_t o[HB][32];
  float l_part[HB];  // this lane's share of sum_j 2^(s_j - m_ref)
  // --- the phases of one tile --------------------------------------------
  // S^T = C Q^^T of tile `it` (ring buffer it % kDepth) for tokens 0-15
  // (s[.][0]) and 16-31 (s[.][1]); the copies of tile `refill_it` go out
  // spread over the k-steps, so that their issue overlaps the matrix ops. The
  // tile operands go through a ring of kSRing register slots: the read for
  // k-step ks + kSRing - 1 is issued before the matrix ops of k-step ks, and
  // the scheduling fences keep the compiler from hoisting every read (which
  // would need more registers than a wave has).
  constexpr int kSRing = 3;
  auto score_tile = [&](int it, int refill_it, const TileSrc& refill_src, f32x4_t (&s)[HB][2]) {
    const int refill_buf = refill_it % kDepth;
    const LDS uint8_t* tile = lds + (it % kDepth) * kTileB;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) s[hb][0] = s[hb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t ra0[kSRing], ra1[kSRing];
    auto read_s = [&](int ks) {
      const int off = ((ks & 1) ? s_off1 : s_off0) + 128 * (ks >> 1);
      ra0[ks % kSRing] = *reinterpret_cast<const LDS u32x4_t*>(tile + off);
      ra1[ks % kSRing] = *reinterpret_cast<const LDS u32x4_t*>(tile + off + 16 * kRowB);
    };
#pragma unroll
    for (int ks = 0; ks < kSRing - 1; ++ks) read_s(ks);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int i = ks * kCopies / 18; i < (ks + 1) * kCopies / 18; ++i) issue_copy(refill_src, i, refill_buf);
      if (ks + kSRing - 1 < 18) read_s(ks + kSRing - 1);
      const bf16x8_t a0 = as_bf16x8(ra0[ks % kSRing]);
      const bf16x8_t a1 = as_bf16x8(ra1[ks % kSRing]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        s[hb][0] = mfma16x16x32(a0, qb[hb][ks], s[hb][0]);
        s[hb][1] = mfma16x16x32(a1, qb[hb][ks], s[hb][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax reference of tile `it`: the lane holds tokens 4q4+i and 16+4q4+i
  // of head (hb, l16); rows past the split end (last tile only) get score
  // -inf, weight 0. Only the first tile of a split (thr = -inf) and a score
  // beyond the headroom need the head-wide max: the four lanes of a head
  // combine theirs, so they agree on the reference.
  auto softmax_ref = [&](int it, f32x4_t (&s)[HB][2]) {
    const int nv = t_end - (t_begin + it * kTok);  // valid rows in the tile (may exceed 32)
    const bool full_tile = nv >= kTok;
    float smax[HB];
    bool over = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      if (!full_tile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (4 * q4 + i >= nv) s[hb][0][i] = kNegInf;
          if (16 + 4 * q4 + i >= nv) s[hb][1][i] = kNegInf;
        }
      }
      float mx = fmaxf(s[hb][0][0], s[hb][1][0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) mx = fmaxf(mx, fmaxf(s[hb][0][i], s[hb][1][i]));
      smax[hb] = mx;
      over |= mx > thr[hb];
    }
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float mx = smax[hb] * a.scale_log2;
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (m_ref[hb] == kNegInf) {
          m_ref[hb] = mx;                            // first tile of the split
        } else if (mx > m_ref[hb] + kRefHeadroom) {  // rare: restart with a raised reference
          m_ref[hb] = mx;
          restart_flag = 1;
        }
        thr[hb] = (m_ref[hb] + kRefHeadroom) / a.scale_log2;
      }
    }
  };
  // weight k of the lane (k = 8 hb + i; i < 4: token 4q4+i, else 16+4q4+i-4)
  auto weight = [&](const f32x4_t (&s)[HB][2], int k) {
    const int hb = k >> 3, i = k & 7;
    const float v = i < 4 ? s[hb][0][i] : s[hb][1][i - 4];
    return exp2_hw(fmaf(v, a.scale_log2, -m_ref[hb]));
  };
  // the weights as PV B operands (token order matching the transposed reads)
  auto pack = [&](const float (&p)[8 * HB], bf16x8_t (&pb)[HB]) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float* q = p + 8 * hb;
      l_part[hb] += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
      uint4 pw;
      pw.x = cvt_bf16x2(q[0], q[1]);
      pw.y = cvt_bf16x2(q[2], q[3]);
      pw.z = cvt_bf16x2(q[4], q[5]);
      pw.w = cvt_bf16x2(q[6], q[7]);
      pb[hb] = as_bf16x8(pw);
    }
  };
  // O^T[c, h] += sum_t C[t, c] P[h, t] for the tile in ring buffer `buf`;
  // B-operand element e is token 4q4+e (e < 4) or 16+4q4+(e-4), matching the
  // two transposed reads. pv_start issues the first transposed reads (they do
  // not depend on P); pv_run runs `extra(cb)` in the shadow of column block
  // cb's matrix ops.
  constexpr int kTRing = 4;
  i16x4_t tlo[kTRing], thi[kTRing];
  auto read_t = [&](const LDS uint8_t* tile, int cb) {
    const int off = t_off[cb & 3] + 128 * (cb >> 2);
    tlo[cb % kTRing] = lds_read_tr(tile + off);
    thi[cb % kTRing] = lds_read_tr(tile + off + 16 * kRowB);
  };
  auto pv_start = [&](int buf) {
    const LDS uint8_t* tile = lds + buf * kTileB;
#pragma unroll
    for (int cb = 0; cb < kTRing - 1; ++cb) read_t(tile, cb);
  };
  auto pv_run = [&](int buf, const bf16x8_t (&pb)[HB], auto&& extra) {
    const LDS uint8_t* tile = lds + buf * kTileB;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      if (cb + kTRing - 1 < 32) read_t(tile, cb + kTRing - 1);
      const bf16x8_t at = join_tr(tlo[cb % kTRing], thi[cb % kTRing]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) o[hb][cb] = mfma16x16x32(at, pb[hb], o[hb][cb]);
      extra(cb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One attempt normally; a further attempt only if some tile's max exceeded
  // its head's reference by more than kRefHeadroom (the reference is raised to
  // that tile max, a strictly larger observed value, so attempts are finite).
  // A flagged attempt still runs to the end of the split (its accumulators
  // are discarded); testing the flag only after the tile loop keeps the loop
  // free of extra exits, which the register allocator needs to keep the
  // accumulators resident in AGPRs.
  for (;;) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) o[hb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      l_part[hb] = 0.f;
    }
    f32x4_t s[HB][2];
    if constexpr (kDepth == 4) {
      // Software pipeline: while the matrix cores run the PV of tile it - 1,
      // the VALU computes the weights of tile it (a wave overlaps only a few
      // VALU ops with each of its own matrix ops, so the 8 HB weights are
      // spread over the 32 column blocks). Tile it - 1 stays in its ring
      // buffer, so 2 tiles are in flight: tile it + 2 is refilled into the
      // buffer of tile it - 2.
#pragma unroll
      for (int j = 0; j < 2; ++j) issue_tile(j, j);
      bf16x8_t pb[HB];
      {
        const TileSrc refill = tile_src(2);
        wait_vm<kCopies>();  // tile 0 has landed, tile 1 may be pending
        tile_barrier();
        settle(refill);
        score_tile(0, 2, refill, s);
        softmax_ref(0, s);
        float p[8 * HB];
#pragma unroll
        for (int k = 0; k < 8 * HB; ++k) p[k] = weight(s, k);
        pack(p, pb);
      }
      for (int it = 1; it < ntiles; ++it) {
        // tile `it` has landed once only the copies of tile it + 1 are pending;
        // after the barrier every wave is also done with tile it - 2's buffer
        const TileSrc refill = tile_src(it + 2);
        wait_vm<kCopies>();
        tile_barrier();
        settle(refill);
        score_tile(it, it + 2, refill, s);
        pv_start((it - 1) % kDepth);
        softmax_ref(it, s);
        float p[8 * HB];
        constexpr int kStep = 32 / (8 * HB);  // column blocks per weight
        pv_run((it - 1) % kDepth, pb, [&](int cb) {
          if (cb % kStep == 0) p[cb / kStep] = weight(s, cb / kStep);
        });
        pack(p, pb);
      }
      pv_start((ntiles - 1) % kDepth);
      pv_run((ntiles - 1) % kDepth, pb, [](int) {});
    } else {
#pragma unroll
      for (int j = 0; j < kDepth - 1; ++j) issue_tile(j, j);
      for (int it = 0; it < ntiles; ++it) {
        // tile `it` has landed once only the copies of the kDepth - 2 tiles
        // after it are pending; the buffer refilled in this iteration was last
        // read in iteration it - 1
        const TileSrc refill = tile_src(it + kDepth - 1);
        wait_vm<(kDepth - 2) * kCopies>();
        tile_barrier();
        settle(refill);
        score_tile(it, it + kDepth - 1, refill, s);
        pv_start(it % kDepth);
        softmax_ref(it, s);
        float p[8 * HB];
#pragma unroll
        for (int k = 0; k < 8 * HB; ++k) p[k] = weight(s, k);
        bf16x8_t pb[HB];
        pack(p, pb);
        pv_run(it % kDepth, pb, [](int) {});
      }
    }
    wait_vm_all();
    __syncthreads();
    if (!restart_flag) break;
    __syncthreads();  // every thread has seen the flag before it is cleared
    if (tid == 0) restart_flag = 0;
  }

#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = (w * HB + hb) * 16 + l16;
    // the four lanes of a head hold disjoint token subsets of l
    float l_tot = l_part[hb] + __shfl_xor(l_part[hb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = 1.0f / l_tot;
    uint16_t* po = a.part_out + (slot * H + h) * kDc + 4 * q4;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      uint2 v;
      v.x = cvt_bf16x2(o[hb][cb][0] * inv, o[hb][cb][1] * inv);
      v.y = cvt_bf16x2(o[hb][cb][2] * inv, o[hb][cb][3] * inv);
      *reinterpret_cast<uint2*>(po + 16 * cb) = v;
    }
    if (q4 == 0) a.part_lse[slot * H + h] = (m_ref[hb] + log2_hw(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// 3. split merge + W_UV projection
// ---------------------------------------------------------------------------
// grid: H * n_groups workgroups of 8 waves; a workgroup serves one head and
// `bpg` consecutive blocks of 16 batch rows, so W_UV,h is staged in LDS once
// per workgroup. Workgroups of one head share an XCD (linear id % 8 = h % 8).
// W_UV,h [512 x 128] is stored unpadded (256-byte rows) with an XOR swizzle of
// the 16-byte chunk index, and the merged o~ rows with a 1056-byte pitch; with
// these, the transposed W_UV reads (4 rows x 32 bytes per 16-lane group, rows
// 8 q4 + 0..3) and the 16-byte o~ reads (16 rows at one offset) are free of
// LDS bank conflicts, as measured with the SQ_LDS_BANK_CONFLICT counter.
constexpr int kORowB = 1056;  // merged o~ row in LDS: 512 bf16 + 32 bytes pad

__device__ __forceinline__ int wuv_swizzle(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }

__global__ __launch_bounds__(512) void mla_merge_project_kernel(MlaArgs a, int n_groups, int bpg) {
  __shared__ __attribute__((aligned(1024))) uint8_t w_smem[kDc * 256];   // 131072
  __shared__ __attribute__((aligned(16))) uint8_t o_smem[16 * kORowB];   // 16896
  LDS uint8_t* w_lds = (LDS uint8_t*)w_smem;
  LDS uint8_t* o_lds = (LDS uint8_t*)o_smem;

  const int H = a.num_heads;
  const int B = a.batch;
  const int x = blockIdx.x;
  const int h = ((x >> 3) / n_groups) * 8 + (x & 7);
  const int grp = (x >> 3) % n_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  const int64_t rows = (int64_t)B * H;

  {  // stage W_UV,h by the load-to-LDS path: 128 KiB = 128 wave-wide copies
    const uint16_t* wsrc = a.w_uv + (int64_t)h * kDc * 128;
    for (int k = w; k < 128; k += 8) {
      const int p = k * 64 + lane;   // 16-byte chunk in LDS
      const int row = p >> 4;
      const int c = (p & 15) ^ wuv_swizzle(row);
      load_to_lds16(wsrc + row * 128 + 8 * c, w_lds + k * 1024);
    }
  }

  // transposed-read offsets for this wave's 16 output columns (n-block w)
  const int tr_row = 8 * q4 + (l16 >> 2);        // + 32 ks (+4 for the upper half)
  const int tr_chunk = 2 * w + ((l16 & 3) >> 1);
  const int tr_half = 8 * (l16 & 1);

  const int nbb = (B + 15) / 16;
  for (int bbi = 0; bbi < bpg; ++bbi) {
    const int bb = grp * bpg + bbi;
    if (bb >= nbb) break;
    // Merge the splits: thread (slot r, 16 columns). With R < 16 valid rows in
    // the block, G = the largest power of two with G R <= 16 slots serve one
    // row, slot group g summing the splits s = g (mod G); the G partial rows
    // are then added through LDS. The weights exp(lse_s - lse) use all splits.
    {
      const int R = min(16, B - bb * 16);
      int G = 1;
      while (2 * G * R <= 16) G *= 2;
      const int r = tid >> 5;
      const int cs = tid & 31;
      const int rr = r / G, g = r % G;
      const int bidx = bb * 16 + rr;
      float acc[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
      if (rr < R) {
        const int64_t row_id = (int64_t)bidx * H + h;
        // the splits of this sequence: slots s * B + b (fixed) or P_b + s
        // (balanced, from the table the attention launch wrote)
        const bool bal = a.num_splits == 0;
        // (the table is clamped to the slots that exist)
        const int P = bal ? min(max(a.split_table[2 * bidx], 0), a.slots) : 0;
        const int n_s = bal ? min(a.split_table[2 * bidx + 1], a.slots - P) : a.num_splits;
        const int64_t s_base = bal ? (int64_t)P * H + h : row_id;
        const int64_t s_step = bal ? (int64_t)H : rows;
        // max and normaliser of the split lse values: the 32 threads of the
        // row (one half-wave) read every 32nd split each and combine
        float M = kNegInf;
        for (int s = cs; s < n_s; s += 32) M = fmaxf(M, a.part_lse[s_base + s * s_step]);
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        float lse_out = kNegInf;
        if (M != kNegInf) {
          const float m2 = M * kLog2e;
          float z = 0.f;
          for (int s = cs; s < n_s; s += 32) {
            const float v = a.part_lse[s_base + s * s_step];
            if (v != kNegInf) z += exp2_hw(fmaf(v, kLog2e, -m2));
          }
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) z += __shfl_xor(z, off);
          const float inv_z = 1.0f / z;
          // the partial rows are loaded kMergeBatch splits at a time, so their
          // loads are in flight together; an empty split (lse -inf) was never
          // written: its row is replaced by zeros rather than skipped
          constexpr int kMergeBatch = 4;
          for (int s0 = g; s0 < n_s; s0 += kMergeBatch * G) {
            uint4 u[kMergeBatch][2];
            float wgt[kMergeBatch];
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
              const int s = s0 + j * G;
              const float v = s < n_s ? a.part_lse[s_base + s * s_step] : kNegInf;
              wgt[j] = v == kNegInf ? 0.f : exp2_hw(fmaf(v, kLog2e, -m2)) * inv_z;
              const int s_in = s < n_s ? s : 0;
              const uint4* src = reinterpret_cast<const uint4*>(a.part_out + (s_base + s_in * s_step) * kDc + 16 * cs);
              u[j][0] = src[0];
              u[j][1] = src[1];
            }
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
              const bool live = wgt[j] != 0.f;
              float f[16];
              unpack_bf16x8(live ? u[j][0] : make_uint4(0u, 0u, 0u, 0u), f);
              unpack_bf16x8(live ? u[j][1] : make_uint4(0u, 0u, 0u, 0u), f + 8);
#pragma unroll
              for (int e = 0; e < 16; ++e) acc[e] = fmaf(wgt[j], f[e], acc[e]);
            }
          }
          lse_out = M + log2_hw(z) * kLn2;
        }
        if (g == 0 && cs == 0 && a.lse) a.lse[row_id] = lse_out;
      }
      auto store_row = [&](int slot, const float* v) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4_t w;
          w.x = cvt_bf16x2(v[8 * j + 0], v[8 * j + 1]);
          w.y = cvt_bf16x2(v[8 * j + 2], v[8 * j + 3]);
          w.z = cvt_bf16x2(v[8 * j + 4], v[8 * j + 5]);
          w.w = cvt_bf16x2(v[8 * j + 6], v[8 * j + 7]);
          *reinterpret_cast<LDS u32x4_t*>(o_lds + slot * kORowB + 2 * (16 * cs + 8 * j)) = w;
        }
      };
      store_row(r, acc);
      if (G > 1) {  // add the G partial rows of each valid row into slot rr
        __syncthreads();
        float fin[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) fin[e] = 0.f;
        if (g == 0 && rr < R) {
          for (int gg = 0; gg < G; ++gg) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u32x4_t w =
                  *reinterpret_cast<const LDS u32x4_t*>(o_lds + (rr * G + gg) * kORowB + 2 * (16 * cs + 8 * j));
              float f[8];
              unpack_bf16x8(uint4{w.x, w.y, w.z, w.w}, f);
#pragma unroll
              for (int e = 0; e < 8; ++e) fin[8 * j + e] += f[e];
            }
          }
        }
        __syncthreads();
        if (g == 0) store_row(rr, fin);
      }
    }
    wait_vm_all();
    __syncthreads();

    // out[b, e] = sum_c o~[b, c] W_UV[h, c, e]; wave w owns columns 16w .. 16w+15
    f32x4_t acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      const u32x4_t av = *reinterpret_cast<const LDS u32x4_t*>(o_lds + l16 * kORowB + 2 * (32 * ks + 8 * q4));
      const int row_lo = 32 * ks + tr_row;
      const int row_hi = row_lo + 4;
      const i16x4_t lo = lds_read_tr(w_lds + row_lo * 256 + 16 * (tr_chunk ^ wuv_swizzle(row_lo)) + tr_half);
      const i16x4_t hi = lds_read_tr(w_lds + row_hi * 256 + 16 * (tr_chunk ^ wuv_swizzle(row_hi)) + tr_half);
      acc2 = mfma16x16x32(as_bf16x8(av), join_tr(lo, hi), acc2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bidx = bb * 16 + 4 * q4 + i;
      if (bidx < B) a.out[((int64_t)bidx * H + h) * 128 + 16 * w + l16] = acc2[i];
    }
    __syncthreads();  // o_lds is rewritten by the next block
  }
}

}  // namespace

hipError_t launch_mla_absorb(const MlaArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(8 * a.num_heads), dim3(64), 0, st, a);  // H is a multiple of 8
  return hipGetLastError();
}

// Head counts with an attention shape: NW waves of HB blocks of 16 heads, NW
// dividing the 36 copies of a tile.
template <bool kPaged, typename F>
bool with_attend_shape(int num_heads, F&& f) {
  switch (num_heads) {
    case 16: f(mla_attend_kernel<1, 1, kPaged>, 1); return true;
    case 32: f(mla_attend_kernel<2, 1, kPaged>, 2); return true;
    case 48: f(mla_attend_kernel<3, 1, kPaged>, 3); return true;
    case 64: f(mla_attend_kernel<4, 1, kPaged>, 4); return true;
    case 96: f(mla_attend_kernel<3, 2, kPaged>, 3); return true;
    case 128: f(mla_attend_kernel<4, 2, kPaged>, 4); return true;
    default: return false;
  }
}

hipError_t launch_mla_attend(const MlaArgs& a, hipStream_t st) {
  const dim3 grid = a.num_splits > 0 ? dim3(a.num_splits, a.batch) : dim3(a.slots, 1);
  auto launch = [&](auto kernel, int nw) { hipLaunchKernelGGL(kernel, grid, dim3(64 * nw), 0, st, a); };
  const bool ok = a.page_shift > 0 ? with_attend_shape<true>(a.num_heads, launch)
                                   : with_attend_shape<false>(a.num_heads, launch);
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

int mla_attend_blocks_per_cu(int num_heads) {
  int n = 0;
  const bool ok = with_attend_shape<false>(num_heads, [&](auto kernel, int nw) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel), 64 * nw,
                                                     0) != hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
  });
  return ok ? n : 0;
}

hipError_t launch_mla_merge_project(const MlaArgs& a, hipStream_t st) {
  const int nbb = (a.batch + 15) / 16;
  // enough workgroups for one per CU (256), each covering bpg batch blocks
  int bpg = (nbb * a.num_heads + 255) / 256;
  bpg = bpg < 1 ? 1 : (bpg > nbb ? nbb : bpg);
  const int n_groups = (nbb + bpg - 1) / bpg;
  hipLaunchKernelGGL(mla_merge_project_kernel, dim3(a.num_heads * n_groups), dim3(512), 0, st, a,
                     n_groups, bpg);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  hipError_t e = launch_mla_absorb(a, st);
  if (e != hipSuccess) return e;
  e = launch_mla_attend(a, st);
  if (e != hipSuccess) return e;
  return launch_mla_merge_project(a, st);
}

}  // namespace da
