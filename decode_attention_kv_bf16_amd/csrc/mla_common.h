// Device code shared by the absorbed-MLA attention kernels (bf16 and E4M3
// latent caches): operand types, tile geometry, LDS and copy helpers, the
// split assignment and the score chain of the 32x32x16 form.
#pragma once

#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
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
// LDS row of one head's normalised 512-wide output when a split stages it for
// the store: 1 KiB + 16 bytes, so that the 32 heads a store instruction covers
// fall on different banks.
constexpr int kOutRowB = kDc * 2 + 16;

// Where the absorbed queries q^ [B, H, 576] (bf16) live. When H is a
// multiple of 32 they are stored in the operand order of the 32x32x16
// attention kernels: for sequence b and head block hb (heads 32 hb .. + 31),
// 36 k-steps of 1 KiB, step ks holding for lane l = 32 g + i the 8 values
// q^[b, 32 hb + i][16 ks + 8 g .. + 7]. A wave's load of one step is then one
// contiguous KiB; in row order it touched 32 rows at 32 bytes each, and the
// 147 KiB of a sequence's queries took about 3.7 us longer to arrive at the
// start of every split. Other head counts keep rows [B, H, 576].
// qhat_index: element offset of q^[b, h, c] for c a multiple of 8.
__device__ __forceinline__ int64_t qhat_index(const MlaArgs& a, int b, int h, int c) {
  if (a.num_heads % 32 == 0) {
    const int64_t blk = (int64_t)b * (a.num_heads / 32) + h / 32;
    return (blk * 36 + c / 16) * 512 + ((((c >> 3) & 1) << 5) + (h & 31)) * 8;
  }
  return ((int64_t)b * a.num_heads + h) * kRowE + c;
}

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

// The swizzle of the 32x32x16 kernel, whose operand reads take other row
// sets: (a) 16-byte reads of 32 consecutive rows at one logical chunk and
// (b) transposing 8-byte reads of 4 consecutive rows x 64 bytes per 32 lanes.
// With f(r) = r mod 8 both conflict 2-way (rows one apart on the same banks;
// measured 50% conflict cycles); f(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)
// gives rows 4k and 4k + 2 disjoint chunk sets and any 8 rows of one parity
// 8 different ones, and measured no conflict cycles for either pattern. f is
// the same for rows r and r + 16, not for r and r + 8.
__device__ __forceinline__ int row_swizzle32(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

// Load-to-LDS copies as in da_device.h, with the LDS address handed to the
// asm in M0 through an "{m0}" operand instead of saving and restoring M0
// inside it (fewer scalar registers live across the unrolled loop). The
// s_nop is the wait state an LDS copy needs after M0 is written.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voffset), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

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
// score chain of the 32x32x16 form
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The score chain in vector registers. The 32x32 output accumulators take all
// 256 accumulation registers of a wave; left to itself the compiler also puts
// the score accumulator there and moves 16 output registers out and back on
// every tile. Written as asm with "v" operands, the chain stays in vector
// registers. Hazards the compiler does not see in asm: a chained operation
// reading the previous one's result as its accumulator input with the same
// shape and registers needs no wait (the hardware forwards it); vector-ALU
// reads of the final result need the result written back, so the last step
// of the chain is followed by 24 wait states inside its own asm block. The
// A and B operands come from LDS and global loads, whose completion the
// compiler's own waits cover (it sees the asm's register operands).
__device__ __forceinline__ void qk_first(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_last(f32x16_t& s, bf16x8_t a, bf16x8_t b) {
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 7"
      : "+v"(s)
      : "v"(a), "v"(b));
}

}  // namespace
}  // namespace da
