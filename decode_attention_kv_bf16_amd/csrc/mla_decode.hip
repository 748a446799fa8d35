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
//  1. mla_absorb_kernel   q^ = [q_nope W_UK^T | q_rope] (bf16) for all (b, h),
//     stored in the attention kernels' operand order (qhat_index).
//  2. mla_attend_kernel   one workgroup per (split, sequence); for 128 heads,
//     4 waves of 32 heads each (one wave per SIMD, accumulators in AGPRs).
//     32-row latent tiles are copied HBM -> LDS by the buffer load-to-LDS
//     path (buffer_load_dwordx4 ... lds, no register staging) into a ring of
//     4 tiles; each tile is read from LDS as the A operand of S^T (row-major
//     16-byte reads) and, transposed by ds_read_b64_tr_b16, as the A operand
//     of O^T. Each head's softmax reference max is fixed by its first tile, so
//     the accumulators are never rescaled in the loop (see kRefHeadroom).
//     Each split writes its normalised o~_s (bf16) and lse_s.
//  3. mla_merge_project_kernel  merges the splits by log-sum-exp, corrects each
//     lse for the bf16 rounding of q~ (with q~_lo from kernel 1) and
//     multiplies by W_UV,h on the matrix cores (W_UV,h staged in LDS, read
//     transposed).
#include "mla_common.h"

namespace da {
namespace {

// ---------------------------------------------------------------------------
// 1. query absorption
// ---------------------------------------------------------------------------
// A workgroup of 4 waves serves one head h, one of the kAbsorbParts slices
// of the 512 latent columns and up to kAbsorbRows batch rows. W_UK[h] rows of
// its slice are copied HBM -> LDS by the load-to-LDS path; q_nope rows of its
// batch block by ordinary loads into LDS. Wave w computes
// q~^T[c, b] = sum_e W_UK[h, c, e] q_nope[b, h, e] for its kAbsorbCols / 4
// columns on 16x16x32 matrix ops (both operands read from LDS, 16-byte reads
// of 16 rows at one chunk, rows XOR-swizzled by row mod 16), then writes
// bf16(q~) and q~_lo = bf16(q~ - bf16(q~)) into LDS, so that every row of q^
// and of q~_lo leaves in whole 16-byte pieces. The workgroups of the first
// slice also copy q_rope into q^. Eighth slices and 32-row blocks (24 KiB of
// LDS) let several workgroups share a CU, so one's copies overlap another's
// stores (about 1% faster per MLA call than quarter slices of 64 rows).
constexpr int kAbsorbRows = 32;    // batch rows per workgroup
constexpr int kAbsorbParts = 8;    // column slices per head
constexpr int kAbsorbCols = kDc / kAbsorbParts;   // latent columns per workgroup
constexpr int kAbsorbCB = kAbsorbCols / 64;       // 16-column blocks per wave
constexpr int kAbsorbBB = kAbsorbRows / 16;       // 16-row batch blocks
constexpr int kAbsorbOutB = 2 * kAbsorbCols * 2 + 16;   // staged row: hi | lo (bf16) + pad

__device__ __forceinline__ int absorb_chunk(int row, int chunk) { return chunk ^ (row & 15); }

__global__ __launch_bounds__(256) void mla_absorb_kernel(MlaArgs a) {
  // W rows (256 x 256 B), then q rows (64 x 256 B); once both are read, the
  // same bytes stage the outputs (64 rows x kAbsorbOutB)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kAbsorbCols * 256 + kAbsorbRows * 256];
  static_assert(kAbsorbRows * kAbsorbOutB <= kAbsorbCols * 256 + kAbsorbRows * 256, "staging fits");
  LDS uint8_t* w_lds = (LDS uint8_t*)smem;
  LDS uint8_t* q_lds = w_lds + kAbsorbCols * 256;

  const int H = a.num_heads;
  const int B = a.batch;
  // grid: (head, slice) pairs, batch blocks. The slices of a head share an
  // XCD (linear id mod 8 picks the XCD), so its q_nope rows come from one L2.
  // With H a multiple of 64 the 8 heads h = 8k .. 8k + 7 also share one (XCD
  // k mod 8): their pieces of q^ in operand order fill whole 128-byte lines,
  // which that XCD's L2 then writes back whole. Otherwise head h goes to XCD
  // h mod 8.
  const int x = blockIdx.x;
  int h, part;   // the head and its column slice
  if (H % 64 == 0) {
    const int t = x >> 3, t2 = t >> 3;
    h = (t2 / kAbsorbParts) * 64 + (x & 7) * 8 + (t & 7);
    part = t2 % kAbsorbParts;
  } else {
    h = (x / (8 * kAbsorbParts)) * 8 + (x & 7);
    part = (x >> 3) % kAbsorbParts;
  }
  const int b0 = blockIdx.y * kAbsorbRows;
  const int nb = min(kAbsorbRows, B - b0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q4 = lane >> 4, l16 = lane & 15;
  const int c0 = part * kAbsorbCols;

  {  // W_UK[h, c0 .. c0 + kAbsorbCols - 1, :]: kAbsorbCols / 4 wave-wide 1 KiB
     // copies; lane l of copy k fills LDS chunk 64 k + l (row 4k + l / 16)
    const uint16_t* wsrc = a.w_uk + ((int64_t)h * kDc + c0) * 128;
#pragma unroll
    for (int i = 0; i < kAbsorbCols / 16; ++i) {
      const int k = w + 4 * i;
      const int p = k * 64 + lane;
      const int row = p >> 4;
      const int c = absorb_chunk(row, p & 15);
      load_to_lds16(wsrc + row * 128 + 8 * c, w_lds + k * 1024);
    }
  }
  {  // q_nope rows b0 .. b0 + nb - 1 of head h (zeros past the batch)
    for (int p = tid; p < kAbsorbRows * 16; p += 256) {
      const int row = p >> 4, c = p & 15;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < nb) v = *reinterpret_cast<const u32x4_t*>(a.q_nope + ((int64_t)(b0 + row) * H + h) * 128 + 8 * c);
      *reinterpret_cast<LDS u32x4_t*>(q_lds + row * 256 + 16 * absorb_chunk(row, c)) = v;
    }
  }
  wait_vm_all();
  __syncthreads();

  // wave w: columns c0 + 16 (kAbsorbCB w + cb) + (0..15), batch rows 16 bb + (0..15)
  f32x4_t acc[kAbsorbCB][kAbsorbBB];
#pragma unroll
  for (int cb = 0; cb < kAbsorbCB; ++cb)
#pragma unroll
    for (int bb = 0; bb < kAbsorbBB; ++bb) acc[cb][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8_t wa[kAbsorbCB], qb[kAbsorbBB];
#pragma unroll
    for (int cb = 0; cb < kAbsorbCB; ++cb) {
      const int row = 16 * (kAbsorbCB * w + cb) + l16;
      wa[cb] = as_bf16x8(*reinterpret_cast<const LDS u32x4_t*>(w_lds + row * 256 + 16 * absorb_chunk(row, 4 * ks + q4)));
    }
#pragma unroll
    for (int bb = 0; bb < kAbsorbBB; ++bb) {
      const int row = 16 * bb + l16;
      qb[bb] = as_bf16x8(*reinterpret_cast<const LDS u32x4_t*>(q_lds + row * 256 + 16 * absorb_chunk(row, 4 * ks + q4)));
    }
#pragma unroll
    for (int cb = 0; cb < kAbsorbCB; ++cb)
#pragma unroll
      for (int bb = 0; bb < kAbsorbBB; ++bb) acc[cb][bb] = mfma16x16x32(wa[cb], qb[bb], acc[cb][bb]);
  }
  __syncthreads();   // every wave is done reading W and q: their bytes become the staging area

  // lane holds q~[b = 16 bb + l16][c = 16 (kAbsorbCB w + cb) + 4 q4 + i], i = 0..3:
  // bf16(q~) to the row's first part, what the rounding left out (exact in
  // float32) to its second part
  LDS uint8_t* st = w_lds;
#pragma unroll
  for (int cb = 0; cb < kAbsorbCB; ++cb)
#pragma unroll
    for (int bb = 0; bb < kAbsorbBB; ++bb) {
      const f32x4_t v = acc[cb][bb];
      u32x2_t hi, lo;
      hi.x = cvt_bf16x2(v[0], v[1]);
      hi.y = cvt_bf16x2(v[2], v[3]);
      lo.x = cvt_bf16x2(v[0] - bf16_lo(hi.x), v[1] - bf16_hi(hi.x));
      lo.y = cvt_bf16x2(v[2] - bf16_lo(hi.y), v[3] - bf16_hi(hi.y));
      const int row = 16 * bb + l16;
      const int col = 16 * (kAbsorbCB * w + cb) + 4 * q4;
      *reinterpret_cast<LDS u32x2_t*>(st + row * kAbsorbOutB + 2 * col) = hi;
      *reinterpret_cast<LDS u32x2_t*>(st + row * kAbsorbOutB + 2 * (kAbsorbCols + col)) = lo;
    }
  __syncthreads();

  // rows out: each row's kAbsorbCols hi and lo columns are 2 x kAbsorbCols / 8 pieces of 16 B
  constexpr int kPieces = kAbsorbCols / 8;
  for (int p = tid; p < nb * 2 * kPieces; p += 256) {
    const int row = p / (2 * kPieces), piece = p % (2 * kPieces);
    const int is_lo = piece / kPieces, c8 = (piece % kPieces) * 8;   // is_lo: the q~_lo half
    const u32x4_t v = *reinterpret_cast<const LDS u32x4_t*>(st + row * kAbsorbOutB + 2 * (is_lo * kAbsorbCols + c8));
    const int64_t bh = (int64_t)(b0 + row) * H + h;
    uint16_t* dst = is_lo == 0 ? a.q_hat + qhat_index(a, b0 + row, h, c0 + c8) : a.q_lo + bh * kDc + c0 + c8;
    *reinterpret_cast<u32x4_t*>(dst) = v;
  }
  if (part == 0) {  // q_rope (already rotated) into q^: 8 pieces of 16 B per row
    for (int p = tid; p < nb * 8; p += 256) {
      const int row = p >> 3, ch = p & 7;
      const int64_t bh = (int64_t)(b0 + row) * H + h;
      *reinterpret_cast<u32x4_t*>(a.q_hat + qhat_index(a, b0 + row, h, kDc + 8 * ch)) =
          *reinterpret_cast<const u32x4_t*>(a.q_rope + bh * 64 + 8 * ch);
    }
  }
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
      copy16(__builtin_amdgcn_readfirstlane(second) ? src.half[1] : src.half[0], voff[i], dst);
    } else {
      copy16(src, voff[i], dst);
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
// 2b. split-KV latent attention on 32x32x16 matrix ops
// ---------------------------------------------------------------------------
// The same computation, tiles, LDS ring, split assignment and softmax
// reference as mla_attend_kernel, for head counts that are multiples of 32:
// NW waves of 32 heads each, every wave one 32x32 block of heads. A 32x32x16
// operation does the work of two 16x16x32 ones in one instruction, so a
// 32-row tile takes a wave 36 score and 32 value instructions instead of 72
// and 64, and each lane keeps the 32 tokens' scores of one head in 16
// registers. One wave per SIMD issues every instruction of its tile in
// order, so the instructions around the matrix ops (LDS reads, softmax, copy
// issue, waits) bound how busy the matrix core can be; this form issues
// about half as many.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (lane l, g = l / 32):
//   A [32 x 16]: row l % 32, k = 8 g .. 8 g + 7     (8 bf16 per lane)
//   B [16 x 32]: column l % 32, k = 8 g .. 8 g + 7
//   D [32 x 32]: column l % 32, rows 8 i + 4 g + r in register 4 i + r
// Scores S^T = C q^^T: A = the tile's rows (row-major 16-byte LDS reads),
// B = q^ of the lane's head, D = [token x head]: lane l holds head l % 32 at
// tokens 8 i + 4 g + r. Values O^T += C[:, :512]^T P^T in 16 column blocks of
// 32: B = the weights, contraction element e of matrix op m standing for
// token 16 m + 8 (e / 4) + 4 g + e % 4, which is exactly score register
// 8 m + e of the lane; A = the tile read transposed, 4 rows per
// ds_read_b64_tr_b16, two reads per operand (rows 16 m + 4 g .. + 3 and
// 16 m + 8 + 4 g .. + 3).
template <int NW, bool kPaged>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_attend32_kernel(MlaArgs a) {
  constexpr int kCopies = kTileDma / NW;
  static_assert(kTileDma % NW == 0, "copies split evenly over the waves");
  constexpr int kDepth = (3 * kCopies <= 63) ? 4 : 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDepth * kTileB];
  LDS uint8_t* lds = (LDS uint8_t*)smem;
  static_assert(kDepth * kTileB >= NW * 32 * kOutRowB, "the output staging fits in the ring");

  constexpr int H = NW * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int j16 = lane & 15, q16 = lane >> 4;
  const SplitWork work = assign_split(a, lane, blockIdx.x == 0 && w == 0);
  if (!work.valid) return;
  const int b = work.b;
  const int64_t slot = work.slot;
  int t_begin = work.t_begin;   // re-read per pass of the restart loop (see there)
  const int t_end = work.t_end;

  if (t_begin >= t_end) {  // fixed splits only: a split past the sequence's end
    for (int i = tid; i < H; i += NW * 64) a.part_lse[slot * H + i] = kNegInf;
    return;
  }

  const uint16_t* cache_b = a.cache + (int64_t)b * a.cache_sb;
  const int ntiles = (t_end - t_begin + kTok - 1) / kTok;

  // HBM -> LDS copies of one tile, exactly as in mla_attend_kernel
  const uint32_t row_bytes = (uint32_t)a.cache_st * 2u;
  uint32_t voff[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int p = (w + NW * i) * 64 + lane;
    const int row = p / kChunks;
    const int c = (p - row * kChunks) ^ row_swizzle32(row);
    voff[i] = (uint32_t)(kPaged ? row & 15 : row) * row_bytes + 16u * (uint32_t)c;
  }
  const uint32_t lds_w0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds + (uint32_t)w * 1024u);
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
  auto settle = [&](const TileSrc& src) {
    if constexpr (kPaged) asm volatile("" ::"s"(src.half[0]), "s"(src.half[1]));
  };
  auto issue_copy = [&](const TileSrc& src, int i, int buf) {
    const uint32_t dst = lds_w0 + (uint32_t)(buf * kTileB + NW * i * 1024);
    if constexpr (kPaged) {
      constexpr int kHalf = kTileDma / 2;
      const int second = NW * i >= kHalf ? 1 : NW * i + NW <= kHalf ? 0 : (w + NW * i >= kHalf);
      copy16(__builtin_amdgcn_readfirstlane(second) ? src.half[1] : src.half[0], voff[i], dst);
    } else {
      copy16(src, voff[i], dst);
    }
  };
  auto issue_tile = [&](int it, int buf) {
    const TileSrc src = tile_src(it);
    settle(src);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) issue_copy(src, i, buf);
  };

  // absorbed query of the lane's head as B operands: q^[h][16 ks + 8 g .. + 8]
  const int h = 32 * w + l32;
  bf16x8_t qb[36];
  {
    // operand order (H is a multiple of 32 here): one contiguous KiB per step
    const uint16_t* qp = a.q_hat + qhat_index(a, b, 32 * w, 0) + 8 * lane;
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 512 * ks));
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) asm volatile("" ::"v"(qb[ks]));
  }

  float m_ref = kNegInf;  // reference max (log2 units) of the lane's head, fixed by the first tile
  float thr = kNegInf;    // raw score above which the reference must be raised
  // score operand reads: row l32, logical chunk 2 ks + g -> 8 (ks / 4) + ((2 (ks % 4) + g) ^ f)
  const int f_s = row_swizzle32(l32);
  int s_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) s_off[m] = l32 * kRowB + 16 * ((2 * m + g) ^ f_s);
  // transposed reads: rows r_t (+ 16 m) and r_t + 8 (+ 16 m) with r_t = 4 (q16 / 2) + j16 / 4,
  // columns 32 cb + 16 (q16 % 2) + 0..15; the swizzle differs for the two rows
  const int r_t = 4 * (q16 >> 1) + (j16 >> 2);
  int t_off[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int cbl = 0; cbl < 2; ++cbl)
      t_off[hf][cbl] = (r_t + 8 * hf) * kRowB +
                       16 * ((4 * cbl + 2 * (q16 & 1) + ((j16 & 3) >> 1)) ^ row_swizzle32(r_t + 8 * hf)) +
                       8 * (j16 & 1);

  __shared__ int restart_flag;
  if (tid == 0) restart_flag = 0;

  f32x16_t o[16];
  float l_part;  // this lane's share of sum_j 2^(s_j - m_ref) (the other tokens are in lane l ^ 32)

  // S^T of tile `it`; the copies of tile `refill_it` go out spread over the k-steps
  constexpr int kSRing = 5;
  auto score_tile = [&](int it, int refill_it, const TileSrc& refill_src, f32x16_t& s) {
    const int refill_buf = refill_it % kDepth;
    const LDS uint8_t* tile = lds + (it % kDepth) * kTileB;
    u32x4_t ra[kSRing];
#pragma unroll
    for (int ks = 0; ks < kSRing - 1; ++ks)
      ra[ks] = *reinterpret_cast<const LDS u32x4_t*>(tile + s_off[ks & 3] + 128 * (ks >> 2));
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
#pragma unroll
      for (int i = ks * kCopies / 36; i < (ks + 1) * kCopies / 36; ++i) issue_copy(refill_src, i, refill_buf);
      const int kn = ks + kSRing - 1;
      if (kn < 36) ra[kn % kSRing] = *reinterpret_cast<const LDS u32x4_t*>(tile + s_off[kn & 3] + 128 * (kn >> 2));
      if (ks == 0)
        qk_first(s, as_bf16x8(ra[0]), qb[0]);
      else if (ks < 35)
        qk_next(s, as_bf16x8(ra[ks % kSRing]), qb[ks]);
      else
        qk_last(s, as_bf16x8(ra[ks % kSRing]), qb[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax reference of tile `it` (as in mla_attend_kernel): rows past the
  // split end get score -inf; only a split's first tile and a score beyond the
  // headroom need the head-wide max, taken with the partner lane l ^ 32.
  auto softmax_ref = [&](int it, f32x16_t& s) {
    const int nv = t_end - (t_begin + it * kTok);
    if (nv < kTok) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * g + (r & 3) >= nv) s[r] = kNegInf;
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
  auto pack = [&](const float (&p)[16], bf16x8_t (&pb)[2]) {
    l_part += (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
              (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint4 pw;
      pw.x = cvt_bf16x2(p[8 * m + 0], p[8 * m + 1]);
      pw.y = cvt_bf16x2(p[8 * m + 2], p[8 * m + 3]);
      pw.z = cvt_bf16x2(p[8 * m + 4], p[8 * m + 5]);
      pw.w = cvt_bf16x2(p[8 * m + 6], p[8 * m + 7]);
      pb[m] = as_bf16x8(pw);
    }
  };
  // O^T += C^T P^T for the tile in ring buffer `buf`, matrix op k = 16 m + cb;
  // `extra(k)` runs in the shadow of matrix op k
  constexpr int kTRing = 4;
  i16x4_t tlo[kTRing], thi[kTRing];
  auto read_t = [&](const LDS uint8_t* tile, int k) {
    const int m = k >> 4, cb = k & 15;
    const int off = 128 * (cb >> 1) + 16 * m * kRowB;
    tlo[k % kTRing] = lds_read_tr(tile + t_off[0][cb & 1] + off);
    thi[k % kTRing] = lds_read_tr(tile + t_off[1][cb & 1] + off);
  };
  auto pv_start = [&](int buf) {
    const LDS uint8_t* tile = lds + buf * kTileB;
#pragma unroll
    for (int k = 0; k < kTRing - 1; ++k) read_t(tile, k);
  };
  auto pv_run = [&](int buf, const bf16x8_t (&pb)[2], auto&& extra) {
    const LDS uint8_t* tile = lds + buf * kTileB;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if (k + kTRing - 1 < 32) read_t(tile, k + kTRing - 1);
      const int m = k >> 4, cb = k & 15;
      o[cb] = mfma32x32x16(join_tr(tlo[k % kTRing], thi[k % kTRing]), pb[m], o[cb]);
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
    f32x16_t s;
    bf16x8_t pb[2];
    if constexpr (kDepth == 4) {
      // as in mla_attend_kernel: the weights of tile `it` are computed in the
      // shadow of the value product of tile it - 1; tiles it + 1 and it + 2
      // are in flight
#pragma unroll
      for (int j = 0; j < 2; ++j) issue_tile(j, j);
      {
        const TileSrc refill = tile_src(2);
        wait_vm<kCopies>();
        tile_barrier();
        settle(refill);
        score_tile(0, 2, refill, s);
        softmax_ref(0, s);
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = weight(s, r);
        pack(p, pb);
      }
      for (int it = 1; it < ntiles; ++it) {
        const TileSrc refill = tile_src(it + 2);
        wait_vm<kCopies>();
        tile_barrier();
        settle(refill);
        score_tile(it, it + 2, refill, s);
        pv_start((it - 1) % kDepth);
        softmax_ref(it, s);
        float p[16];
        pv_run((it - 1) % kDepth, pb, [&](int k) {
          if ((k & 1) == 0) p[k >> 1] = weight(s, k >> 1);
        });
        pack(p, pb);
      }
      pv_start((ntiles - 1) % kDepth);
      pv_run((ntiles - 1) % kDepth, pb, [](int) {});
    } else {
#pragma unroll
      for (int j = 0; j < kDepth - 1; ++j) issue_tile(j, j);
      for (int it = 0; it < ntiles; ++it) {
        const TileSrc refill = tile_src(it + kDepth - 1);
        wait_vm<(kDepth - 2) * kCopies>();
        tile_barrier();
        settle(refill);
        score_tile(it, it + kDepth - 1, refill, s);
        pv_start(it % kDepth);
        softmax_ref(it, s);
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = weight(s, r);
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

  // o~_s = O / l (bf16) through LDS (the ring is free: every wave has passed
  // the barrier above), so that each head's 1 KiB row leaves in whole 16-byte
  // pieces: lane l holds columns 32 cb + 8 i + 4 g .. + 3 of head l % 32
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
  uint16_t* po = a.part_out + (slot * H + 32 * w) * kDc;
#pragma unroll 4
  for (int r = 0; r < 32; ++r)
    *reinterpret_cast<u32x4_t*>(po + r * kDc + 8 * lane) =
        *reinterpret_cast<const LDS u32x4_t*>(stage + r * kOutRowB + 16 * lane);
  if (g == 0) a.part_lse[slot * H + h] = (m_ref + log2_hw(l_tot)) * kLn2;
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

// Per thread, the merge is online over its splits: a running reference m,
// normaliser z and 16 weighted columns, rescaled when m grows. A batch of
// kMergeBatch splits (their o~_s pieces and lse_s) is loaded at once, so a
// row of up to kMergeBatch splits per thread is one round trip; the first
// batch of the next block is loaded while the current block is projected.
constexpr int kMergeBatch = 8;

struct MergeRow {
  int n_s;            // splits of the row the thread serves (0: no row)
  int64_t s_base;     // part_lse index of split 0 of that row and head
  int64_t s_step;     // index step between its splits
};

struct MergeBatch {
  uint4 u[kMergeBatch][2];
  float lse[kMergeBatch];
};

__global__ __launch_bounds__(512) void mla_merge_project_kernel(MlaArgs a, int n_groups, int bpg) {
  __shared__ __attribute__((aligned(1024))) uint8_t w_smem[kDc * 256];   // 131072
  __shared__ __attribute__((aligned(16))) uint8_t o_smem[16 * kORowB];   // 16896
  __shared__ float m_sm[16], z_sm[16];  // reference and normaliser of each thread row
  __shared__ float lse_sm[16];          // merged lse of the block's rows, before the correction
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
  const int r = tid >> 5;        // thread (row slot r, columns 16 cs .. 16 cs + 15)
  const int cs = tid & 31;
  const int64_t rows = (int64_t)B * H;
  const bool bal = a.num_splits == 0;

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

  // Rows of block bb: R <= 16 valid rows; G = the largest power of two with
  // G R <= 16 thread rows serve one row, group g taking the splits s = g
  // (mod G). Slot r serves row r / G, group r % G.
  auto block_rows = [&](int bb) { return min(16, B - bb * 16); };
  auto groups_of = [](int R) {
    int G = 1;
    while (2 * G * R <= 16) G *= 2;
    return G;
  };
  auto row_of = [&](int bb) -> MergeRow {
    const int R = block_rows(bb);
    const int G = groups_of(R);
    const int rr = r / G;
    MergeRow m{0, 0, 0};
    if (rr >= R) return m;
    const int bidx = bb * 16 + rr;
    if (bal) {
      // the splits of this sequence: slots P_b .. P_b + S_b - 1 (from the
      // table the attention launch wrote), clamped to the slots that exist
      const int P = min(max(a.split_table[2 * bidx], 0), a.slots);
      m.n_s = min(a.split_table[2 * bidx + 1], a.slots - P);
      m.s_base = (int64_t)P * H + h;
      m.s_step = H;
    } else {
      m.n_s = a.num_splits;          // slots s * B + b
      m.s_base = (int64_t)bidx * H + h;
      m.s_step = rows;
    }
    return m;
  };
  // loads of the thread's splits g + G (j0 + j), j < kMergeBatch; splits that
  // do not exist read nothing (lse -inf)
  auto load_batch = [&](const MergeRow& m, int G, int g, int j0, MergeBatch& bt) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int s = g + G * (j0 + j);
      bt.lse[j] = kNegInf;
      bt.u[j][0] = bt.u[j][1] = make_uint4(0u, 0u, 0u, 0u);
      if (s < m.n_s) {
        const int64_t idx = m.s_base + s * m.s_step;
        bt.lse[j] = a.part_lse[idx];
        const uint4* src = reinterpret_cast<const uint4*>(a.part_out + idx * kDc + 16 * cs);
        bt.u[j][0] = src[0];
        bt.u[j][1] = src[1];
      }
    }
  };

  const int nbb = (B + 15) / 16;
  const int bb0 = grp * bpg;
  MergeRow cur = bb0 < nbb ? row_of(bb0) : MergeRow{0, 0, 0};
  MergeBatch bt;
  if (bb0 < nbb) load_batch(cur, groups_of(block_rows(bb0)), r % groups_of(block_rows(bb0)), 0, bt);

  for (int bbi = 0; bbi < bpg; ++bbi) {
    const int bb = bb0 + bbi;
    if (bb >= nbb) break;
    const int R = block_rows(bb);
    const int G = groups_of(R);
    const int rr = r / G, g = r % G;
    // q~_lo of row r of the block (columns 16 cs ..), for the lse correction
    uint4 lo[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    if (r < R && a.lse) {
      const uint4* src = reinterpret_cast<const uint4*>(a.q_lo + ((int64_t)(bb * 16 + r) * H + h) * kDc + 16 * cs);
      lo[0] = src[0];
      lo[1] = src[1];
    }
    // online merge of the thread's splits (log2 domain)
    float m2 = kNegInf, z = 0.f;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int j0 = 0;; j0 += kMergeBatch) {
      float bm = kNegInf;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) bm = fmaxf(bm, bt.lse[j] * kLog2e);
      if (bm != kNegInf) {
        const float mn = fmaxf(m2, bm);
        const float f = exp2_hw(m2 - mn);   // 0 when m2 is -inf
        z *= f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] *= f;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
          // an empty split (lse -inf: a fixed split past the sequence's end,
          // or no split) wrote no pieces; what its slot holds is never used
          if (bt.lse[j] == kNegInf) continue;
          const float wj = exp2_hw(fmaf(bt.lse[j], kLog2e, -mn));
          z += wj;
          float fv[16];
          unpack_bf16x8(bt.u[j][0], fv);
          unpack_bf16x8(bt.u[j][1], fv + 8);
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = fmaf(wj, fv[e], acc[e]);
        }
        m2 = mn;
      }
      if (g + G * (j0 + kMergeBatch) >= cur.n_s) break;
      load_batch(cur, G, g, j0 + kMergeBatch, bt);
    }
    // this wave's W_UV copies have landed (the barriers below make every
    // wave's visible); waited for here, before the next block's loads go out
    if (bbi == 0) wait_vm_all();
    // the next block's rows and first batch, in flight during this block's
    // combine and projection
    MergeRow nxt{0, 0, 0};
    if (bbi + 1 < bpg && bb + 1 < nbb) {
      nxt = row_of(bb + 1);
      const int G1 = groups_of(block_rows(bb + 1));
      load_batch(nxt, G1, r % G1, 0, bt);
    }

    auto store_row = [&](int slot, const float* v) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4_t wv;
        wv.x = cvt_bf16x2(v[8 * j + 0], v[8 * j + 1]);
        wv.y = cvt_bf16x2(v[8 * j + 2], v[8 * j + 3]);
        wv.z = cvt_bf16x2(v[8 * j + 4], v[8 * j + 5]);
        wv.w = cvt_bf16x2(v[8 * j + 6], v[8 * j + 7]);
        *reinterpret_cast<LDS u32x4_t*>(o_lds + slot * kORowB + 2 * (16 * cs + 8 * j)) = wv;
      }
    };
    if (G == 1) {
      // one thread row per row: o~ = acc / z, lse = m + log z
      if (rr < R) {
        const float inv = z > 0.f ? 1.0f / z : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] *= inv;
        if (cs == 0) lse_sm[rr] = z > 0.f ? (m2 + log2_hw(z)) * kLn2 : kNegInf;
      }
      store_row(r, acc);
    } else {
      // G groups per row: share each group's (m, z), scale its columns by
      // 2^(m_g - M) / Z and add the G rows through LDS
      if (cs == 0) {
        m_sm[r] = m2;
        z_sm[r] = z;
      }
      __syncthreads();
      float M = kNegInf, Z = 0.f;
      if (rr < R) {
        for (int gg = 0; gg < G; ++gg) M = fmaxf(M, m_sm[rr * G + gg]);
        if (M != kNegInf)
          for (int gg = 0; gg < G; ++gg) Z += z_sm[rr * G + gg] * exp2_hw(m_sm[rr * G + gg] - M);
      }
      const float f = (rr < R && Z > 0.f && m2 != kNegInf) ? exp2_hw(m2 - M) / Z : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] *= f;
      store_row(r, acc);
      __syncthreads();
      float fin[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) fin[e] = 0.f;
      if (g == 0 && rr < R) {
        for (int gg = 0; gg < G; ++gg) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x4_t wv =
                *reinterpret_cast<const LDS u32x4_t*>(o_lds + (rr * G + gg) * kORowB + 2 * (16 * cs + 8 * j));
            float fv[8];
            unpack_bf16x8(uint4{wv.x, wv.y, wv.z, wv.w}, fv);
#pragma unroll
            for (int e = 0; e < 8; ++e) fin[8 * j + e] += fv[e];
          }
        }
        if (cs == 0) lse_sm[rr] = Z > 0.f ? (M + log2_hw(Z)) * kLn2 : kNegInf;
      }
      __syncthreads();
      if (g == 0) store_row(rr, fin);
    }
    __syncthreads();

    // lse of row r: the scores were computed with bf16(q~); with q~ itself
    // every score of the row moves by scale q~_lo . c_j, which moves the
    // log-sum-exp by sum_j p_j scale q~_lo . c_j = scale q~_lo . o~ to first
    // order (o~ = sum_j p_j c_j, the merged row in LDS). What remains is of
    // second order in these shifts (~1e-6 at the method's scales).
    if (a.lse) {
      float d = 0.f;
      if (r < R) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4_t ov = *reinterpret_cast<const LDS u32x4_t*>(o_lds + r * kORowB + 2 * (16 * cs + 8 * j));
          float fo[8], fl[8];
          unpack_bf16x8(uint4{ov.x, ov.y, ov.z, ov.w}, fo);
          unpack_bf16x8(lo[j], fl);
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(fo[e], fl[e], d);
        }
      }
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) d += __shfl_xor(d, off);
      if (r < R && cs == 0) a.lse[(int64_t)(bb * 16 + r) * H + h] = lse_sm[r] + a.scale * d;
    }

    // out[b, e] = sum_c o~[b, c] W_UV[h, c, e]; wave w owns columns 16w .. 16w+15
    f32x4_t acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      const u32x4_t av = *reinterpret_cast<const LDS u32x4_t*>(o_lds + l16 * kORowB + 2 * (32 * ks + 8 * q4));
      const int row_lo = 32 * ks + tr_row;
      const int row_hi = row_lo + 4;
      const i16x4_t lo_t = lds_read_tr(w_lds + row_lo * 256 + 16 * (tr_chunk ^ wuv_swizzle(row_lo)) + tr_half);
      const i16x4_t hi_t = lds_read_tr(w_lds + row_hi * 256 + 16 * (tr_chunk ^ wuv_swizzle(row_hi)) + tr_half);
      acc2 = mfma16x16x32(as_bf16x8(av), join_tr(lo_t, hi_t), acc2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bidx = bb * 16 + 4 * q4 + i;
      if (bidx < B) a.out[((int64_t)bidx * H + h) * 128 + 16 * w + l16] = acc2[i];
    }
    __syncthreads();  // o_lds is rewritten by the next block
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_mla_absorb(const MlaArgs& a, hipStream_t st) {
  // H is a multiple of 8: (head, slice) pairs in runs of 8 heads per slice
  hipLaunchKernelGGL(mla_absorb_kernel, dim3(kAbsorbParts * a.num_heads, (a.batch + kAbsorbRows - 1) / kAbsorbRows), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

// Head counts with an attention shape. Multiples of 32 run the 32x32x16
// kernel (NW waves of 32 heads); 16 and 48 the 16x16x32 one (NW waves of HB
// blocks of 16 heads). NW divides the 36 copies of a tile.
template <bool kPaged, typename F>
bool with_attend_shape(int num_heads, F&& f) {
  switch (num_heads) {
    case 16: f(mla_attend_kernel<1, 1, kPaged>, 1); return true;
    case 32: f(mla_attend32_kernel<1, kPaged>, 1); return true;
    case 48: f(mla_attend_kernel<3, 1, kPaged>, 3); return true;
    case 64: f(mla_attend32_kernel<2, kPaged>, 2); return true;
    case 96: f(mla_attend32_kernel<3, kPaged>, 3); return true;
    case 128: f(mla_attend32_kernel<4, kPaged>, 4); return true;
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
