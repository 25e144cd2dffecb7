// MLA decode attention over a paged bf16 latent cache, bf16 MFMA on gfx950.
//
// Computes, per sequence b and query head h (moeflux mla_attn_forward.rs,
// mla_sdpa_folded; turbospark deepseek2/attn.rs, encode_mla_attention_decode):
//   s[t]   = scale * q_abs[b,h,:] . row_t            (row_t = [c_kv ; k_pe], 576 wide)
//   p      = softmax over t < len_b
//   v[h,:] = sum_t p[t] * row_t[:512]                (V is the row's first 512)
// Every head reads the same rows (MQA over the compressed cache), so the 128
// heads are the MFMA's free dimension: one workgroup of 4 waves streams a range
// of rows once through LDS and each wave multiplies its 32 heads against it.
//
// Per 32-row tile and wave:
//   S^T[t][h] = K[t][:] . Q^T[:][h]   36 x mfma_f32_32x32x16_bf16 (A = K from LDS,
//                                      B = the wave's 32 q_abs rows: 32 k-blocks in
//                                      VGPRs, the 4 rope k-blocks from LDS)
//   softmax numerators in fp32, one head per lane, exp2 domain, against a
//                                      per-head reference max (restart if exceeded)
//   O^T[c][h] += V^T[c][t] . P^T[t][h] 32 x mfma (A = V^T via LDS transpose
//                                      reads, B = every wave's P through LDS)
// The fp32 accumulator O^T (128 latent columns x 128 heads per wave) lives in
// the 256 AGPRs of each lane; the resident query (128 VGPRs), scores and
// fragments share the 256 VGPRs.  O is only ever touched by MFMAs.
//
// The tile loop is a software pipeline with one barrier per tile: after the
// barrier that publishes tile i and the P of tile i - 1, one stream of MFMAs
// runs the scores of tile i as one unbroken accumulate chain, then the P*V of
// tile i - 1 with tile i's softmax cut into slices between those MFMAs (it
// writes tile i's P into one of two P buffers, by tile parity); the copies of
// tile i + 2 go out into the buffer tile i - 1 has left, the V^T fragments of
// tile i are read as registers free up, and the wave waits for its copies of
// tile i + 1 before the next barrier.  Tiles stream HBM -> LDS with 16-byte
// direct-to-LDS loads, three buffers deep.
// With one wave per SIMD nothing else hides a wave's own issue: an MFMA of 32
// cycles covers about four VALU or LDS instructions issued behind it, more
// stretch it, and P*V MFMAs placed inside the score chain cost more than
// their own issue time.  Hence the chain is kept whole and the softmax is
// spread over the 32 P*V MFMAs, a few instructions after each.
// The LDS tile is 32 rows x 72 sixteen-byte granules with an XOR swizzle of the
// granule index inside each aligned group of 8, chosen so that both the
// row-wise K reads (16 rows, one granule each) and the transpose V reads (4
// rows x 4 granules per 32 lanes) hit 16 distinct 16-byte bank groups.
//
// Split-K (flash decoding): grid = (splits, queries).  With more than one split
// the non-empty (query, split) pairs are packed onto the first workgroups, a
// query's splits on one XCD; each writes the normalised partial O (fp16 with a
// power-of-two exponent per head) and its lse, merged by
// attn_combine_f16_kernel.  A single split writes v_combine and lse directly.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "mla_common.h"

// The tile copies set M0 inside inline asm.  No compiler-generated code in this
// translation unit reads M0 (checked in the generated assembly), so declaring
// it clobbered is only documentation; silence the reserved-register warning.
#pragma clang diagnostic ignored "-Winline-asm"

namespace {

constexpr int kH = 128, kC = 512, kW = 576;
constexpr int kTile = 32;                     // rows per tile
constexpr int kGran = kW / 8;                 // 72 granules of 16 B per row
constexpr int kTileGran = kTile * kGran;      // 2304
constexpr int kThreads = 256;                 // 4 waves x 32 heads
constexpr int kLoads = kTileGran / kThreads;  // 9 granules per thread per tile
constexpr int kBufs = 3;
constexpr int kTileBytes = kTileGran * 16;    // 36864
constexpr int kMaxSplitTiles = 1024;          // 32768 rows per split
constexpr int kMaxPacked = 4096;              // queries a packed plan scans (more: one per grid row)
constexpr int kXcds = 8;                      // MI355X: 8 XCDs, each with its own L2
constexpr int kQLds = 4;                      // k-blocks of the query kept in LDS (the rope part)
constexpr int kQReg = kW / 16 - kQLds;        // k-blocks of the query kept in VGPRs
constexpr int kPRow = 80;                     // bytes per head row of P in LDS (64 + 16 pad)
constexpr int kPBuf = kH * kPRow;             // one P buffer; two alternate by tile parity
constexpr size_t kSmemBytes =
    kBufs * kTileBytes + (kMaxSplitTiles + 12) * 4 + kH * 4 + 2 * kPBuf + kLoads * kThreads * 4 +
    kQLds * kThreads * 16;
constexpr float kRestartLog2 = 32.0f;         // restart when the max grows by > 2^32
constexpr int kMaxRestarts = 16;              // after that, one last pass that does not vote
constexpr float kLn2 = 0.69314718055994530942f;

static_assert(kLoads * kThreads == kTileGran, "tile must split evenly over the threads");

// LDS granule slot of (row r, granule g) inside a tile.
__device__ __forceinline__ int swz(int r, int g) {
  const int j = (r >> 1) & 7;
  const int s = ((j & 1) << 2) | (j >> 1);
  return r * kGran + (g ^ s);
}

__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  MLA_LDS char* tiles = (MLA_LDS char*)smem;
  MLA_LDS int* tile_base = (MLA_LDS int*)(smem + kBufs * kTileBytes);
  MLA_LDS int* votes = tile_base + kMaxSplitTiles;         // [2] restart votes (a byte per wave), by tile parity; [8] the slot
  MLA_LDS float* l_heads = (MLA_LDS float*)(votes + 12);   // [128] softmax denominators
  MLA_LDS char* p_lds = (MLA_LDS char*)(l_heads + kH);     // [2][128 heads][kPRow] bf16 P, slot order
  MLA_LDS uint32_t* goff_lds = (MLA_LDS uint32_t*)(p_lds + 2 * kPBuf);  // [kLoads][256]
  // [4 waves][kQLds][64 lanes] query fragments, in the order the lanes read them
  MLA_LDS bf16x8_t* qpe_lds = (MLA_LDS bf16x8_t*)(goff_lds + kLoads * kThreads);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  int split = blockIdx.x;
  int b = blockIdx.y;
  int rows = a.split_rows;  // rows per split
  int slot = b * a.num_splits + split;  // partial slot of this (query, split)
  int len = -1;                         // this query's rows (the packed plan finds it)
  if (a.num_splits > 1 && a.B > 1 && a.B <= kMaxPacked) {
    // Packed plan: the non-empty (query, split) pairs, query-major, go to the
    // first workgroups in dispatch order, so a ragged batch's work starts at
    // once on every compute unit and the empty workgroups leave (a single
    // query keeps the direct mapping: its splits are all non-empty, or empty
    // at the end only).  Query b has
    // ceil(len_b / rows) non-empty splits; an exclusive scan over the queries
    // finds this workgroup's pair, whose index is also its partial slot.
    const int w = blockIdx.y * gridDim.x + blockIdx.x;
    // [4] wave totals, the pair, block sums: the tile table's area, free
    // until the end of the prologue (the query's copies use the P area)
    MLA_LDS int* scan = tile_base;
    const int nchunks = (a.B + kThreads - 1) / kThreads;  // uniform
    // All lengths read up front (one latency, not one per chunk).  Only the
    // chunks that hold queries are loaded and divided: the loops below leave
    // at the first empty chunk by a uniform branch, since every chunk costs
    // a few divisions per thread and the plan runs before any copy goes out.
    int lens[kMaxPacked / kThreads];
#pragma unroll
    for (int i = 0; i < kMaxPacked / kThreads; ++i) lens[i] = 0;
#pragma unroll
    for (int i = 0; i < kMaxPacked / kThreads; ++i) {
      if (i >= nchunks) break;
      const int q = i * kThreads + tid;
      const int lq = q < a.B ? a.seq_lens[q] : 0;
      lens[i] = lq < a.max_len ? lq : a.max_len;
    }
    auto pairs_of = [&](int r) -> int {  // this thread's non-empty splits at r rows
      int n = 0;
#pragma unroll
      for (int i = 0; i < kMaxPacked / kThreads; ++i) {
        if (i >= nchunks) break;
        n += lens[i] > 0 ? (lens[i] + r - 1) / r : 0;
      }
      return n;
    };
    // block-wide sum; each call k uses its own LDS slots, so no barrier is
    // needed after it
    int nsum = 0;
    auto block_sum = [&](float v0, int v1, float* s0) -> int {
      for (int o = 32; o > 0; o >>= 1) {
        v0 += __shfl_xor(v0, o, 64);
        v1 += __shfl_xor(v1, o, 64);
      }
      MLA_LDS int* r = scan + 16 + 8 * nsum++;
      if (lane == 0) {
        ((MLA_LDS float*)r)[wave] = v0;
        r[4 + wave] = v1;
      }
      __syncthreads();
      const MLA_LDS float* rf = (const MLA_LDS float*)r;
      *s0 = (rf[0] + rf[1]) + (rf[2] + rf[3]);
      return r[4] + r[5] + r[6] + r[7];
    };
    float tot = 0.f;
    if (a.auto_slots > 0) {
#pragma unroll
      for (int i = 0; i < kMaxPacked / kThreads; ++i) {
        if (i >= nchunks) break;
        tot += (float)lens[i];
      }
    }
    // the host plan's number of non-empty splits (and the total rows)
    int total = block_sum(tot, pairs_of(rows), &tot);
    if (a.auto_slots > 0) {
      // Rows per split from the lengths themselves: the smallest multiple of
      // 64 (at least 128) found by a few refinements of total / slots whose
      // non-empty splits fit auto_slots workgroups (about one per compute
      // unit), so a ragged batch is not split for its longest sequence.  If
      // no refinement fits, the host's plan (sized for the longest) stays.
      const int cap = kMaxSplitTiles * kTile;
      auto round64 = [&](float r) -> int {
        const float c = (float)cap;
        r = r < c ? r : c;
        int ri = ((int)ceilf(r) + 63) / 64 * 64;
        ri = ri < 128 ? 128 : ri;
        return ri < cap ? ri : cap;
      };
      int r = round64(tot / (float)a.auto_slots);
      float unused;
      int n = r == rows ? total : block_sum(0.f, pairs_of(r), &unused);
      for (int it = 0; it < 3 && n > a.auto_slots && r < cap; ++it) {
        r = round64((float)r * (float)n / (float)a.auto_slots);
        n = block_sum(0.f, pairs_of(r), &unused);
      }
      if (n <= a.auto_slots) {
        rows = r;
        total = n;
      }
    }
    if (a.auto_slots > 0 && w == 0 && tid == 0) a.part_first[a.B] = rows;  // for the merge
    int cnts[kMaxPacked / kThreads];
#pragma unroll
    for (int i = 0; i < kMaxPacked / kThreads; ++i) cnts[i] = 0;
#pragma unroll
    for (int i = 0; i < kMaxPacked / kThreads; ++i) {
      if (i >= nchunks) break;
      cnts[i] = lens[i] > 0 ? (lens[i] + rows - 1) / rows : 0;
    }
    // Workgroups go to the XCDs round robin (w % 8 on this chip).  The
    // workgroups w < total take the pairs: XCD x's n_x = ceil((total - x) / 8)
    // of them take one contiguous run of pairs, so the splits of a query share
    // an XCD's L2 and its query is read from memory once per XCD, not per split.
    if (w >= total) return;  // no work for this workgroup (uniform)
    int p = w / kXcds;
    for (int x = 0; x < w % kXcds; ++x) p += (total - x + kXcds - 1) / kXcds;
    int carry = 0;
#pragma unroll
    for (int i = 0; i < kMaxPacked / kThreads; ++i) {
      if (i >= nchunks) break;  // uniform
      const int q = i * kThreads + tid;
      const int cnt = cnts[i];
      int x = cnt;  // inclusive scan inside the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        x += lane >= o ? y : 0;
      }
      if (lane == 63) scan[wave] = x;
      __syncthreads();
      int before = carry;
      for (int v = 0; v < wave; ++v) before += scan[v];
      const int excl = before + x - cnt;
      if (p >= excl && p < excl + cnt) {
        scan[4] = q;
        scan[5] = p - excl;
        scan[10] = excl;
        scan[11] = lens[i];
      }
      carry += scan[0] + scan[1] + scan[2] + scan[3];
      __syncthreads();  // the totals are read before the next chunk rewrites them
    }
    b = scan[4];
    split = scan[5];
    len = scan[11];
    // a device plan packs the slots by pair; the host plan keeps b * S + split
    slot = a.auto_slots > 0 ? p : b * a.num_splits + split;
    if (a.auto_slots > 0 && split == 0 && tid == 0) a.part_first[b] = scan[10];
  }
  // uniform across the workgroup (read from LDS above): keep them scalar.  The
  // partial slot is only needed after the tile loop: it waits in LDS.
  b = __builtin_amdgcn_readfirstlane(b);
  split = __builtin_amdgcn_readfirstlane(split);
  rows = __builtin_amdgcn_readfirstlane(rows);
  if (tid == 0) votes[8] = slot;
  const int hf = lane >> 5;          // which half of the wave
  const int l32 = lane & 31;
  const int head = wave * 32 + l32;  // this lane's head in the S^T layout

  if (len < 0) {
    len = a.seq_lens[b];
    len = len < a.max_len ? len : a.max_len;
  }
  len = __builtin_amdgcn_readfirstlane(len);
  const int row_begin = split * rows;
  int row_end = row_begin + rows;
  row_end = row_end < len ? row_end : len;

  // Outputs of this (sequence, split): with one partition v_combine and lse
  // directly, otherwise the fp16 partial [128 heads][512] in its slot, its
  // exponent and lse.
  const size_t bs0 = (size_t)__builtin_amdgcn_readfirstlane(slot);
  float* out_lse = a.num_splits == 1 ? (a.lse ? a.lse + (size_t)b * kH + head : nullptr)
                                     : a.part_lse + bs0 * kH + head;

  if (row_begin >= row_end) {  // nothing to attend in this partition
    if (a.num_splits == 1) {
      float* out_o = a.v_combine + (size_t)b * kH * kC + (size_t)head * kC;
      for (int c = hf * 4; c < kC; c += 8)
        *reinterpret_cast<f32x4_t*>(out_o + c) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else if (hf == 0) {
      a.part_exp[bs0 * kH + head] = 0.f;
    }
    if (out_lse && hf == 0) *out_lse = -INFINITY;
    return;
  }
  const int ntiles = (row_end - row_begin + kTile - 1) / kTile;
  const char* pool = static_cast<const char*>(a.pool);
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)tiles;

  // Byte offset, inside a tile of 32 consecutive rows, of granule copy k of
  // this thread: LDS slot p = (k*4 + wave)*64 + lane holds granule
  // (p % 72) ^ swizzle(row) of row p / 72.  In registers for the first two
  // tiles' copies; in LDS (read by this thread only) for the later ones.
  uint32_t goff[kLoads];
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int p = (k * 4 + wave) * 64 + lane;
    const int r = p / kGran;
    const int x = p - r * kGran;
    const int j = (r >> 1) & 7;
    goff[k] = (uint32_t)(r * (kW * 2) + (x ^ (((j & 1) << 2) | (j >> 1))) * 16);
  }

  // Physical first row of tile i from the block table; -1 marks a bad table
  // entry (or a query whose sequence index is out of range).
  const int sq = __builtin_amdgcn_readfirstlane(a.q_seq ? a.q_seq[b] : b);  // uniform
  const bool seq_ok = sq >= 0 && sq < a.num_seqs;
  const int32_t* trow = a.table + (size_t)(seq_ok ? sq : 0) * a.max_blocks;
  auto tile_blk = [&](int i) -> int { return seq_ok ? trow[(row_begin + i * kTile) / a.block] : -1; };
  auto tile_row = [&](int i, int blk) -> int {
    return blk >= 0 && blk < a.num_blocks ? blk * a.block + ((row_begin + i * kTile) % a.block) : -1;
  };
  // Source of tile i: the address of its first row (a bad table entry reads
  // row 0 and makes the output NaN).  A tile never crosses a block, so all its
  // 32 rows lie inside the pool even where the split ends first.
  auto base_src = [&](int raw) -> const char* {
    const int base = __builtin_amdgcn_readfirstlane(raw);
    return pool + (size_t)(base < 0 ? 0 : base) * (kW * 2);
  };
  // Copy k of this wave into a 36 KB LDS area: 16 bytes per lane straight
  // into the area's 1 KB slot k*4 + wave, at M0 + 16 * lane.  Issued from asm
  // so that the compiler does not treat every later LDS read as aliasing the
  // copy; the explicit vmcnt waits order them.
  auto copy_to = [&](uint32_t area, int k, uint32_t off, const char* src) {
    const uint32_t lds = area + (uint32_t)((k * 4 + wave) * 1024);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(src), "s"(lds)
                 : "memory");
  };
  // A tile's copy k.  The cache rows are read once per call, so their copies
  // carry the non-temporal hint: the stream does not displace from the caches
  // what is read again (the query, the split partials the merge reads back,
  // the next kernels' inputs).  32 x 16384: 165.7 -> 160.9 us.
  auto issue_load = [&](int i, int k, uint32_t off, const char* src) {
    const uint32_t lds =
        tiles_lds + (uint32_t)((i % kBufs) * kTileBytes) + (uint32_t)((k * 4 + wave) * 1024);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(src), "s"(lds)
                 : "memory");
  };
  auto issue_tile_from = [&](int i, const char* src) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) issue_load(i, k, goff_lds[k * kThreads + tid], src);
  };
  // Table entries of tiles 0 and 1 as scalar loads: they are waited for with
  // lgkmcnt, so their wait does not also wait for the query's copies issued
  // after them (vector loads complete in order).
  // No branch around them (a branch would make the compiler wait at its
  // end): a load that is not needed reads a valid word instead (tile 0's
  // entry for a missing tile 1, a length for a query without a sequence).
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  const int32_t* e0 = seq_ok ? trow + row_begin / a.block : a.seq_lens;
  const int32_t* e1 = seq_ok && ntiles > 1 ? trow + (row_begin + kTile) / a.block : e0;
  const int blk0_raw = *(const_i32p)e0, blk1_raw = *(const_i32p)e1;
  // this thread's share of every tile's entry (consumed at the prologue's end)
  int tblk[kMaxSplitTiles / kThreads];
#pragma unroll
  for (int j = 0; j < kMaxSplitTiles / kThreads; ++j) {
    const int i = tid + j * kThreads;
    tblk[j] = i < ntiles ? tile_blk(i) : 0;
  }

  // The wave's 32 query rows as MFMA B operands: lane -> head l32, columns
  // 16*kb + 8*hf .. +7 of the 576.  The first kQReg k-blocks stay in VGPRs;
  // the rope k-blocks go to LDS (the register file holds O, Q and the
  // pipeline's fragments, and no more).  Loaded straight into that layout, a
  // load instruction would touch 32 rows, 32 bytes from each, and the wave's
  // 36 of them take thousands of cycles to issue; instead the rows (36 KB per
  // wave, contiguous) come through LDS in four rounds of 9 k-blocks: round
  // r's copies (9 per lane, each 1 KB of 3-4 rows) put head h's bytes
  // 288 r .. +287 at granule 18 h + g of the wave's slots (granule
  // G = 64 k + lane of copy k), and each lane reads its 9 fragments back
  // (two-way bank conflicts at most).  Rounds go through tile buffer 2 and
  // the 36 KB from the P buffers on (P, copy offsets, rope query: written
  // only after the barrier below), so tiles 0 and 1 take buffers 0 and 1 at
  // once: their copies go out as soon as their table entries are in, and the
  // query's rounds arrive meanwhile.  Each wave reads only its own slots.
  const uint32_t qarea[2] = {tiles_lds + 2u * kTileBytes, (uint32_t)(uintptr_t)p_lds};
  static_assert(2 * kPBuf + kLoads * kThreads * 4 + kQLds * kThreads * 16 >= kTileBytes,
                "the P, offset and rope-query areas hold one round of the query");
  const char* qrow = static_cast<const char*>(a.q_abs) + ((size_t)b * kH + wave * 32) * (kW * 2);
  uint32_t qoff[9], qrd[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const int G = 64 * k + lane;
    qoff[k] = (uint32_t)((G / 18) * (kW * 2) + (G % 18) * 16);
    const int R = 18 * l32 + 2 * k + hf;  // this lane's fragment k of a round
    qrd[k] = (uint32_t)((((R >> 6) * 4 + wave) * 1024) + (R & 63) * 16);
  }
  auto q_round = [&](int r, int area) {
#pragma unroll
    for (int k = 0; k < 9; ++k) copy_to(qarea[area], k, qoff[k], qrow + 288 * r);
  };
  auto q_read = [&](int area, int k) {
    return *(const MLA_LDS bf16x8_t*)(uintptr_t)(qarea[area] + qrd[k]);
  };
  q_round(0, 0);
  q_round(1, 1);
  // the table entries are used (and waited for) only once the rounds are out
  __builtin_amdgcn_sched_barrier(0);
  const char* src0 = base_src(tile_row(0, seq_ok ? blk0_raw : -1));
  const char* src1 = ntiles > 1 ? base_src(tile_row(1, seq_ok ? blk1_raw : -1)) : pool;
#pragma unroll
  for (int k = 0; k < kLoads; ++k) issue_load(0, k, goff[k], src0);
#pragma unroll
  for (int k = 0; k < kLoads; ++k) issue_load(1, k, goff[k], src1);
  asm volatile("s_waitcnt vmcnt(18)" ::: "memory");  // rounds 0 and 1, the table entries (older)
  bf16x8_t qf[kQReg];
  bf16x8_t qpe[kQLds];
#pragma unroll
  for (int k = 0; k < 9; ++k) qf[k] = q_read(0, k);
#pragma unroll
  for (int k = 0; k < 9; ++k) qf[9 + k] = q_read(1, k);
  // this wave's reads of its slots are done before its next copies land there
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  q_round(2, 0);
  q_round(3, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // rounds 2 and 3 (and tiles 0 and 1)
#pragma unroll
  for (int k = 0; k < 9; ++k) qf[18 + k] = q_read(0, k);
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const bf16x8_t v = q_read(1, k);
    if (27 + k < kQReg) qf[27 + k < kQReg ? 27 + k : 0] = v;
    else qpe[27 + k - kQReg < kQLds ? 27 + k - kQReg : 0] = v;
  }
  static_assert(kQReg == 32 && kQLds == 4, "four rounds of 9 k-blocks cover the 576 columns");
  // every wave has read its query (and, in a packed plan, the scan in the
  // tile table's area) before the areas below are written
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kLoads; ++k) goff_lds[k * kThreads + tid] = goff[k];

  // The first row of every tile of this split, for the later copies.
  int bad_tile = 0;
#pragma unroll
  for (int j = 0; j < kMaxSplitTiles / kThreads; ++j) {
    const int i = tid + j * kThreads;
    if (i < ntiles) {
      const int r = tile_row(i, tblk[j]);
      tile_base[i] = r;
      bad_tile |= r < 0;
    }
  }
#pragma unroll
  for (int j = 0; j < kQLds; ++j) qpe_lds[(wave * kQLds + j) * 64 + lane] = qpe[j];
  // any bad table entry in the split makes its outputs NaN
  const bool bad = __syncthreads_or(bad_tile) != 0;

  // Loop-invariant parts of the LDS read addresses (bytes inside a tile); the
  // others follow by XOR (the swizzle touches granule bits 1..2 only):
  //   K rows for k-block kb:   qk0 ^ ((kb & 3) << 5), + (kb >> 2) * 128
  //   V^T for column block cb: ((pv0 ^ 64*(cb & 1)) ^ 32*rr) + 9216*rr, + (cb >> 1) * 128
  const uint32_t qk0 = (uint32_t)swz(l32, hf) * 16;
  uint32_t pv0;
  {
    const int k16 = lane & 15, g16 = (lane >> 4) & 1;
    pv0 = (uint32_t)(swz(4 * hf + (k16 >> 2), 2 * g16 + ((k16 & 3) >> 1)) * 16 + 8 * (k16 & 1));
  }
  const uint32_t p_row = (uint32_t)(l32 * kPRow + hf * 16);  // + head block * 32 * kPRow

  auto tile_src = [&](int i) -> const char* { return base_src(tile_base[i]); };
  // Tiles past the split's end (the pipeline's look-ahead) re-read the pool's
  // first 32 rows into the buffer they would use.
  auto issue_tile = [&](int i) { issue_tile_from(i, i < ntiles ? tile_src(i) : pool); };
  // Rows of tile i past the split's end hold whatever the pool has there
  // (possibly NaN).  They get probability 0, but 0 * NaN would still reach O
  // through P*V, so once this wave's copies of the tile have landed it
  // overwrites its own granules of those rows with zeros; the barrier that
  // publishes the tile follows.  Once per split at most.
  auto zero_tail = [&](int i) {
    const int t0 = row_begin + i * kTile;
    if (i >= ntiles || t0 + kTile <= row_end) return;
    const int rlast = row_end - 1 - t0;
    MLA_LDS char* buf = tiles + (i % kBufs) * kTileBytes;
    int slot = wave * 64 + lane;
    asm volatile("" : "+v"(slot));  // computed here, not kept live across the tile loop
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      if ((slot + k * 256) / kGran > rlast)
        *(MLA_LDS f32x4_t*)(buf + (slot + k * 256) * 16) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  f32x16_t o[kC / 32];  // cleared by MFMAs at every (re)start
  // p = 2^(s*scale*log2e - m_ref) with a per-head reference m_ref taken from
  // the first tile (0 if that tile has no finite score for the head, so that
  // later exponents stay finite).  If a later tile's maximum exceeds it by
  // more than kRestartLog2 (p would leave the safe range), the workgroup
  // restarts the split with the largest maximum seen as the new reference;
  // each restart raises some head's reference by more than kRestartLog2, and
  // after kMaxRestarts the last pass runs without voting, so the loop always
  // ends.  O is never rescaled: MFMAs of zero operands clear it at every
  // (re)start.
  const float c = a.scale_log2;
  float m_ref = -INFINITY;
  float m_seen = -INFINITY;
  float l_run = 0.f;
  bool fresh = true;  // the next tile is the first since the (re)start
  bool may_vote = true;

  // K fragment of k-block kb: base qa[kb & 3] of the tile, + (kb >> 2) * 128.
  // The bases are made opaque so that the constant offsets fold into the
  // reads instead of becoming 36 hoisted addresses.
  auto kbases = [&](uint32_t t, uint32_t* qa) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qa[m] = t + (qk0 ^ (uint32_t)(m << 5));
      asm volatile("" : "+v"(qa[m]));
    }
  };
  auto kaddr = [&](const uint32_t* qa, int kb) {
    return (const MLA_LDS bf16x8_t*)(uintptr_t)(qa[kb & 3] + (kb >> 2) * 128);
  };
  // V^T fragment for this wave's column block 4*wave + cbl and k-block kb:
  // two transpose reads of 4 rows x 4 columns each.
  auto vread = [&](const uint32_t* va, int cbl, int kb) {
    const uint32_t off = kb * (16 * kGran * 16) + (cbl >> 1) * 128;
    const s16x4_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4_t*)(uintptr_t)(va[(cbl & 1) * 2] + off));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MLA_LDS s16x4_t*)(uintptr_t)(va[(cbl & 1) * 2 + 1] + off));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  const char* src2 = pool;  // source of the tile two ahead of the current phase

  // V^T fragments of the tile whose P*V comes next (column blocks 4*wave ..
  // +3 as (cb >> 1) = 2*wave + (cbl >> 1), cb & 1 = cbl & 1; two k-blocks).
  s16x8_t vf[2][4];

  // One MFMA phase of the pipeline, after the barrier that published tile
  // `it` and the P of tile it - 1:
  //   scores of tile it: S^T = K Q^T, 36 MFMAs in one accumulator chain with
  //     nothing else between its links but their K reads (two ahead), the
  //     copies and the rope-query reads;
  //   P*V of tile it - 1 (kMode > 0): O^T += V^T P^T, 32 MFMAs after the
  //     chain, with the softmax of tile it in slices between them (its VALU
  //     work runs while they execute); head block outer, so one P fragment
  //     serves four MFMAs in a row;
  //   the nine copies of tile it + 2 into the buffer tile it - 1 has left;
  //   the V^T fragments of tile it, each read as soon as the P*V MFMAs of
  //     tile it - 1 are done with its registers.
  // kMode 0: no P*V (the first tile of a (re)start); returns the scores for
  // softmax().  kMode 2: with the P*V and tile it's softmax; when a restart
  // was voted the numerators are formed but no state is updated; `pend` gets
  // softmax()'s result.  kMode 1: the phase after the split's last tile, its
  // P*V alone and the vote it acts on.  The copies always look two tiles
  // ahead, past the split's end too (they re-read the pool's first rows into
  // the free buffer), so every phase but the last issues the same nine.
  auto mfma_phase = [&](auto mode, int it, bool keep, bool& pend, int& vote) -> f32x16_t {
    constexpr int kMode = decltype(mode)::value;
    const uint32_t tile = tiles_lds + (uint32_t)((it % kBufs) * kTileBytes);
    // the copies of tile it + 2 read from src2 (found during the previous
    // phase); tile it + 3's base is read now and turned into the next src2 at
    // the end, so no LDS round trip stands between the barrier and the MFMAs
    const char* nsrc = src2;
    const int raw3 = tile_base[it + 3 < ntiles ? it + 3 : 0];
    // the restart votes of tile it - 1, read now, used in the softmax slices
    // one byte per wave in the word of tile it - 1's parity
    uint32_t vv = 0;
    if (kMode > 0) vv = votes[(it - 1) & 1];
    uint32_t qa[4];
    if constexpr (kMode != 1) kbases(tile, qa);
    uint32_t va[4];
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        va[c1 * 2 + rr] = tile + (((pv0 ^ (uint32_t)(64 * c1)) ^ (uint32_t)(32 * rr)) + 9216u * rr) +
                          (uint32_t)(wave * 256);
    const uint32_t pbuf = p_row + (uint32_t)(((it - 1) & 1) * kPBuf);
    auto pread = [&](int x, int kb) {
      return *(const MLA_LDS bf16x8_t*)(p_lds + pbuf + x * (32 * kPRow) + kb * 32);
    };
    bf16x8_t kf[2];
    if constexpr (kMode != 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[kb] = *kaddr(qa, kb);
    }
    bf16x8_t pf[2];  // P fragments (k-block, head block) in MFMA order, two in flight
    if (kMode > 0) {
      pf[0] = pread(0, 0);
      pf[1] = pread(1, 0);
    }
    // P*V step m of tile it - 1 (m = kb*16 + hb*4 + cbl), then tile it's V^T
    // fragment in the registers the step has finished with
    auto pv_step = [&](int m) {
      const int kb = m >> 4, hb = (m >> 2) & 3, cbl = m & 3, f = (m >> 2) & 1;
      if (kMode > 0) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(o[cbl * 4 + hb])
                     : "v"(vf[kb][cbl]), "v"(pf[f]));
      }
      // the P fragment two steps on replaces the one just finished
      if (kMode > 0 && cbl == 3 && m + 8 < 32) pf[f] = pread(((m >> 2) + 2) & 3, (m + 8) >> 4);
      if (kMode != 1 && hb == 3) vf[kb][cbl] = vread(va, cbl, kb);
    };
    __builtin_amdgcn_sched_barrier(0);
    // The score MFMAs are asm too (an exact-register accumulate chain needs
    // no wait states between its links), which keeps the compiler from moving
    // the resident query between registers around the P*V asm.
    f32x16_t s = f32x16_t{};
    if constexpr (kMode != 1) {
    uint32_t noff = goff_lds[tid];
    bf16x8_t qp[kQLds];  // the LDS-resident query k-blocks, read in the phase's last quarter
    const MLA_LDS bf16x8_t* qsrc = qpe_lds + wave * (kQLds * 64) + lane;
#pragma unroll
    for (int n = 0; n < kW / 16; ++n) {
      const bf16x8_t qn = n < kQReg ? qf[n < kQReg ? n : 0] : qp[n < kQReg ? 0 : n - kQReg];
      if (n == 0)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(kf[0]), "v"(qn));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kf[n % 2]), "v"(qn));
      if (n + 2 < kW / 16) kf[n % 2] = *kaddr(qa, n + 2);
      if (n >= 24 && n < 24 + 2 * kQLds && (n & 1) == 0) qp[(n - 24) >> 1] = qsrc[((n - 24) >> 1) * 64];
      if (kMode == 0 && n < 32) pv_step(n);  // the V^T reads only
      if ((n & 3) == 3) {  // copy n / 4 of tile it + 2; the next copy's offset
        const int k = n >> 2;
        const uint32_t off = noff;
        if (k + 1 < kLoads) noff = goff_lds[(k + 1) * kThreads + tid];
        issue_load(it + 2, k, off, nsrc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    }
    if constexpr (kMode == 0) {
      // VALU reads of an MFMA result wait 18 cycles after a 16-pass MFMA; the
      // compiler does not see into asm, so pad here
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s));
      src2 = it + 3 < ntiles ? base_src(raw3) : pool;
      return s;
    } else {
      // softmax() of tile it in slices between the 32 P*V steps (the
      // reference max is fixed after a (re)start's first tile, so it is read
      // here, never raised); the maxima use v_max3 directly (fmaxf would add a
      // canonicalising max per input, and v_max3 drops a quiet NaN the same way).  u = s * scale * log2e - m_ref is the exponent of
      // every numerator; rows past the split's end get u = -inf (numerator 0,
      // no part in the maximum).  The tile's largest u only feeds the restart
      // vote and the reference of a restart.
      const int lim = row_end - (row_begin + it * kTile);
      const bool tail = lim < kTile;
      float e = 0.f;
      float u[16];
      float p[16];
      bf16x8_t pb[2];
      float q01 = 0.f, q23 = 0.f, q45 = 0.f, q67 = 0.f;
      float mx[5];
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        pv_step(t);
        if constexpr (kMode == 1) {  // no tile of its own: only the vote it acts on
          if (t == 0) vote = __builtin_amdgcn_readfirstlane((int)vv);
          __builtin_amdgcn_sched_barrier(0);
          continue;
        }
        // Each slice is pinned to its step: its inputs pass through an empty
        // asm at the step's start and its results at the step's end, so no
        // pass can gather the slices into one long VALU run between two MFMAs.
        if (t == 1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(s));
        if (t >= 2 && t < 6) {
          asm volatile("" : "+v"(s));
#pragma unroll
          for (int j = 4 * (t - 2); j < 4 * (t - 2) + 4; ++j) {
            u[j] = fmaf(s[j], c, -m_ref);
            asm volatile("" : "+v"(u[j]));
          }
        }
        if (t == 5 && tail) {
          int l = lim - 4 * hf;
          asm volatile("" : "+v"(l));
#pragma unroll
          for (int j = 0; j < 16; ++j) u[j] = (j >> 2) * 8 + (j & 3) < l ? u[j] : -INFINITY;
        }
        if (t == 6) {
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[0]) : "v"(u[0]), "v"(u[1]), "v"(u[2]));
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[1]) : "v"(u[3]), "v"(u[4]), "v"(u[5]));
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[2]) : "v"(u[6]), "v"(u[7]), "v"(u[8]));
        }
        if (t == 7) {
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[3]) : "v"(u[9]), "v"(u[10]), "v"(u[11]));
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[4]) : "v"(u[12]), "v"(u[13]), "v"(u[14]));
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(mx[0]) : "v"(mx[0]), "v"(mx[1]), "v"(u[15]));
        }
        if (t == 8) {
          asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(e) : "v"(mx[2]), "v"(mx[3]), "v"(mx[4]));
          asm volatile("v_max_f32 %0, %1, %2" : "=v"(e) : "v"(e), "v"(mx[0]));
        }
        if (t == 9) {
          float lo, hi;
          wave_halves(e, &lo, &hi);
          asm volatile("v_max_f32 %0, %1, %2" : "=v"(e) : "v"(lo), "v"(hi));
          vote = __builtin_amdgcn_readfirstlane((int)vv);
          keep = keep && vote == 0;
          if (keep) m_seen = fmaxf(m_seen, e + m_ref);
          asm volatile("" : "+v"(m_seen), "+v"(e));
        }
        if (t >= 10 && t < 18) {
#pragma unroll
          for (int j = 2 * (t - 10); j < 2 * (t - 10) + 2; ++j) {
            asm volatile("" : "+v"(u[j]));
            p[j] = __builtin_amdgcn_exp2f(u[j]);
            asm volatile("" : "+v"(p[j]));
          }
        }
        if (t == 18 || t == 19) {
          const int h0 = 8 * (t - 18);
#pragma unroll
          for (int j = h0; j < h0 + 8; ++j) pb[t - 18][j - h0] = (__bf16)p[j];
          asm volatile("" : "+v"(pb[t - 18]));
        }
        if (t == 20) {
          q01 = (p[0] + p[1]) + (p[2] + p[3]);
          q23 = (p[4] + p[5]) + (p[6] + p[7]);
          asm volatile("" : "+v"(q01), "+v"(q23));
        }
        if (t == 21) {
          q45 = (p[8] + p[9]) + (p[10] + p[11]);
          q67 = (p[12] + p[13]) + (p[14] + p[15]);
          asm volatile("" : "+v"(q45), "+v"(q67));
        }
        if (t == 22) {
          if (keep) l_run += (q01 + q23) + (q45 + q67);
          asm volatile("" : "+v"(l_run));
        }
        if (t == 23) {
          MLA_LDS char* prow = p_lds + p_row + (uint32_t)((it & 1) * kPBuf) + wave * (32 * kPRow);
          *(MLA_LDS bf16x8_t*)prow = pb[0];
          *(MLA_LDS bf16x8_t*)(prow + 32) = pb[1];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pend = may_vote && e > kRestartLog2;
      src2 = it + 3 < ntiles ? base_src(raw3) : pool;
      return s;
    }
  };

  // Softmax numerators of tile it (lane = head, 16 rows per lane, the rest in
  // lane ^ 32), written as bf16 into P buffer it & 1 in slot order: head row h
  // holds slot kb*16 + hf*8 + j <-> row 16*kb + 8*(j/4) + 4*hf + j%4, the
  // order both MFMA operands of P*V use.  The denominator sums the fp32
  // numerators (so lse stays exact to fp32, independent of the split plan).
  // Returns whether this lane's maximum left the reference's safe range.
  auto softmax = [&](f32x16_t s, int it) -> bool {
    // row (j >> 2) * 8 + (j & 3) + 4 * hf of the tile is valid iff that is < lim
    const int lim = row_end - (row_begin + it * kTile);
    const bool tail = lim < kTile;
    float u[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) u[j] = s[j] * c;
    if (tail) {  // rows past the end: numerator 0, no part in the maximum
      int l = lim - 4 * hf;
      asm volatile("" : "+v"(l));  // formed here, on the split's last tile only
#pragma unroll
      for (int j = 0; j < 16; ++j) u[j] = (j >> 2) * 8 + (j & 3) < l ? u[j] : -INFINITY;
    }
    float e = fmaxf(fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3])), fmaxf(fmaxf(u[4], u[5]), fmaxf(u[6], u[7])));
    e = fmaxf(e, fmaxf(fmaxf(fmaxf(u[8], u[9]), fmaxf(u[10], u[11])),
                       fmaxf(fmaxf(u[12], u[13]), fmaxf(u[14], u[15]))));
    float lo, hi;
    wave_halves(e, &lo, &hi);
    const float mt = fmaxf(lo, hi);
    m_seen = fmaxf(m_seen, mt);
    if (fresh) {
      m_ref = fmaxf(m_ref, mt);
      if (m_ref == -INFINITY) m_ref = 0.f;  // no finite score yet (fmaxf drops NaN)
    }
    fresh = false;
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(u[j] - m_ref);
    bf16x8_t pb[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) pb[j >> 3][j & 7] = (__bf16)p[j];
    float q0 = (p[0] + p[1]) + (p[2] + p[3]), q1 = (p[4] + p[5]) + (p[6] + p[7]);
    float q2 = (p[8] + p[9]) + (p[10] + p[11]), q3 = (p[12] + p[13]) + (p[14] + p[15]);
    l_run += (q0 + q1) + (q2 + q3);
    MLA_LDS char* prow = p_lds + p_row + (uint32_t)((it & 1) * kPBuf) + wave * (32 * kPRow);
    *(MLA_LDS bf16x8_t*)prow = pb[0];
    *(MLA_LDS bf16x8_t*)(prow + 32) = pb[1];
    return may_vote && mt > m_ref + kRestartLog2;
  };

  // The pipeline, per (re)start: tiles 0 and 1 are copied, then phase it
  // (it = 0 .. ntiles) runs the MFMAs of tile it's scores and tile it - 1's
  // P*V, with tile it's softmax inside its tail (after it for tile 0, whose
  // phase has no P*V).  One barrier per tile publishes its
  // P, its restart vote and tile it + 1 (whose copies this wave waits for
  // just before it: the nine newer copies are tile it + 2's).  Buffers: tile
  // it + 2 goes into the buffer of tile it - 1, whose K and V^T reads all
  // ended before that barrier; P alternates between two buffers, so the
  // barrier of tile it also separates the P*V reads of tile it - 1 from the
  // writes of tile it + 1.  A restart vote is read after the barrier and
  // acted on after the next MFMA phase (its P*V is then discarded).
  const bf16x8_t zf = bf16x8_t{};
  int restarts = 0;
  for (;;) {
    // O = 0 at every (re)start: 0 x 0 + 0 for each 32 x 32 block
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %2, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %3, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %4, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %5, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %6, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %7, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %8, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %9, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %10, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %11, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %12, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %13, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %14, %16, %16, 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %15, %16, %16, 0"
        : "=a"(o[0]), "=a"(o[1]), "=a"(o[2]), "=a"(o[3]), "=a"(o[4]), "=a"(o[5]),
          "=a"(o[6]), "=a"(o[7]), "=a"(o[8]), "=a"(o[9]), "=a"(o[10]), "=a"(o[11]),
          "=a"(o[12]), "=a"(o[13]), "=a"(o[14]), "=a"(o[15])
        : "v"(zf));
    if (restarts > 0) {  // the first pass's copies went out in the prologue
      issue_tile(0);
      issue_tile(1);
    }
    src2 = 2 < ntiles ? tile_src(2) : pool;
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // tile 0 (tile 1's copies are newer)
    zero_tail(0);
    __syncthreads();
    bool pending = false;
    int vote = 0;
    f32x16_t s = mfma_phase(std::integral_constant<int, 0>{}, 0, true, pending, vote);
    pending = softmax(s, 0);
    bool restart = false;
    // the restart vote of tile it - 1 (a byte per wave, by parity; the ballot
    // runs in every lane: inside the branch it would see lane 0 only)
    auto publish_vote = [&](int it) {
      const bool wave_vote = __ballot(pending) != 0;
      if (lane == 0) ((MLA_LDS uint8_t*)(votes + ((it - 1) & 1)))[wave] = wave_vote ? 1 : 0;
    };
    for (int it = 1; it < ntiles; ++it) {
      publish_vote(it);
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // this wave's copies of tile it
      zero_tail(it);
      __syncthreads();
      mfma_phase(std::integral_constant<int, 2>{}, it, true, pending, vote);
      if (vote != 0) {
        restart = true;
        break;
      }
    }
    if (!restart) {  // past the last tile: its P*V alone (no copy of this tile is read)
      publish_vote(ntiles);
      __syncthreads();
      mfma_phase(std::integral_constant<int, 1>{}, ntiles, false, pending, vote);
      restart = vote != 0;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!restart) break;
    __syncthreads();  // every wave's copies have landed before the buffers are reused
    m_ref = m_seen;
    if (++restarts >= kMaxRestarts) may_vote = false;
    l_run = 0.f;
    fresh = true;
  }

  // The last accumulate MFMAs may still be in flight: pad before reading O.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
                 "+a"(o[6]), "+a"(o[7]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]),
                 "+a"(o[14]), "+a"(o[15]));

  // ---- finish: this wave's 128 columns of every head, normalised by the
  // head's denominator (owned by the lanes that computed its scores) ----
  // The lane's coordinates again, from its position in the wave, so that
  // nothing derived from the thread index stays live across the tile loop
  // (which holds every register; a value kept across it is spilled, and a
  // reload here would wait for every store in flight).
  {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int hf = lane >> 5, l32 = lane & 31, head = wave * 32 + l32;
  float l_lo, l_hi;
  wave_halves(l_run, &l_lo, &l_hi);
  const float l = l_lo + l_hi;
  if (hf == 0) l_heads[head] = l;
  {  // the head's lse, before the outputs (nothing of it stays live past here)
    float* out_lse = a.num_splits == 1 ? (a.lse ? a.lse + (size_t)b * kH + head : nullptr)
                                       : a.part_lse + bs0 * kH + head;
    if (out_lse && hf == 0) *out_lse = bad ? NAN : (m_ref + log2f(l)) * kLn2;
  }
  __syncthreads();
  const size_t bs = (size_t)__builtin_amdgcn_readfirstlane(votes[8]);  // the partial slot
  // The outputs leave through LDS, one head block at a time: each wave
  // transposes its 128 columns of 32 heads in its own part of the tile
  // buffers (free since the barrier above; LDS operations of one wave run in
  // order, so the area is reused from block to block without a barrier), so
  // that every store instruction writes whole 128-byte lines of one head's
  // consecutive columns.  Straight from the accumulator layout a store would
  // put 16 or 32 bytes into each of 32 rows, and a lone workgroup's stores
  // would then take longer than several of its tiles.  16-byte chunks are
  // XOR-swizzled by head, so neither side has more bank conflicts than its
  // width requires.
  MLA_LDS char* stage = tiles + wave * 16384;
  if (a.num_splits == 1) {
    // fp32 v_combine: head r's 128 columns are 32 chunks of 4 floats (chunk c
    // at slot c ^ r); read back as 2 heads x 512 bytes per instruction
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float inv_l = bad ? NAN : 1.0f / l_heads[hb * 32 + l32];
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int chunk = cbl * 8 + q4 * 2 + hf;  // columns 4 * chunk .. + 3
          const f32x16_t& ob = o[cbl * 4 + hb];
          f32x4_t v{ob[4 * q4 + 0] * inv_l, ob[4 * q4 + 1] * inv_l, ob[4 * q4 + 2] * inv_l,
                    ob[4 * q4 + 3] * inv_l};
          *(MLA_LDS f32x4_t*)(stage + l32 * 512 + ((chunk ^ l32) << 4)) = v;
        }
      }
      float* dst = a.v_combine + ((size_t)b * kH + hb * 32) * kC + wave * 128 + l32 * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 2 * i + hf;
        const f32x4_t v = *(const MLA_LDS f32x4_t*)(stage + r * 512 + ((l32 ^ r) << 4));
        *reinterpret_cast<f32x4_t*>(dst + (size_t)r * kC) = v;
      }
    }
  } else {
    // fp16 partial: O / l * 2^-e with e the exponent that brings the head's
    // largest magnitude into [2^14, 2^15) (f16_range_exp), so that neither a
    // huge |V| overflows binary16 nor a tiny one falls into its subnormals;
    // the largest |O| / l of each head over the four waves meets in LDS (the
    // P area, free after the barrier above).
    MLA_LDS float* amax_lds = (MLA_LDS float*)p_lds;  // [4 waves][128 heads]
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      float mx = 0.f;
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(o[cbl * 4 + hb][j]));
      float m_lo, m_hi;
      wave_halves(mx, &m_lo, &m_hi);
      mx = fmaxf(m_lo, m_hi);
      if (hf == 0) amax_lds[wave * kH + hb * 32 + l32] = mx / l_heads[hb * 32 + l32];
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int h = hb * 32 + l32;
      const float amax = fmaxf(fmaxf(amax_lds[h], amax_lds[kH + h]),
                               fmaxf(amax_lds[2 * kH + h], amax_lds[3 * kH + h]));
      const int e = f16_range_exp(amax);
      const float scale = pow2f(-e);
      const float inv_l = bad ? NAN : scale / l_heads[h];
      // head r's 128 columns are 16 chunks of 8 halves (chunk c at slot
      // c ^ (r & 15)), each written as two 4-half pieces by the lane pair
      // hf = 0, 1 (in swapped order for r >= 16, so that rows r and r + 16
      // fall in different banks); read back as 4 heads x 256 bytes per
      // instruction
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int chunk = cbl * 4 + q4;  // columns 8 * chunk .. + 7
          const f32x16_t& ob = o[cbl * 4 + hb];
          typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
          const f16x4_t v{(_Float16)(ob[4 * q4 + 0] * inv_l), (_Float16)(ob[4 * q4 + 1] * inv_l),
                          (_Float16)(ob[4 * q4 + 2] * inv_l), (_Float16)(ob[4 * q4 + 3] * inv_l)};
          *(MLA_LDS f16x4_t*)(stage + l32 * 256 + ((chunk ^ (l32 & 15)) << 4) +
                              ((hf ^ (l32 >> 4)) << 3)) = v;
        }
      }
      if (wave == 0 && hf == 0) a.part_exp[bs * kH + h] = (float)e;
      _Float16* dst = a.part_oh + (bs * kH + hb * 32) * kC + wave * 128 + (lane & 15) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4);
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        u32x4_t v = *(const MLA_LDS u32x4_t*)(stage + r * 256 + (((lane & 15) ^ (r & 15)) << 4));
        if (i >= 4) v = __builtin_shufflevector(v, v, 2, 3, 0, 1);  // rows 16..31: halves swapped
        *reinterpret_cast<u32x4_t*>(dst + (size_t)r * kC) = v;
      }
    }
  }
  }
}

// Merge the normalised partials of every split: lse = log sum_s exp(lse_s),
// v = sum_s exp(lse_s - lse) O_s.  This one takes the generic kernel's fp32
// partials (any H and C): one workgroup per (sequence, 2 heads), 128 threads
// per head, 4 consecutive latent columns per thread and step; the max and the
// weight sum over splits are wavefront reductions.  C % 4 == 0.
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
  const int b = blockIdx.y;
  const int h = blockIdx.x * 2 + (threadIdx.x >> 7);
  const int c0 = (threadIdx.x & 127) * 4;
  const int lane = threadIdx.x & 63;
  const int S = a.num_splits;
  if (h >= a.H) return;  // odd head counts: the second half-block is idle (whole waves)
  const float* lse_s = a.part_lse + (size_t)b * S * a.H + h;  // stride H over s

  // A split that read a bad table entry has lse NaN, which fmaxf would drop:
  // it makes the whole merge NaN instead.
  float m = -INFINITY;
  bool nan_lse = false;
  for (int s = lane; s < S; s += 64) {
    const float l = lse_s[(size_t)s * a.H];
    m = fmaxf(m, l);
    nan_lse |= l != l;
  }
  m = wave_max(m);
  if (__ballot(nan_lse) != 0) m = NAN;
  float* dst = a.v_combine + ((size_t)b * a.H + h) * a.C;
  if (m == -INFINITY) {  // empty sequence
    for (int c = c0; c < a.C; c += 512) *reinterpret_cast<f32x4_t*>(dst + c) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (a.lse && (threadIdx.x & 127) == 0) a.lse[(size_t)b * a.H + h] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < S; s += 64) wsum += expf(lse_s[(size_t)s * a.H] - m);
  wsum = wave_sum(wsum);
  const float inv = 1.0f / wsum;
  for (int c = c0; c < a.C; c += 512) {
    f32x4_t acc{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float ls = lse_s[(size_t)s * a.H];
      if (ls == -INFINITY) continue;
      const size_t off = (((size_t)b * S + s) * a.H + h) * a.C + c;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.part_o + off);
      acc += expf(ls - m) * v;
    }
    *reinterpret_cast<f32x4_t*>(dst + c) = acc * inv;
  }
  if (a.lse && (threadIdx.x & 127) == 0) a.lse[(size_t)b * a.H + h] = m + logf(wsum);
}

// The same merge for the MFMA kernel's partials (H = 128, C = 512), stored as
// fp16 times 2^-e_s: O_s = 2^e_s * (stored value), and 2^e_s folds into the
// split's weight.  A wave covers one (sequence, head), 8 consecutive latent
// columns per lane, so every split's partial row is one 1 KB coalesced read;
// the rows go eight at a time, one memory round trip per batch of 8 splits.
// A query with more than 8 splits gets W = 2 or 4 waves per head (W from its
// own number of splits, so a query's result does not depend on the rest of
// the batch): wave w takes batches w, w + W, ..., and the W sums meet in LDS
// and are added in wave order.  With up to 8 splits the workgroup's four
// waves take four heads.  The grid holds 32 * W workgroups per query for the
// W of the host's plan; a query with more waves per head than that (a device
// plan with shorter splits) takes its heads in several rounds.  Lane s % 64
// forms split s's weight.
__global__ void __launch_bounds__(256) attn_combine_f16_kernel(AttnArgs a) {
  __shared__ f32x4_t wsums[4][2][64];  // each wave's batch sums (columns 0-3, 4-7 of a lane)
  const int b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Query b's ceil(len / rows) partials sit in consecutive slots from
  // part_first[b] (rows, chosen by the split kernel, in part_first[B]); no
  // workgroup wrote the slots of empty splits, so they are not read.
  int len = a.seq_lens[b];
  len = len < a.max_len ? len : a.max_len;
  // (with the host's plan: split_rows, and slot b * num_splits + split)
  int rows = a.split_rows, first_raw = b * a.num_splits;
  if (a.auto_slots > 0) {
    rows = a.part_first[a.B];
    first_raw = a.part_first[b];  // both loads in flight together
  }
  const int S = __builtin_amdgcn_readfirstlane(len > 0 ? (len + rows - 1) / rows : 0);
  const int nb = (S + 7) / 8;                         // batches of 8 splits
  const int W = nb <= 1 ? 1 : (nb == 2 ? 2 : 4);      // waves per head (uniform)
  const size_t first = S > 0 ? (size_t)first_raw : 0;
  // rounds of 4 (head, wave) tasks: the W waves of a head share a workgroup
  for (int xb = blockIdx.x; xb < kH * W / 4; xb += gridDim.x) {
    const int h = __builtin_amdgcn_readfirstlane((xb * 4 + wave) / W);
    const int w = wave % W;
    const float* lse_s = a.part_lse + first * kH + h;  // stride kH over s
    const float* exp_s = a.part_exp + first * kH + h;
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    const _Float16* src = a.part_oh + (first * kH + h) * kC + lane * 8;
    const size_t sstride = (size_t)kH * kC;

    // One memory round trip for everything that needs only the slot range: this
    // wave's first eight partial rows (batch w; the last row repeated past the
    // end; slot 0 for an empty query, never used) and this lane's split lse and
    // exponent.
    f16x8_t v0[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = 8 * w + j;
      const int sj = s < S ? s : (S > 0 ? S - 1 : 0);  // uniform
      v0[j] = *reinterpret_cast<const f16x8_t*>(src + (size_t)sj * sstride);
    }
    const float ls0 = lane < S ? lse_s[(size_t)lane * kH] : -INFINITY;
    const float ex0 = lane < S ? exp_s[(size_t)lane * kH] : 0.f;

    float m = ls0;
    bool nan_lse = ls0 != ls0;  // a bad table entry: NaN through the merge, as above
    for (int s = 64 + lane; s < S; s += 64) {
      const float l = lse_s[(size_t)s * kH];
      m = fmaxf(m, l);
      nan_lse |= l != l;
    }
    m = wave_max(m);
    if (__ballot(nan_lse) != 0) m = NAN;
    const bool empty = m == -INFINITY;  // an empty sequence (the same for every head of it)
    float wsum = empty ? 1.f : expf(ls0 - m);  // 0 for lanes past the splits (ls0 = -inf)
    if (!empty)
      for (int s = 64 + lane; s < S; s += 64) wsum += expf(lse_s[(size_t)s * kH] - m);
    wsum = wave_sum(wsum);
    const float inv = 1.0f / wsum;

    f32x4_t lo{0.f, 0.f, 0.f, 0.f}, hi{0.f, 0.f, 0.f, 0.f};
    int chunk = -1;  // the 64 splits whose weights the lanes hold
    float wl = 0.f;
    // batch jb of this wave (eight rows v of splits 8 jb ...): the lane's
    // weight for the batch's 64-split chunk, then the rows added in order;
    // a split past the end re-read the last row and an empty split's
    // unwritten row is read too, and both are dropped by a select (not
    // multiplied by 0, which keeps NaN)
    auto add_batch = [&](int jb, const f16x8_t (&v)[8]) {
      const int s0 = 8 * jb;
      if (s0 / 64 != chunk) {
        // this lane's split 64 * chunk + lane: its weight, 0 for an empty split
        chunk = s0 / 64;
        const int sl = 64 * chunk + lane;
        wl = 0.f;
        if (sl < S) {
          const float ls = chunk == 0 ? ls0 : lse_s[(size_t)sl * kH];
          const float ex = chunk == 0 ? ex0 : exp_s[(size_t)sl * kH];
          if (ls != -INFINITY) wl = ldexpf(expf(ls - m), (int)ex);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sj = s0 + j;  // uniform
        const float wj =
            sj < S ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), sj & 63)) : 0.f;
        const f32x4_t l4 = lo + wj * f32x4_t{(float)v[j][0], (float)v[j][1], (float)v[j][2], (float)v[j][3]};
        const f32x4_t h4 = hi + wj * f32x4_t{(float)v[j][4], (float)v[j][5], (float)v[j][6], (float)v[j][7]};
        const bool use = wj != 0.f;
        lo = use ? l4 : lo;
        hi = use ? h4 : hi;
      }
    };
    // the first batch came with the lse; the later ones, eight loads in
    // flight each, no branches
    if (!empty && w < nb) add_batch(w, v0);
    for (int jb = w + W; jb < nb && !empty; jb += W) {
      f16x8_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int sj = 8 * jb + j < S ? 8 * jb + j : S - 1;  // uniform
        v[j] = *reinterpret_cast<const f16x8_t*>(src + (size_t)sj * sstride);
      }
      add_batch(jb, v);
    }
    if (W > 1) {  // the head's W sums, added in wave order by its first wave
      wsums[wave][0][lane] = lo;
      wsums[wave][1][lane] = hi;
      __syncthreads();
      if (w == 0) {
        lo = wsums[wave][0][lane];
        hi = wsums[wave][1][lane];
        for (int q = 1; q < W; ++q) {
          lo = lo + wsums[wave + q][0][lane];
          hi = hi + wsums[wave + q][1][lane];
        }
      }
      __syncthreads();  // read before the next round writes them
      if (w != 0) continue;
    }
    float* dst = a.v_combine + ((size_t)b * kH + h) * kC + lane * 8;
    // the packed fp16 copy: this lane's 8 columns are one 16-byte chunk, in
    // the pair order c0 c4 c1 c5 c2 c6 c3 c7
    auto put_packed = [&](f32x4_t lo4, f32x4_t hi4) {
      if (!a.vc_pk) return;
      const f16x8_t hv = {(_Float16)lo4[0], (_Float16)hi4[0], (_Float16)lo4[1], (_Float16)hi4[1],
                          (_Float16)lo4[2], (_Float16)hi4[2], (_Float16)lo4[3], (_Float16)hi4[3]};
      *reinterpret_cast<f16x8_t*>(a.vc_pk + packed_index(h, b, lane * 8, a.B, kC)) = hv;
    };
    if (empty) {  // empty sequence
      *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      put_packed(f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f});
      if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = -INFINITY;
      continue;
    }
    lo = lo * inv;
    hi = hi * inv;
    *reinterpret_cast<f32x4_t*>(dst) = lo;
    *reinterpret_cast<f32x4_t*>(dst + 4) = hi;
    put_packed(lo, hi);
    if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = m + logf(wsum);
  }
}

}  // namespace

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, hipStream_t s) {
  const size_t smem = kSmemBytes;
  // The dynamic LDS limit is raised once per device (the launch may come from
  // any host thread and any current device).
  static std::mutex mu;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> g(mu);
    if (!attr_set[dev]) {
      e = hipFuncSetAttribute((const void*)attn_mfma_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL(attn_mfma_kernel, dim3(a.num_splits, a.B), dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s) {
  if (a.part_oh) {
    // 32 * W workgroups per query for the waves per head of the host plan's
    // splits (a query with more splits takes its heads in rounds)
    const int nb = (a.num_splits + 7) / 8, W = nb <= 1 ? 1 : (nb == 2 ? 2 : 4);
    hipLaunchKernelGGL(attn_combine_f16_kernel, dim3(kH / 4 * W, a.B), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_combine_kernel, dim3((a.H + 1) / 2, a.B), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

int attn_mfma_max_split_rows() { return kMaxSplitTiles * kTile; }
