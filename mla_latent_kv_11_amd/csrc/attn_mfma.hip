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
//                                      B = the wave's 32 q_abs rows kept in VGPRs)
//   softmax numerators in fp32, one head per lane, exp2 domain, against a
//                                      per-head reference max (restart if exceeded)
//   O^T[c][h] += V^T[c][t] . P^T[t][h] 32 x mfma (A = V^T via LDS transpose
//                                      reads, B = P^T straight from the S^T registers)
// The fp32 accumulator O^T (32 heads x 512) lives in the 256 AGPRs of each
// lane (one head per lane); the resident Q (144 VGPRs), scores and fragments
// share the 256 VGPRs.  O is only ever touched by MFMAs inside the loop.
//
// Tiles stream HBM -> LDS with 16-byte direct-to-LDS loads, three buffers deep;
// a wave waits for its copies of tile i + 1 just before the barrier that
// publishes tile i's P, so the next tile's first K fragments are read during
// tile i's P*V.
// The LDS tile is 32 rows x 72 sixteen-byte granules with an XOR swizzle of the
// granule index inside each aligned group of 8, chosen so that both the
// row-wise K reads (16 rows, one granule each) and the transpose V reads (4
// rows x 4 granules per 32 lanes) hit 16 distinct 16-byte bank groups.
//
// Split-K (flash decoding): grid = (splits, batch). A split with a single
// partition writes v_combine/lse directly; otherwise it writes the normalised
// partial O (fp16 with a power-of-two exponent per head) and its lse, merged
// by attn_combine_f16_kernel.
#include <math.h>

#include <mutex>

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
constexpr int kMaxSplitTiles = 4096;          // 131072 rows per split
constexpr int kPRow = 80;                     // bytes per head row of P in LDS (64 + 16 pad)
constexpr size_t kSmemBytes =
    kBufs * kTileBytes + (kMaxSplitTiles + 8) * 4 + kH * 4 + kH * kPRow + kLoads * kThreads * 4;
constexpr float kRestartLog2 = 32.0f;         // restart when the max grows by > 2^32
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
  MLA_LDS int* votes = tile_base + kMaxSplitTiles;         // [2][4] restart votes, by tile parity
  MLA_LDS float* l_heads = (MLA_LDS float*)(votes + 8);    // [128] softmax denominators
  MLA_LDS char* p_lds = (MLA_LDS char*)(l_heads + kH);     // [128 heads][kPRow] bf16 P, slot order
  MLA_LDS uint32_t* goff_lds = (MLA_LDS uint32_t*)(p_lds + kH * kPRow);  // [kLoads][256]

  const int split = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hf = lane >> 5;          // which half of the wave
  const int l32 = lane & 31;
  const int head = wave * 32 + l32;  // this lane's head in the S^T layout

  int len = a.seq_lens[b];
  len = len < a.max_len ? len : a.max_len;
  const int row_begin = split * a.split_rows;
  int row_end = row_begin + a.split_rows;
  row_end = row_end < len ? row_end : len;

  // Outputs of this (sequence, split): with one partition v_combine and lse
  // directly, otherwise the fp16 partial [128 heads][512], its exponent and lse.
  const size_t bs = (size_t)b * a.num_splits + split;
  float* out_lse = a.num_splits == 1 ? (a.lse ? a.lse + (size_t)b * kH + head : nullptr)
                                     : a.part_lse + bs * kH + head;

  if (row_begin >= row_end) {  // nothing to attend in this partition
    if (a.num_splits == 1) {
      float* out_o = a.v_combine + (size_t)b * kH * kC + (size_t)head * kC;
      for (int c = hf * 4; c < kC; c += 8)
        *reinterpret_cast<f32x4_t*>(out_o + c) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else if (hf == 0) {
      a.part_exp[bs * kH + head] = 0.f;
    }
    if (out_lse && hf == 0) *out_lse = -INFINITY;
    return;
  }
  const int ntiles = (row_end - row_begin + kTile - 1) / kTile;

  // Physical first row of every tile of this split; -1 marks a bad table entry
  // (or a query whose sequence index is out of range).
  const int sq = a.q_seq ? a.q_seq[b] : b;
  const bool seq_ok = sq >= 0 && sq < a.num_seqs;
  const int32_t* trow = a.table + (size_t)(seq_ok ? sq : 0) * a.max_blocks;
  for (int i = tid; i < ntiles; i += kThreads) {
    const int t0 = row_begin + i * kTile;
    const int blk = seq_ok ? trow[t0 / a.block] : -1;
    tile_base[i] = (blk >= 0 && blk < a.num_blocks) ? blk * a.block + (t0 % a.block) : -1;
  }
  // Byte offset, inside a tile of 32 consecutive rows, of granule copy k of
  // this thread: LDS slot p = (k*4 + wave)*64 + lane holds granule
  // (p % 72) ^ swizzle(row) of row p / 72.
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int p = (k * 4 + wave) * 64 + lane;
    const int r = p / kGran;
    const int x = p - r * kGran;
    const int j = (r >> 1) & 7;
    goff_lds[k * kThreads + tid] = (uint32_t)(r * (kW * 2) + (x ^ (((j & 1) << 2) | (j >> 1))) * 16);
  }

  // The wave's 32 query rows as MFMA B operands: lane -> head l32, columns
  // 16*kb + 8*hf .. +7 of the 576.
  bf16x8_t qf[kW / 16];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q_abs) + ((size_t)b * kH + head) * kW + 8 * hf;
#pragma unroll
    for (int kb = 0; kb < kW / 16; ++kb)
      qf[kb] = *reinterpret_cast<const bf16x8_t*>(q + 16 * kb);
  }
  // Consume the Q loads here, so that the only vector-memory operations in
  // flight inside the tile loop are the tile copies counted by hand below.
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
               "v"(qf[6]), "v"(qf[7]), "v"(qf[8]), "v"(qf[9]), "v"(qf[10]), "v"(qf[11]),
               "v"(qf[12]), "v"(qf[13]), "v"(qf[14]), "v"(qf[15]), "v"(qf[16]), "v"(qf[17]));
  asm volatile("" ::"v"(qf[18]), "v"(qf[19]), "v"(qf[20]), "v"(qf[21]), "v"(qf[22]),
               "v"(qf[23]), "v"(qf[24]), "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]),
               "v"(qf[29]), "v"(qf[30]), "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]),
               "v"(qf[35]));
  __syncthreads();

  const char* pool = static_cast<const char*>(a.pool);
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)tiles;

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

  // Source of tile i: the address of its first row (a bad table entry reads
  // row 0 and makes the output NaN) and its last valid row; rows past it
  // re-read that row and get probability 0.
  auto tile_src = [&](int i, const char** src, int* rlast) {
    const int base = __builtin_amdgcn_readfirstlane(tile_base[i]);
    *src = pool + (size_t)(base < 0 ? 0 : base) * (kW * 2);
    const int t0 = row_begin + i * kTile;
    *rlast = (t0 + kTile <= row_end) ? kTile - 1 : row_end - 1 - t0;
  };
  // Copy granule k of tile i: 16 bytes per lane straight into LDS at
  // M0 + 16 * lane.  Issued from asm so that the compiler does not treat every
  // later LDS read as aliasing the copy; the explicit vmcnt waits order them.
  auto clamp_rows = [&](uint32_t off, int rlast) {  // rows past rlast re-read row rlast
    const int r = (int)(off / (kW * 2));
    return r > rlast ? off - (uint32_t)((r - rlast) * (kW * 2)) : off;
  };
  auto issue_load = [&](int i, int k, uint32_t off, const char* src) {
    const uint32_t lds = tiles_lds + (uint32_t)((i % kBufs) * kTileBytes + (k * 4 + wave) * 1024);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(src), "s"(lds)
                 : "memory");
  };
  auto issue_tile = [&](int i) {
    const char* src;
    int rlast;
    tile_src(i, &src, &rlast);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      uint32_t off = goff_lds[k * kThreads + tid];
      if (rlast < kTile - 1) off = clamp_rows(off, rlast);
      issue_load(i, k, off, src);
    }
  };

  f32x16_t o[kC / 32];
#pragma unroll
  for (int cb = 0; cb < kC / 32; ++cb) o[cb] = f32x16_t{};
  // p = 2^(s*scale*log2e - m_ref) with a per-head reference m_ref taken from
  // the first tile.  If a later tile's maximum exceeds it by more than
  // kRestartLog2 (p would leave the safe range), the workgroup restarts the
  // split with the largest maximum seen as the new reference.  The restart
  // never touches O in registers: the next accumulation simply takes C = 0.
  const float c = a.scale_log2;
  float m_ref = -INFINITY;
  float m_seen = -INFINITY;
  float l_run = 0.f;
  bool bad = false;
  bool pending = false;
  bool fresh = true;     // the next tile is the first since the (re)start
  int zero_c = 0;        // 1: the next accumulation starts from C = 0

  issue_tile(0);
  if (ntiles > 1) issue_tile(1);
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
  bf16x8_t kf[5];  // K fragments of the next five k-blocks
  // Iteration ntiles only collects the last tile's restart vote.
  for (int i = 0; i <= ntiles; ++i) {
    // Tile i > 0 was waited for before the previous tile's P barrier.
    if (i + 1 >= ntiles) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if (i == 0) {
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // tile 0 (tile 1's copies are newer)
    }
    if (lane == 0) votes[(i & 1) * 4 + wave] = __ballot(pending) != 0;
    __syncthreads();
    bool restart;
    {
      const MLA_LDS int* v = votes + (i & 1) * 4;
      restart = (v[0] | v[1] | v[2] | v[3]) != 0;
    }
    if (restart) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      m_ref = m_seen;
      l_run = 0.f;
      pending = false;
      fresh = true;
      zero_c = 1;
      issue_tile(0);
      if (ntiles > 1) issue_tile(1);
      i = -1;
      continue;
    }
    if (i == ntiles) break;
    bad |= tile_base[i] < 0;
    // Copies of tile i + 2 go out between the score MFMAs.  Past the split's
    // end they still go out (no branch in the MFMA sequence): they re-read the
    // pool's first 32 rows into the idle third buffer, and the vmcnt(0) at
    // the top of the last passes drains them.
    const char* nsrc = pool;
    int nrlast = kTile - 1;
    uint32_t noff[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) noff[k] = goff_lds[k * kThreads + tid];
    if (i + 2 < ntiles) {
      tile_src(i + 2, &nsrc, &nrlast);
      if (nrlast < kTile - 1) {  // the split's last tile: once per split
#pragma unroll
        for (int k = 0; k < kLoads; ++k) noff[k] = clamp_rows(noff[k], nrlast);
      }
    }

    const uint32_t tile = tiles_lds + (uint32_t)((i % kBufs) * kTileBytes);

    // ---- scores S^T (rows x heads): two accumulators (even / odd k-block),
    // K fragments read five k-blocks ahead; the next tile's copies are issued
    // between the MFMAs ----
    f32x16_t s;
    {
      f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
      uint32_t qa[4];
      kbases(tile, qa);
      if (i == 0) {  // otherwise read during the previous tile's P*V
#pragma unroll
        for (int kb = 0; kb < 5; ++kb) kf[kb] = *kaddr(qa, kb);
      }
#pragma unroll
      for (int kb = 0; kb < kW / 16; ++kb) {
        if (kb & 1)
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb % 5], qf[kb], s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb % 5], qf[kb], s0, 0, 0, 0);
        if (kb + 5 < kW / 16) kf[kb % 5] = *kaddr(qa, kb + 5);
        if ((kb & 3) == 3) issue_load(i + 2, kb >> 2, noff[kb >> 2], nsrc);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = s0 + s1;
    }

    // ---- V^T fragments for this wave's 128 latent columns (column blocks
    // 4*wave .. +3: (cb >> 1) = 2*wave + (cbl >> 1), cb & 1 = cbl & 1).  They do
    // not depend on P, so they are read now and land while the softmax runs. ----
    s16x8_t vf[2][4];
    {
      uint32_t va[2][2];
#pragma unroll
      for (int c1 = 0; c1 < 2; ++c1)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          va[c1][rr] = tile + (((pv0 ^ (uint32_t)(64 * c1)) ^ (uint32_t)(32 * rr)) + 9216u * rr) +
                       (uint32_t)(wave * 256);
      auto vread = [&](int cbl, int kb) {
        const uint32_t off = kb * (16 * kGran * 16) + (cbl >> 1) * 128;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (MLA_LDS s16x4_t*)(uintptr_t)(va[cbl & 1][0] + off));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (MLA_LDS s16x4_t*)(uintptr_t)(va[cbl & 1][1] + off));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 4; ++x) vf[kb][x] = vread(x, kb);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- softmax numerators: lane = head, 16 rows per lane (the rest in lane ^ 32) ----
    const int t0 = row_begin + i * kTile;
    const bool tail = t0 + kTile > row_end;
    if (tail) {  // rows past the end do not take part in the maximum
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = t0 + (j >> 2) * 8 + hf * 4 + (j & 3);
        s[j] = t < row_end ? s[j] : __builtin_nanf("");
      }
    }
    // extreme of the raw scores (max for a positive scale, min for a negative one);
    // fmax/fmin ignore the NaN of masked rows
    float e;
    if (c >= 0.f) {
      e = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      e = fmaxf(e, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
      float lo, hi;
      wave_halves(e, &lo, &hi);
      e = fmaxf(lo, hi);
    } else {
      e = fminf(fminf(fminf(s[0], s[1]), fminf(s[2], s[3])), fminf(fminf(s[4], s[5]), fminf(s[6], s[7])));
      e = fminf(e, fminf(fminf(fminf(s[8], s[9]), fminf(s[10], s[11])),
                         fminf(fminf(s[12], s[13]), fminf(s[14], s[15]))));
      float lo, hi;
      wave_halves(e, &lo, &hi);
      e = fminf(lo, hi);
    }
    const float mt = e * c;
    m_seen = fmaxf(m_seen, mt);
    if (fresh) m_ref = fmaxf(m_ref, mt);
    fresh = false;
    pending = mt > m_ref + kRestartLog2;

    // This lane's 16 numerators, bf16, into the shared P in slot order: head
    // row h holds slot kb*16 + hf*8 + j <-> row 16*kb + 8*(j/4) + 4*hf + j%4,
    // the order both MFMA operands of P*V use.  The denominator sums the fp32
    // numerators (so lse stays exact to fp32, independent of the split plan).
    {
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(s[j], c, -m_ref));
      if (tail) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int t = t0 + (j >> 2) * 8 + hf * 4 + (j & 3);
          p[j] = t < row_end ? p[j] : 0.f;
        }
      }
      bf16x8_t pb[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) pb[j >> 3][j & 7] = (__bf16)p[j];
      float q0 = (p[0] + p[1]) + (p[2] + p[3]), q1 = (p[4] + p[5]) + (p[6] + p[7]);
      float q2 = (p[8] + p[9]) + (p[10] + p[11]), q3 = (p[12] + p[13]) + (p[14] + p[15]);
      l_run += (q0 + q1) + (q2 + q3);
      MLA_LDS char* prow = p_lds + p_row + wave * (32 * kPRow);
      *(MLA_LDS bf16x8_t*)prow = pb[0];
      *(MLA_LDS bf16x8_t*)(prow + 32) = pb[1];
    }
    // this wave's copies of tile i + 1 (all but the newest kLoads) have landed
    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    __syncthreads();  // every head's P is visible, and so is tile i + 1

    // ---- O^T += V^T P^T for this wave's 128 latent columns and all 128 heads:
    // V is read from LDS once per workgroup ----
    {
      bf16x8_t pf[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {  // the first half's fragments first
#pragma unroll
        for (int x = 0; x < 4; ++x)
          pf[kb][x] = *(const MLA_LDS bf16x8_t*)(p_lds + p_row + x * (32 * kPRow) + kb * 32);
        __builtin_amdgcn_sched_barrier(0);
      }
      // first k-block, 16 MFMAs in one block; C = 0 right after a restart
      // (one uniform branch per tile)
      asm volatile(
          "s_cmp_eq_u32 %24, 0\n\t"
          "s_cbranch_scc1 1f\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %16, %20, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %16, %21, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %16, %22, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %16, %23, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %4, %17, %20, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %5, %17, %21, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %6, %17, %22, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %7, %17, %23, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %8, %18, %20, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %9, %18, %21, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %10, %18, %22, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %11, %18, %23, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %12, %19, %20, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %13, %19, %21, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %14, %19, %22, 0\n\t"
          "v_mfma_f32_32x32x16_bf16 %15, %19, %23, 0\n\t"
          "s_branch 2f\n"
          "1:\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %16, %20, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %1, %16, %21, %1\n\t"
          "v_mfma_f32_32x32x16_bf16 %2, %16, %22, %2\n\t"
          "v_mfma_f32_32x32x16_bf16 %3, %16, %23, %3\n\t"
          "v_mfma_f32_32x32x16_bf16 %4, %17, %20, %4\n\t"
          "v_mfma_f32_32x32x16_bf16 %5, %17, %21, %5\n\t"
          "v_mfma_f32_32x32x16_bf16 %6, %17, %22, %6\n\t"
          "v_mfma_f32_32x32x16_bf16 %7, %17, %23, %7\n\t"
          "v_mfma_f32_32x32x16_bf16 %8, %18, %20, %8\n\t"
          "v_mfma_f32_32x32x16_bf16 %9, %18, %21, %9\n\t"
          "v_mfma_f32_32x32x16_bf16 %10, %18, %22, %10\n\t"
          "v_mfma_f32_32x32x16_bf16 %11, %18, %23, %11\n\t"
          "v_mfma_f32_32x32x16_bf16 %12, %19, %20, %12\n\t"
          "v_mfma_f32_32x32x16_bf16 %13, %19, %21, %13\n\t"
          "v_mfma_f32_32x32x16_bf16 %14, %19, %22, %14\n\t"
          "v_mfma_f32_32x32x16_bf16 %15, %19, %23, %15\n\t"
          "2:"
          : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]),
            "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]),
            "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15])
          : "v"(vf[0][0]), "v"(vf[0][1]), "v"(vf[0][2]), "v"(vf[0][3]), "v"(pf[0][0]),
            "v"(pf[0][1]), "v"(pf[0][2]), "v"(pf[0][3]), "s"(zero_c)
          : "scc");
      __builtin_amdgcn_sched_barrier(0);
      // the first K fragments of tile i + 1 go out between the second half's
      // MFMAs, where the first half's fragments are dead
      uint32_t nqa[4];
      kbases(tiles_lds + (uint32_t)(((i + 1) % kBufs) * kTileBytes), nqa);
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+a"(o[cbl * 4 + hb])
                       : "v"(vf[1][cbl]), "v"(pf[1][hb]));
          const int n = cbl * 4 + hb;
          if (n % 3 == 0 && n / 3 < 5) kf[n / 3] = *kaddr(nqa, n / 3);
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    zero_c = 0;
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
  float l_lo, l_hi;
  wave_halves(l_run, &l_lo, &l_hi);
  const float l = l_lo + l_hi;
  if (hf == 0) l_heads[head] = l;
  __syncthreads();
  if (a.num_splits == 1) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float inv_l = bad ? NAN : 1.0f / l_heads[hb * 32 + l32];
      float* dst = a.v_combine + (size_t)b * kH * kC + (size_t)(hb * 32 + l32) * kC + wave * 128;
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = cbl * 32 + q4 * 8 + hf * 4;
          const f32x16_t& ob = o[cbl * 4 + hb];
          f32x4_t v{ob[4 * q4 + 0] * inv_l, ob[4 * q4 + 1] * inv_l, ob[4 * q4 + 2] * inv_l,
                    ob[4 * q4 + 3] * inv_l};
          *reinterpret_cast<f32x4_t*>(dst + col) = v;
        }
      }
    }
  } else {
    // fp16 partial: O / l * 2^-e with e >= 0 the smallest exponent that keeps
    // the head's largest magnitude under 2^15 (0 unless |V| is huge); the
    // largest |O| / l of each head over the four waves meets in LDS (the P
    // area, free after the barrier above).
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
      // floor(log2 amax) from the exponent bits; e keeps amax * 2^-e below 2^15
      const int lg = (int)((__float_as_uint(amax) >> 23) & 255u) - 127;
      const int e = (amax >= 32768.f && amax <= 3.0e38f) ? lg - 14 : 0;
      const float scale = __uint_as_float((uint32_t)(127 - e) << 23);
      const float inv_l = bad ? NAN : scale / l_heads[h];
      _Float16* dst = a.part_oh + (bs * kH + h) * kC + wave * 128;
#pragma unroll
      for (int cbl = 0; cbl < 4; ++cbl) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = cbl * 32 + q4 * 8 + hf * 4;
          const f32x16_t& ob = o[cbl * 4 + hb];
          typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
          const f16x4_t v{(_Float16)(ob[4 * q4 + 0] * inv_l), (_Float16)(ob[4 * q4 + 1] * inv_l),
                          (_Float16)(ob[4 * q4 + 2] * inv_l), (_Float16)(ob[4 * q4 + 3] * inv_l)};
          *reinterpret_cast<f16x4_t*>(dst + col) = v;
        }
      }
      if (wave == 0 && hf == 0) a.part_exp[bs * kH + h] = (float)e;
    }
  }
  if (out_lse && hf == 0) *out_lse = bad ? NAN : (m_ref + log2f(l)) * kLn2;
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
// split's weight.  One wave per (sequence, head), 8 consecutive latent columns
// per lane, so every split's partial row is one 1 KB coalesced read per wave;
// four heads per workgroup.
__global__ void __launch_bounds__(256) attn_combine_f16_kernel(AttnArgs a) {
  const int b = blockIdx.y;
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int S = a.num_splits;
  const float* lse_s = a.part_lse + (size_t)b * S * kH + h;  // stride kH over s
  const float* exp_s = a.part_exp + (size_t)b * S * kH + h;

  float m = -INFINITY;
  bool nan_lse = false;  // a bad table entry: NaN through the merge, as above
  for (int s = lane; s < S; s += 64) {
    const float l = lse_s[(size_t)s * kH];
    m = fmaxf(m, l);
    nan_lse |= l != l;
  }
  m = wave_max(m);
  if (__ballot(nan_lse) != 0) m = NAN;
  float* dst = a.v_combine + ((size_t)b * kH + h) * kC + lane * 8;
  if (m == -INFINITY) {  // empty sequence
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < S; s += 64) wsum += expf(lse_s[(size_t)s * kH] - m);
  wsum = wave_sum(wsum);
  const float inv = 1.0f / wsum;

  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  const _Float16* src = a.part_oh + ((size_t)b * S * kH + h) * kC + lane * 8;
  const size_t sstride = (size_t)kH * kC;
  f32x4_t lo{0.f, 0.f, 0.f, 0.f}, hi{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float ls = lse_s[(size_t)s * kH];
    if (ls == -INFINITY) continue;  // an empty split leaves its partial unwritten
    const float w = ldexpf(expf(ls - m), (int)exp_s[(size_t)s * kH]);
    const f16x8_t v = *reinterpret_cast<const f16x8_t*>(src + (size_t)s * sstride);
    lo += w * f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    hi += w * f32x4_t{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
  }
  *reinterpret_cast<f32x4_t*>(dst) = lo * inv;
  *reinterpret_cast<f32x4_t*>(dst + 4) = hi * inv;
  if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = m + logf(wsum);
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
  if (a.part_oh)
    hipLaunchKernelGGL(attn_combine_f16_kernel, dim3(kH / 4, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel, dim3((a.H + 1) / 2, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

int attn_mfma_max_split_rows() { return kMaxSplitTiles * kTile; }
