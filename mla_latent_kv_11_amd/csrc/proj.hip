// Projection, norm, append and absorb kernels of the MLA decode step.
//
//  gemm_nt_kernel     y = x W^T for fp32 / bf16 / 4-bit affine (group 64) weights
//                     (moeflux gpu_matvec.rs, encode_matvec and MatvecSpec; the
//                     same weight applied to a batch of token vectors as in
//                     encode_matvec_n_tokens), batched over heads for W_UV.
//  rmsnorm_rows       in-place RMSNorm of the q LoRA latent (q_a_layernorm).
//  append_rows_kernel latent RMSNorm + YaRN RoPE of k_pe + one rounded row into
//                     the paged slot (turbospark deepseek2/attn.rs, the fused
//                     cache row; moeflux mla_attn_forward.rs, the cache append).
//  absorb_kernel      q' = W_UK^T q_nope and RoPE(q_pe) packed as q_abs rows
//                     (turbospark deepseek2/attn.rs, encode_mla_absorb_q).
//  qb_absorb_kernel   q_b and the absorb in one launch, q kept in LDS (moeflux
//                     mla_attn_forward.rs, the Q chain into mla_q_prime_4bit).
//  merge_uv_kernel    the split-K merge of decode attention and W_UV in one
//                     launch (moeflux mla_attn_forward.rs, mla_sdpa_folded's
//                     output expanded per head).
#include <math.h>

#include <mutex>
#include <type_traits>

#include "mla_common.h"

namespace {

// ---------------------------------------------------------------------------
// y[z][b][o] = sum_k W[row(z, o)][k] x[z][b][k]; tile 64 outputs x 32 tokens,
// K chunks of 32 through LDS; each thread owns 4 outputs x 2 tokens.
// ---------------------------------------------------------------------------
constexpr int kTO = 64, kTB = 32, kTK = 32;

__global__ void __launch_bounds__(256) gemm_nt_kernel(GemmArgs a) {
  __shared__ float ws[kTO][kTK + 1];
  __shared__ float xs[kTB][kTK + 1];
  const int z = blockIdx.z;
  const int o0 = blockIdx.x * kTO;
  const int b0 = blockIdx.y * kTB;
  const int tid = threadIdx.x;
  const int to = tid >> 4;   // outputs 4*to .. +3
  const int tb = tid & 15;   // tokens 2*tb .. +1
  const int64_t wrow = a.w_row0 + (int64_t)z * a.w_zrows;
  const float* x = a.x + (int64_t)z * a.x_z;
  float acc[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};

  for (int k0 = 0; k0 < a.K; k0 += kTK) {
#pragma unroll
    for (int i = 0; i < (kTO * kTK) / 256; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 5, c = e & 31;
      const int o = o0 + r, k = k0 + c;
      ws[r][c] = (o < a.O && k < a.K) ? weight_at(a.w, wrow + o, k) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < (kTB * kTK) / 256; ++i) {
      const int e = tid + 256 * i;
      const int r = e >> 5, c = e & 31;
      const int bb = b0 + r, k = k0 + c;
      xs[r][c] = (bb < a.B && k < a.K) ? x[(int64_t)bb * a.x_b + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kTK; ++kk) {
      float wv[4], xv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = ws[4 * to + i][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) xv[j] = xs[2 * tb + j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = fmaf(wv[i], xv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = o0 + 4 * to + i, bb = b0 + 2 * tb + j;
      if (o >= a.O || bb >= a.B) continue;
      if (a.yp)
        a.yp[packed_index(0, bb, (int64_t)z * a.y_z + o, a.B, a.yp_K)] = (_Float16)acc[i][j];
      else
        a.y[(int64_t)z * a.y_z + (int64_t)bb * a.y_b + o] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// 4-bit affine weights on MFMA (v_mfma_f32_32x32x16_f16, fp32 accumulate).
//
// A workgroup owns 32 weight rows x 32 tokens and nw waves; wave w takes U
// consecutive units of 128 k (unit u covers k = 128u .. 128u + 127) starting at
// unit (s*nw + w)*U, where s is the workgroup's K split.  Tokens are the M
// operand and weight rows the N operand, so the reduced tile is stored as 32
// consecutive outputs per token.  In a unit, lane-half hh holds k = 128u + 64hh
// + 8st + (0..7) at MFMA step st; register r of a step pairs k-offsets r and
// r + 4, which are the two nibbles ((word >> 4r) & 0x000F000F) of packed word
// st, and the packed activations hold the same pairs.  A nibble becomes an
// exact fp16 integer plus q by bit operations alone: at mantissa bits 0-3
// under the exponent bits 0x6400 it reads 1024 + q, at bits 4-7 under 0x5400
// it reads 64 + q, so pairs 0 and 1 come from the word itself and pairs 2
// and 3 from the word shifted by 8, one mask-and-or each; then q * scale +
// bias in packed fp16 arithmetic.  The next unit's loads are issued before
// the current unit is multiplied.  The nw partial tiles are added in LDS in a
// fixed order.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kQ4MaxWaves = 16;

struct Unit {  // one lane's share of a unit: 64 nibbles of its row, 64 activations
  uint4 w[2];
  uint16_t sc, bi;
  uint4 x[8];
};

// (word & mask) | bits as one v_and_or_b32: gfx950's VOP3 form takes no
// literal and one scalar operand, so the mask comes in a VGPR and the
// exponent bits in an SGPR (the compiler emits a separate and and or).
__device__ __forceinline__ uint32_t and_or(uint32_t word, uint32_t mask_v, uint32_t bits_s) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(word), "v"(mask_v), "s"(bits_s));
  return r;
}

__device__ __forceinline__ f16x8_t dequant8(uint32_t word, f16x2_t s2, f16x2_t b2) {
  const f16x2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const f16x2_t k64 = {(_Float16)64.f, (_Float16)64.f};
  const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u;  // nibbles 0 and 4, 1 and 5 of a word
  const uint32_t w8 = word >> 8;                      // nibbles 2 and 6, 3 and 7 at those bits
  const f16x2_t q0 = __builtin_bit_cast(f16x2_t, and_or(word, lo, 0x64006400u)) - k1024;
  const f16x2_t q1 = __builtin_bit_cast(f16x2_t, and_or(word, hi, 0x54005400u)) - k64;
  const f16x2_t q2 = __builtin_bit_cast(f16x2_t, and_or(w8, lo, 0x64006400u)) - k1024;
  const f16x2_t q3 = __builtin_bit_cast(f16x2_t, and_or(w8, hi, 0x54005400u)) - k64;
  const uint32_t r0 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q0, s2, b2));
  const uint32_t r1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q1, s2, b2));
  const uint32_t r2 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, b2));
  const uint32_t r3 = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q3, s2, b2));
  return __builtin_bit_cast(f16x8_t, uint4{r0, r1, r2, r3});
}

// Q8_0: a lane's share of a unit is two 34-byte blocks of its row (64 of the
// unit's 128 k).  The q bytes of a block start 2 bytes into it, so they are
// read as 8 aligned dwords from the 4-byte boundary at or below their start,
// plus the 16-bit word after those (used when the start is 2 mod 4, and
// otherwise read from inside the block so no load passes its end).
struct UnitQ8 {
  uint32_t q[2][8];
  uint16_t qx[2];
  uint16_t d[2];
  uint4 x[8];
};

// 8 signed bytes (k0..k3 in lo, k4..k7 in hi) times a binary16 scale, as fp16
// in the pair order k0 k4 k1 k5 k2 k6 k3 k7 of the packed activations: byte
// pairs become fp16 1024 + (q + 128) by their bit patterns (the sign bit of
// each byte flipped, 0x64 above it), then 1152 is subtracted (exact) and the
// products d * q are rounded once to fp16.
__device__ __forceinline__ f16x8_t dequant8_q8(uint32_t lo, uint32_t hi, f16x2_t d2) {
  const f16x2_t k1152 = {(_Float16)1152.f, (_Float16)1152.f};
  uint32_t r[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // result bytes: lo.b, 0, hi.b, 0
    const uint32_t sel = (uint32_t)b | (0x0cu << 8) | ((uint32_t)(4 + b) << 16) | (0x0cu << 24);
    const uint32_t t = __builtin_amdgcn_perm(hi, lo, sel) ^ 0x64806480u;
    const f16x2_t q = __builtin_bit_cast(f16x2_t, t) - k1152;
    r[b] = __builtin_bit_cast(uint32_t, q * d2);
  }
  return __builtin_bit_cast(f16x8_t, uint4{r[0], r[1], r[2], r[3]});
}

// Row tile bx (32 output rows) of y = x W^T for the token tile blockIdx.y and
// the (z, K split) pair blockIdx.z.
template <int U, bool kQ8>
__device__ __forceinline__ void gemm_mfma_body(const GemmArgs& a, int bx, int nw, int S, float* red) {
  const int zz = blockIdx.z / S, s = blockIdx.z - zz * S;
  const int o0 = bx * 32, b0 = blockIdx.y * 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int units = a.K >> 7;
  const int ubeg = (s * nw + wave) * U;

  int row = o0 + l32;
  row = row < a.O ? row : a.O - 1;  // rows past the end read a valid row; never stored
  const uint32_t wrow = (uint32_t)(a.w_row0 + (int64_t)zz * a.w_zrows + row);
  // Per-lane 32-bit byte offsets from uniform bases (the matrices are under
  // 2 GiB), so each load takes one address register instead of a 64-bit pointer.
  const char* wbase = static_cast<const char*>(a.w.data);
  const char* sbase = reinterpret_cast<const char*>(a.w.scales);
  const char* bbase = reinterpret_cast<const char*>(a.w.biases);
  const char* xbase = reinterpret_cast<const char*>(a.xp);
  // Row-major 4-bit rows: the lane's 32 bytes of a unit at 64 B per unit along
  // its row (a load instruction touches 32 rows).  MLA_Q4G64_T: a 2 KB block
  // per (32-row tile, unit), lane (wrow % 32) + 32 hh at 16 B steps in each
  // 1 KB half, so a load instruction reads 1 KB in one piece.
  const bool tiled = a.w.dtype == MLA_Q4G64_T;
  const uint32_t tblk = (wrow >> 5) * (uint32_t)(a.w.cols >> 7), tlane = (wrow & 31u) + 32u * hh;
  const uint32_t woff = tiled ? tblk * 2048u + 16u * tlane : wrow * (uint32_t)(a.w.cols >> 1) + 32u * hh;
  const uint32_t soff = tiled ? tblk * 128u + 2u * tlane : wrow * (uint32_t)(a.w.cols >> 6) * 2u + 2u * hh;
  const uint32_t wstep = tiled ? 2048u : 64u, whalf = tiled ? 1024u : 16u, sstep = tiled ? 128u : 4u;
  const uint32_t xoff =
      (uint32_t)((zz * gridDim.y + blockIdx.y) * units) * 8192u + 16u * lane;  // + 8192 per unit
  // Q8_0: byte offset of the lane's first block (+ 136 per unit), and the
  // shift that realigns each block's q bytes (unit strides keep it fixed)
  const uint32_t q8off = wrow * (uint32_t)((a.w.cols >> 5) * 34) + 68u * hh;
  const uint32_t q8sh[2] = {((q8off + 2u) & 2u) * 8u, ((q8off + 36u) & 2u) * 8u};

  using UnitT = typename std::conditional<kQ8, UnitQ8, Unit>::type;
  UnitT ub[2];
  auto issue = [&](int slot, int ku) {
    const uint32_t xo = xoff + 8192u * ku;
    if constexpr (kQ8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t blk = q8off + 136u * ku + 34u * j, qs = blk + 2u, al = qs & ~3u;
        ub[slot].d[j] = *reinterpret_cast<const uint16_t*>(wbase + blk);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          ub[slot].q[j][i] = *reinterpret_cast<const uint32_t*>(wbase + al + 4u * i);
        ub[slot].qx[j] = *reinterpret_cast<const uint16_t*>(wbase + ((qs & 2u) ? al + 32u : al + 30u));
      }
    } else {
      const uint32_t wo = woff + wstep * ku, so = soff + sstep * ku;
      ub[slot].w[0] = *reinterpret_cast<const uint4*>(wbase + wo);
      ub[slot].w[1] = *reinterpret_cast<const uint4*>(wbase + wo + whalf);
      ub[slot].sc = *reinterpret_cast<const uint16_t*>(sbase + so);
      ub[slot].bi = *reinterpret_cast<const uint16_t*>(bbase + so);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      ub[slot].x[st] = *reinterpret_cast<const uint4*>(xbase + xo + 1024u * st);
  };

  // Loads are issued unconditionally (units past the end re-read the last one)
  // so the number of loads in flight is the same on every path and the wait
  // before a unit's MFMAs leaves the next unit's loads outstanding.
  const int ulast = units - 1;
  f32x16_t acc = f32x16_t{};
  issue(0, ubeg < ulast ? ubeg : ulast);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int ku = ubeg + u;
    if (u + 1 < U) issue((u + 1) & 1, ku + 1 < ulast ? ku + 1 : ulast);
    if (ku >= units) continue;
    const UnitT& c = ub[u & 1];
    if constexpr (kQ8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const _Float16 dh = __builtin_bit_cast(_Float16, c.d[j]);
        const f16x2_t d2 = {dh, dh};
        uint32_t qd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          qd[i] = __builtin_amdgcn_alignbit(i < 7 ? c.q[j][i + 1] : (uint32_t)c.qx[j], c.q[j][i],
                                            q8sh[j]);
#pragma unroll
        for (int st4 = 0; st4 < 4; ++st4)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8_t, c.x[4 * j + st4]),
              dequant8_q8(qd[2 * st4], qd[2 * st4 + 1], d2), acc, 0, 0, 0);
      }
    } else {
      const _Float16 sh = (_Float16)bf16_to_f32(c.sc), bh = (_Float16)bf16_to_f32(c.bi);
      const f16x2_t s2 = {sh, sh}, b2 = {bh, bh};
      const uint32_t words[8] = {c.w[0].x, c.w[0].y, c.w[0].z, c.w[0].w,
                                 c.w[1].x, c.w[1].y, c.w[1].z, c.w[1].w};
#pragma unroll
      for (int st = 0; st < 8; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, c.x[st]),
                                                     dequant8(words[st], s2, b2), acc, 0, 0, 0);
    }
  }

#pragma unroll
  for (int j = 0; j < 16; ++j) red[(wave * 16 + j) * 64 + lane] = acc[j];
  __syncthreads();
  const int nthr = nw * 64;
  for (int e = threadIdx.x; e < 1024; e += nthr) {
    const int ln = e & 63, j = e >> 6;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += red[(w * 16 + j) * 64 + ln];
    const int o = o0 + (ln & 31);
    const int t = b0 + (j >> 2) * 8 + (ln >> 5) * 4 + (j & 3);
    if (o >= a.O || t >= a.B) continue;
    if (a.x_exp) v = ldexpf(v, a.x_exp[t]);
    if (a.yp)
      a.yp[packed_index(0, t, (int64_t)zz * a.y_z + o, a.B, a.yp_K)] = (_Float16)v;
    else
      a.y[(int64_t)s * a.y_s + (int64_t)zz * a.y_z + (int64_t)t * a.y_b + o] = v;
  }
}

template <int U>
__global__ void __launch_bounds__(64 * kQ4MaxWaves) gemm_q4_mfma_kernel(GemmArgs a, int nw, int S) {
  extern __shared__ float red[];  // [nw][16][64]
  gemm_mfma_body<U, false>(a, blockIdx.x, nw, S, red);
}

template <int U>
__global__ void __launch_bounds__(64 * kQ4MaxWaves) gemm_q8_mfma_kernel(GemmArgs a, int nw, int S) {
  extern __shared__ float red[];  // [nw][16][64]
  gemm_mfma_body<U, true>(a, blockIdx.x, nw, S, red);
}

// Two products of the same packed activations in one launch: the first
// tiles_a row tiles are a's, the rest b's (same depth, tokens and K splits;
// each workgroup's arithmetic is that of its own single launch).
template <int U, bool kQ8>
__global__ void __launch_bounds__(64 * kQ4MaxWaves) gemm_pair_mfma_kernel(GemmArgs a, GemmArgs b,
                                                                          int tiles_a, int nw, int S) {
  extern __shared__ float red[];  // [nw][16][64]
  const int bx = blockIdx.x;
  if (bx < tiles_a) gemm_mfma_body<U, kQ8>(a, bx, nw, S, red);
  else gemm_mfma_body<U, kQ8>(b, bx - tiles_a, nw, S, red);
}

// fp32 x[z*x_z + b*x_b + k] -> packed fp16; one thread writes one 16-byte chunk
// (8 values of one token), so the stores are contiguous.  blockIdx.x is the
// (z, token tile) pair and y covers its units * 512 chunks, so the chunk's
// coordinates come from shifts and masks (one division per workgroup).
__global__ void __launch_bounds__(256) pack_f16_kernel(const float* x, int64_t x_b, int64_t x_z,
                                                       int32_t B, int32_t K, bool vec,
                                                       _Float16* xp) {
  const int units = K >> 7, tiles = (B + 31) >> 5;
  const int zt = blockIdx.x;  // z * tiles + tile
  const int z = zt / tiles, tile = zt - z * tiles;
  const int cz = blockIdx.y * 256 + threadIdx.x;  // chunk inside this (z, tile)
  if (cz >= units * 512) return;
  const int lane = cz & 63, st = (cz >> 6) & 7, u = cz >> 9;
  const int64_t b = (int64_t)tile * 32 + (lane & 31);
  const int64_t k = (int64_t)u * 128 + (lane >> 5) * 64 + st * 8;
  uint4 o = uint4{0u, 0u, 0u, 0u};
  if (b < B) {
    const float* src = x + z * x_z + b * x_b + k;
    float v[8];
    if (vec) {
      const float4 v0 = reinterpret_cast<const float4*>(src)[0];
      const float4 v1 = reinterpret_cast<const float4*>(src)[1];
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = src[i];
    }
    const f16x8_t h = {(_Float16)v[0], (_Float16)v[4], (_Float16)v[1], (_Float16)v[5],
                       (_Float16)v[2], (_Float16)v[6], (_Float16)v[3], (_Float16)v[7]};
    o = __builtin_bit_cast(uint4, h);
  }
  reinterpret_cast<uint4*>(xp)[(int64_t)zt * units * 512 + cz] = o;
}

// Sum of S <= kMaxKSplits partials p[s * stride]; every load is issued
// unconditionally (clamped to split 0) so they overlap.
__device__ __forceinline__ float sum_splits(const float* p, int S, int64_t stride) {
  float v = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxKSplits; ++sp) {
    const float t = p[(sp < S ? sp : 0) * stride];
    v += sp < S ? t : 0.f;
  }
  return v;
}

// Sum over the 256 threads of a block; every thread gets the total.
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  __syncthreads();
  return t;
}

// Largest value over the threads of a block; every thread gets it.
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, red[i]);
  __syncthreads();
  return t;
}

// fp32 x[b*x_b + k] -> packed fp16 with a power-of-two scale per token: one
// workgroup per token slot of the padded tiles finds the token's largest
// magnitude, then writes its 16-byte chunks (8 values each) times 2^-e; token
// slots past B are zero.  x is read twice (the second time from cache).
__global__ void __launch_bounds__(256) pack_scaled_kernel(const float* x, int64_t x_b, int32_t B,
                                                          int32_t K, bool vec, _Float16* xp,
                                                          int32_t* x_exp) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const float* row = x + (int64_t)(b < B ? b : 0) * x_b;
  auto load8 = [&](int k, float v[8]) {
    if (vec) {
      const float4 v0 = reinterpret_cast<const float4*>(row + k)[0];
      const float4 v1 = reinterpret_cast<const float4*>(row + k)[1];
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = row[k + i];
    }
  };
  // the first kKeep chunks of each thread stay in registers between the two
  // passes (K <= 16384 at 256 threads); deeper rows read the rest twice
  constexpr int kKeep = 8;
  float keep[kKeep][8] = {};
  float m = 0.f;
  if (b < B) {
#pragma unroll
    for (int j = 0; j < kKeep; ++j) {
      const int c = threadIdx.x + 256 * j;
      if (c < K / 8) {
        load8(8 * c, keep[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(keep[j][i]));
      }
    }
    for (int c = threadIdx.x + 256 * kKeep; c < K / 8; c += 256) {
      float v[8];
      load8(8 * c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
  }
  const int e = f16_range_exp(block_max(m, red));  // uniform: b is
  if (b < B && threadIdx.x == 0) x_exp[b] = e;
  const float sc = pow2f(-e);
  auto put = [&](int c, const float* v) {
    uint4 o = uint4{0u, 0u, 0u, 0u};
    if (b < B) {
      const f16x8_t h = {(_Float16)(v[0] * sc), (_Float16)(v[4] * sc), (_Float16)(v[1] * sc),
                         (_Float16)(v[5] * sc), (_Float16)(v[2] * sc), (_Float16)(v[6] * sc),
                         (_Float16)(v[3] * sc), (_Float16)(v[7] * sc)};
      o = __builtin_bit_cast(uint4, h);
    }
    *reinterpret_cast<uint4*>(xp + packed_index(0, b, 8 * c, B, K)) = o;
  };
#pragma unroll
  for (int j = 0; j < kKeep; ++j) {
    const int c = threadIdx.x + 256 * j;
    if (c < K / 8) put(c, keep[j]);
  }
  for (int c = threadIdx.x + 256 * kKeep; c < K / 8; c += 256) {
    float v[8] = {};
    if (b < B) load8(8 * c, v);
    put(c, v);
  }
}


__device__ __forceinline__ float gamma_at(const WeightView& g, int i) {
  return g.dtype == MLA_F32 ? static_cast<const float*>(g.data)[i]
                            : bf16_to_f32(static_cast<const uint16_t*>(g.data)[i]);
}

__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(const float* part, int32_t S,
                                                           int64_t split_stride, int32_t B,
                                                           int32_t n, int64_t stride,
                                                           WeightView gamma, float eps, float* y,
                                                           _Float16* yp, int32_t* yexp) {
  __shared__ float red[4];
  const int64_t b = blockIdx.x;
  constexpr int kPer = 8;  // values per thread kept in registers (n <= 2048)
  float v[kPer];
  float ss = 0.f, mg = 0.f;  // mg: largest |value * gamma| (the output's, before 1 / rms)
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + 256 * r;
    v[r] = i < n ? sum_splits(part + b * stride + i, S, split_stride) : 0.f;
    ss = fmaf(v[r], v[r], ss);
    if (i < n) mg = fmaxf(mg, fabsf(v[r] * gamma_at(gamma, i)));
  }
  for (int i = threadIdx.x + 256 * kPer; i < n; i += 256) {
    const float t = sum_splits(part + b * stride + i, S, split_stride);
    ss = fmaf(t, t, ss);
    mg = fmaxf(mg, fabsf(t * gamma_at(gamma, i)));
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
  // packed output: scaled into binary16's range (the scale's rounding margin
  // is far inside it: the largest scaled value stays below 2^15 (1 + 2^-20))
  int e = 0;
  if (yp) {
    e = f16_range_exp(block_max(mg, red) * inv);
    if (yexp && threadIdx.x == 0) yexp[b] = e;
  }
  const float sc = pow2f(-e);
  auto put = [&](int i, float t) {
    const float o = t * inv * gamma_at(gamma, i);
    if (yp) yp[packed_index(0, b, i, B, n)] = (_Float16)(o * sc);
    else y[b * stride + i] = o;
  };
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = threadIdx.x + 256 * r;
    if (i < n) put(i, v[r]);
  }
  for (int i = threadIdx.x + 256 * kPer; i < n; i += 256)
    put(i, sum_splits(part + b * stride + i, S, split_stride));
}

// v[0..7] = sum over S <= kMaxKSplits of the 16-byte aligned 8-vectors
// p[s * stride .. +7]; the loads of eight splits are issued together (indices
// clamped to valid splits, the extra ones masked).
__device__ __forceinline__ void sum_splits8(const float* p, int S, int64_t stride, float v[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 lo[8], hi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sp = s0 + j < S ? s0 + j : S - 1;
      lo[j] = reinterpret_cast<const float4*>(p + sp * stride)[0];
      hi[j] = reinterpret_cast<const float4*>(p + sp * stride)[1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float m = s0 + j < S ? 1.f : 0.f;
      v[0] = fmaf(m, lo[j].x, v[0]); v[1] = fmaf(m, lo[j].y, v[1]);
      v[2] = fmaf(m, lo[j].z, v[2]); v[3] = fmaf(m, lo[j].w, v[3]);
      v[4] = fmaf(m, hi[j].x, v[4]); v[5] = fmaf(m, hi[j].y, v[5]);
      v[6] = fmaf(m, hi[j].z, v[6]); v[7] = fmaf(m, hi[j].w, v[7]);
    }
  }
}

__device__ __forceinline__ void gamma8(const WeightView& g, int k0, float gm[8]) {
  if (g.dtype == MLA_F32) {
    const float4 a = reinterpret_cast<const float4*>(static_cast<const float*>(g.data) + k0)[0];
    const float4 b = reinterpret_cast<const float4*>(static_cast<const float*>(g.data) + k0)[1];
    gm[0] = a.x; gm[1] = a.y; gm[2] = a.z; gm[3] = a.w;
    gm[4] = b.x; gm[5] = b.y; gm[6] = b.z; gm[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(g.data) + k0);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gm[2 * i] = __uint_as_float(u[i] << 16);
      gm[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

// RMSNorm of the summed split partials of one token per block, straight into
// the packed fp16 layout: thread t owns k = 8t .. 8t + 7, one 16-byte packed
// chunk.  Block = n/8 threads rounded up to whole waves; n % 8 == 0.
__device__ __forceinline__ void rmsnorm_pack_row(const float* part, int32_t S, int64_t split_stride,
                                                 int32_t B, int32_t n, int64_t stride,
                                                 WeightView gamma, float eps, _Float16* yp,
                                                 int32_t* yexp, int64_t b, float* red) {
  const int k0 = 8 * threadIdx.x;
  const bool on = k0 < n;
  float v[8] = {};
  if (on) sum_splits8(part + b * stride + k0, S, split_stride, v);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = on ? fmaf(v[i], v[i], ss) : ss;
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
  float gm[8] = {};
  if (on) gamma8(gamma, k0, gm);
  float o[8];
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i] = on ? v[i] * inv * gm[i] : 0.f;
    mx = fmaxf(mx, fabsf(o[i]));
  }
  // the row scaled into binary16's range by a power of two
  const int e = f16_range_exp(block_max(mx, red));
  if (!on) return;
  if (yexp && threadIdx.x == 0) yexp[b] = e;
  const float sc = pow2f(-e);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= sc;
  const f16x8_t h = {(_Float16)o[0], (_Float16)o[4], (_Float16)o[1], (_Float16)o[5],
                     (_Float16)o[2], (_Float16)o[6], (_Float16)o[3], (_Float16)o[7]};
  *reinterpret_cast<uint4*>(yp + packed_index(0, b, k0, B, n)) = __builtin_bit_cast(uint4, h);
}

__global__ void __launch_bounds__(1024) rmsnorm_pack_kernel(const float* part, int32_t S,
                                                            int64_t split_stride, int32_t B,
                                                            int32_t n, int64_t stride,
                                                            WeightView gamma, float eps,
                                                            _Float16* yp, int32_t* yexp) {
  __shared__ float red[16];
  rmsnorm_pack_row(part, S, split_stride, B, n, stride, gamma, eps, yp, yexp, blockIdx.x, red);
}

// (x, y) -> mscale * (x cos a - y sin a, x sin a + y cos a), a = pos * inv_freq.
// The angle is formed and reduced to [-pi, pi] in fp64 (pos * inv_freq in
// fp32 would lose up to 1e-3 rad at 16k), then sin/cos and the rotation run in
// fp32 (accurate library sincosf, about 1e-7 relative).
__device__ __forceinline__ void rope_pair(float x, float y, int pos, float inv_freq, float mscale,
                                          float* ox, float* oy) {
  const double two_pi = 6.283185307179586476925286766559;
  const double ang = (double)pos * (double)inv_freq;
  const float r = (float)(ang - two_pi * rint(ang / two_pi));
  float sn, cs;
  sincosf(r, &sn, &cs);
  *ox = mscale * (x * cs - y * sn);
  *oy = mscale * (x * sn + y * cs);
}

template <typename T>
__global__ void __launch_bounds__(256) append_rows_kernel(AppendArgs a) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int W = a.C + a.R;
  const int pos = a.positions[b];
  if (pos < 0 || (int64_t)pos >= (int64_t)a.max_blocks * a.block) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_POS_RANGE);
    return;
  }
  const int sq = a.q_seq ? a.q_seq[b] : b;
  if (sq < 0 || sq >= a.num_seqs) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_BAD_SEQ);
    return;
  }
  const int blk = a.table[(size_t)sq * a.max_blocks + pos / a.block];
  if (blk < 0 || blk >= a.num_blocks) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_BAD_BLOCK);
    return;
  }
  const float* src = a.kv_pre + (size_t)b * W;
  auto kv = [&](int i) { return sum_splits(src + i, a.kv_splits, a.kv_split_stride); };
  T* dst = static_cast<T*>(a.pool) + ((size_t)blk * a.block + pos % a.block) * W;
  float ss = 0.f;
  for (int i = threadIdx.x; i < a.C; i += 256) {
    const float v = kv(i);
    ss = fmaf(v, v, ss);
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)a.C + a.eps);
  for (int i = threadIdx.x; i < a.C; i += 256)
    Elem<T>::store(dst, i, kv(i) * inv * gamma_at(a.gamma, i));
  for (int i = threadIdx.x; i < a.R / 2; i += 256) {
    float ox, oy;
    rope_pair(kv(a.C + 2 * i), kv(a.C + 2 * i + 1), pos, a.inv_freq[i], a.rope_mscale, &ox, &oy);
    Elem<T>::store(dst, a.C + 2 * i, ox);
    Elem<T>::store(dst, a.C + 2 * i + 1, oy);
  }
}

// One appended row per block, 8 values per thread: threads t < C/8 own latent
// values 8t .. 8t + 7 (RMSNorm), the next R/8 own k_pe values (4 RoPE pairs
// each); every thread stores 8 cache elements at once.  C % 8 == R % 8 == 0.
template <typename T>
__device__ __forceinline__ void append_row_vec(const AppendArgs& a, int b, float* red) {
  const int W = a.C + a.R;
  const int pos = a.positions[b];
  if (pos < 0 || (int64_t)pos >= (int64_t)a.max_blocks * a.block) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_POS_RANGE);
    return;
  }
  const int sq = a.q_seq ? a.q_seq[b] : b;
  if (sq < 0 || sq >= a.num_seqs) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_BAD_SEQ);
    return;
  }
  const int blk = a.table[(size_t)sq * a.max_blocks + pos / a.block];
  if (blk < 0 || blk >= a.num_blocks) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_BAD_BLOCK);
    return;
  }
  const int k0 = 8 * threadIdx.x;
  const bool latent = k0 < a.C, on = k0 < W;
  float v[8];
  if (on) sum_splits8(a.kv_pre + (size_t)b * W + k0, a.kv_splits, a.kv_split_stride, v);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = latent ? fmaf(v[i], v[i], ss) : ss;
  const float tot = block_sum(ss, red);
  if (!on) return;
  T* dst = static_cast<T*>(a.pool) + ((size_t)blk * a.block + pos % a.block) * W + k0;
  float o[8];
  if (latent) {
    const float inv = 1.0f / sqrtf(tot / (float)a.C + a.eps);
    float gm[8];
    gamma8(a.gamma, k0, gm);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = v[i] * inv * gm[i];
  } else {
    const int i0 = (k0 - a.C) / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rope_pair(v[2 * i], v[2 * i + 1], pos, a.inv_freq[i0 + i], a.rope_mscale, &o[2 * i], &o[2 * i + 1]);
  }
  if constexpr (std::is_same<T, float>::value) {
    reinterpret_cast<float4*>(dst)[0] = float4{o[0], o[1], o[2], o[3]};
    reinterpret_cast<float4*>(dst)[1] = float4{o[4], o[5], o[6], o[7]};
  } else {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = (uint32_t)f32_to_bf16(o[2 * i]) | ((uint32_t)f32_to_bf16(o[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(dst) = uint4{u[0], u[1], u[2], u[3]};
  }
}

template <typename T>
__global__ void __launch_bounds__(256) append_rows_vec_kernel(AppendArgs a) {
  __shared__ float red[4];
  append_row_vec<T>(a, blockIdx.x, red);
}

// The cache append of a step and the RMSNorm of its q latent in one launch:
// workgroups b < B append token b's row, the next B normalise token b - B's
// q latent into the packed layout.  The block has the larger of the two
// thread counts; the surplus threads of the other part only join its sums.
template <typename T>
__global__ void __launch_bounds__(1024) append_qnorm_kernel(AppendArgs a, QNormArgs q) {
  __shared__ float red[16];
  const int b = blockIdx.x;
  if (b < a.B) append_row_vec<T>(a, b, red);
  else rmsnorm_pack_row(q.part, q.S, q.split_stride, a.B, q.n, q.stride, q.gamma, q.eps, q.yp,
                        q.yexp, b - a.B, red);
}

// grid (H, ceil(C/128)); thread = one latent column c of head h.  Each W_UK
// element is read (and dequantised) once per chunk of up to 32 tokens whose
// q_nope rows are staged in LDS.
constexpr int kAbsC = 128, kAbsB = 32;

template <typename T>
__global__ void __launch_bounds__(kAbsC) absorb_kernel(AbsorbArgs a) {
  extern __shared__ float qn[];  // [N][kAbsB]: token-minor so one n is a broadcast row
  const int h = blockIdx.x;
  const int c = blockIdx.y * kAbsC + threadIdx.x;
  const int QW = a.N + a.R;
  const int W = a.C + a.R;
  T* out = static_cast<T*>(a.q_abs);
  const int64_t wrow = (int64_t)h * (a.N + a.V);
  const int cc = c < a.C ? c : a.C - 1;
  for (int b0 = 0; b0 < a.B; b0 += kAbsB) {
    const int nb = (a.B - b0) < kAbsB ? (a.B - b0) : kAbsB;
    for (int e = threadIdx.x; e < kAbsB * a.N; e += kAbsC) {
      const int n = e / kAbsB, bb = e - n * kAbsB;
      qn[e] = bb < nb ? a.q[((size_t)(b0 + bb) * a.H + h) * QW + n] : 0.f;
    }
    __syncthreads();
    float acc[kAbsB];
#pragma unroll
    for (int i = 0; i < kAbsB; ++i) acc[i] = 0.f;
    for (int n = 0; n < a.N; ++n) {
      const float w = weight_at(a.kv_b, wrow + n, cc);
      const float* qrow = qn + n * kAbsB;
#pragma unroll
      for (int i = 0; i < kAbsB; ++i) acc[i] = fmaf(w, qrow[i], acc[i]);
    }
    if (c < a.C)
      for (int i = 0; i < nb; ++i) Elem<T>::store(out, ((size_t)(b0 + i) * a.H + h) * W + c, acc[i]);
    __syncthreads();
  }
  if (blockIdx.y == 0) {
    const int half = a.R / 2;
    for (int e = threadIdx.x; e < a.B * half; e += kAbsC) {
      const int bb = e / half, i = e - bb * half;
      const float* qp = a.q + ((size_t)bb * a.H + h) * QW + a.N;
      float ox, oy;
      rope_pair(qp[2 * i], qp[2 * i + 1], a.positions[bb], a.inv_freq[i], a.rope_mscale, &ox, &oy);
      const size_t o = ((size_t)bb * a.H + h) * W + a.C + 2 * i;
      Elem<T>::store(out, o, ox);
      Elem<T>::store(out, o + 1, oy);
    }
  }
}

// 4-bit or Q8_0 W_UK on MFMA: q'[b][h][c] = sum_n W_UK[h][n][c] q_nope[b][h][n].
// grid (H, ceil(C/128), ceil(B/32)), 256 threads.  The workgroup first loads
// its W_UK slice (128 n x 128 c, 16 bytes per row per thread, coalesced) and
// dequantises it into LDS as fp16 transposed to [c][n], so one MFMA operand
// (8 consecutive n of one c) is one 16-byte LDS read.  Wave w then owns
// columns c0..c0+31 (c0 = 128 blockIdx.y + 32 w) for 32 tokens: the token is
// the MFMA M dimension and k-slot j of lane-half hh at step st is n = n0 +
// 64hh + 8st + j on both operands.  Workgroups with blockIdx.y == 0 also
// rotate q_pe of their tokens.  A staging thread's 32 columns of a row are
// one Q8_0 block (d * q, exact in fp32, then rounded to fp16 like the 4-bit
// values); its bytes are only 2-byte aligned, so they are read as 16-bit words.
constexpr int kAbsN = 128, kAbsCols = 128, kAbsPitch = kAbsN + 8;  // LDS row pitch in halfs

template <typename T, bool kQ8>
__global__ void __launch_bounds__(256) absorb_mfma_kernel(AbsorbArgs a) {
  __shared__ _Float16 wt[kAbsCols * kAbsPitch];  // [c][n]
  const int h = blockIdx.x;
  const int b0 = blockIdx.z * 32;
  const int cw0 = blockIdx.y * kAbsCols;
  const int QW = a.N + a.R;
  const int W = a.C + a.R;
  T* out = static_cast<T*>(a.q_abs);
  if (blockIdx.y == 0) {
    const int half = a.R / 2;
    const int nb = (a.B - b0) < 32 ? (a.B - b0) : 32;
    for (int e = threadIdx.x; e < nb * half; e += 256) {
      const int bb = b0 + e / half, i = e % half;
      const float* qp = a.q + ((size_t)bb * a.H + h) * QW + a.N;
      float ox, oy;
      rope_pair(qp[2 * i], qp[2 * i + 1], a.positions[bb], a.inv_freq[i], a.rope_mscale, &ox, &oy);
      const size_t o = ((size_t)bb * a.H + h) * W + a.C + 2 * i;
      Elem<T>::store(out, o, ox);
      Elem<T>::store(out, o + 1, oy);
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int c0 = wave * 32;  // within the workgroup's columns
  const bool wave_on = cw0 + c0 < a.C;
  const int tok = b0 + l32;
  const bool tok_ok = tok < a.B;
  const float* qp = a.q + ((size_t)(tok_ok ? tok : 0) * a.H + h) * QW;
  // q_nope of (token, head) enters the MFMAs times 2^-qe, its largest
  // magnitude brought into binary16's range; the results are multiplied back.
  // The lane's operands of the first 128 n are read here, before the W_UK
  // slice's loads, so both latencies overlap; the scale is formed after them.
  float4 q0[16];  // n = 64 hh + 8 st + (0..3 | 4..7), st < 8
#pragma unroll
  for (int i = 0; i < 16; ++i)
    q0[i] = wave_on && tok_ok ? *reinterpret_cast<const float4*>(qp + 64 * hh + 4 * i)
                              : float4{0.f, 0.f, 0.f, 0.f};
  int qe = 0;
  float qsc = 1.f;
  auto range_scale = [&]() {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      m = fmaxf(fmaxf(m, fmaxf(fabsf(q0[i].x), fabsf(q0[i].y))), fmaxf(fabsf(q0[i].z), fabsf(q0[i].w)));
    if (tok_ok)
      for (int n = kAbsN + 4 * hh; n < a.N; n += 8) {  // the rest of a deeper q_nope
        const float4 v = *reinterpret_cast<const float4*>(qp + n);
        m = fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
      }
    float lo, hi;
    wave_halves(m, &lo, &hi);
    qe = f16_range_exp(fmaxf(lo, hi));
    qsc = pow2f(-qe);
  };
  const int64_t row0 = (int64_t)h * (a.N + a.V);
  const int64_t cols8 = a.kv_b.cols >> 3, cols64 = a.kv_b.cols >> 6;
  const bool tiled = a.kv_b.dtype == MLA_Q4G64_T;
  // staging role: rows 2np, 2np+1 (np = thread % 64), columns 32 cq .. 32 cq + 31
  const int np = threadIdx.x & 63, cq = threadIdx.x >> 6;
  const int cst = cw0 + 32 * cq;
  const bool st_on = cst < a.C;
  f32x16_t acc = f32x16_t{};
  for (int n0 = 0; n0 < a.N; n0 += kAbsN) {
    if (kQ8 && st_on) {
      const uint8_t* kvb = static_cast<const uint8_t*>(a.kv_b.data);
      const int64_t nblk = a.kv_b.cols >> 5;
      float d[2];
      uint16_t qw[2][16];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint16_t* blk = reinterpret_cast<const uint16_t*>(
            kvb + ((row0 + n0 + 2 * np + r) * nblk + (cst >> 5)) * 34);
        d[r] = (float)__builtin_bit_cast(_Float16, blk[0]);
#pragma unroll
        for (int i = 0; i < 16; ++i) qw[r][i] = blk[1 + i];
      }
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const int8_t q0 = (int8_t)(qw[0][c >> 1] >> (8 * (c & 1)));
        const int8_t q1 = (int8_t)(qw[1][c >> 1] >> (8 * (c & 1)));
        const _Float16 pr[2] = {(_Float16)(d[0] * (float)q0), (_Float16)(d[1] * (float)q1)};
        *reinterpret_cast<uint32_t*>(&wt[(32 * cq + c) * kAbsPitch + 2 * np]) =
            __builtin_bit_cast(uint32_t, pr);
      }
    } else if (st_on) {
      uint4 wv[2];
      float sc[2], bi[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int64_t row = row0 + n0 + 2 * np + r;
        int64_t wq, g;  // uint4 index of the 32 columns, index of their group's scale
        if (tiled) {  // 2 KB block per (32-row tile, 128 columns); see the GEMM body
          const int64_t blk = (row >> 5) * (a.kv_b.cols >> 7) + (cst >> 7);
          const int64_t L = (row & 31) + 32 * ((cst >> 6) & 1);
          wq = blk * 128 + ((cst >> 5) & 1) * 64 + L;
          g = blk * 64 + L;
        } else {
          wq = (row * cols8 + (cst >> 3)) >> 2;
          g = row * cols64 + (cst >> 6);
        }
        wv[r] = static_cast<const uint4*>(a.kv_b.data)[wq];
        sc[r] = bf16_to_f32(a.kv_b.scales[g]);
        bi[r] = bf16_to_f32(a.kv_b.biases[g]);
      }
      const uint32_t w0[4] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w};
      const uint32_t w1[4] = {wv[1].x, wv[1].y, wv[1].z, wv[1].w};
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        const float v0 = fmaf((float)((w0[c >> 3] >> (4 * (c & 7))) & 15u), sc[0], bi[0]);
        const float v1 = fmaf((float)((w1[c >> 3] >> (4 * (c & 7))) & 15u), sc[1], bi[1]);
        const _Float16 pr[2] = {(_Float16)v0, (_Float16)v1};
        *reinterpret_cast<uint32_t*>(&wt[(32 * cq + c) * kAbsPitch + 2 * np]) =
            __builtin_bit_cast(uint32_t, pr);
      }
    }
    if (n0 == 0 && wave_on) range_scale();
    __syncthreads();
    if (wave_on) {
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int nb = 64 * hh + 8 * st;
        f16x8_t qa = f16x8_t{};
        if (tok_ok) {
          const float4 x0 = n0 == 0 ? q0[2 * st] : *reinterpret_cast<const float4*>(qp + n0 + nb);
          const float4 x1 = n0 == 0 ? q0[2 * st + 1] : *reinterpret_cast<const float4*>(qp + n0 + nb + 4);
          qa = f16x8_t{(_Float16)(x0.x * qsc), (_Float16)(x0.y * qsc), (_Float16)(x0.z * qsc),
                       (_Float16)(x0.w * qsc), (_Float16)(x1.x * qsc), (_Float16)(x1.y * qsc),
                       (_Float16)(x1.z * qsc), (_Float16)(x1.w * qsc)};
        }
        const f16x8_t wb = *reinterpret_cast<const f16x8_t*>(&wt[(c0 + l32) * kAbsPitch + nb]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa, wb, acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!wave_on) return;
  const int c = cw0 + c0 + l32;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int t = b0 + (j >> 2) * 8 + hh * 4 + (j & 3);
    const int et = __shfl(qe, t - b0, 64);  // token t's exponent, from lane t - b0
    if (t < a.B) Elem<T>::store(out, ((size_t)t * a.H + h) * W + c, ldexpf(acc[j], et));
  }
}

// ---------------------------------------------------------------------------
// q_b and the absorb of one head, for 4-bit q_b and W_UK with q_nope 128, q_pe
// 64, a latent of at most 512 and a q LoRA rank of at most 1536: q of the head
// never leaves LDS, and the q latent of a token tile is read twice per head
// instead of once per 32 rows of q_b.  grid (H, 2 x token tiles of 32), 1024
// threads, 160 KB of LDS.  Each head has two workgroups: role A (even
// blockIdx.y) computes q_nope (q_b's first four 32-row tiles) and the absorb,
// role B (odd) q_pe (the last two tiles) and its rotation.  Both first copy
// the token tile's packed q latent into LDS by LDS DMA, alone, so q_b starts
// as soon as it lands while the weights stream in.  LDS, role A:
//   [0, 96 KB)        the packed q latent, then
//   [0, 64 KB)        the 16 waves' partial q_b tiles; from the absorb on
//   [0, 128 KB)       W_UK of the head, fp16 [c][n]: 256 bytes per column, its
//                     16-byte chunk k (n = 8k .. 8k + 7) at chunk k ^ (c % 16)
//   [128, 136 KB)     x_exp of the tile's tokens, then q_nope times 2^-qe in
//                     fp16, MFMA layout [step][lane][8]
//   [144, 160 KB)     q_nope fp32 [token][128] (word 0 of a token's row later
//                     holds its exponent)
// role B: the packed q latent, the partial tiles at [0, 64 KB), x_exp at 128
// KB, q_pe fp32 [token][64] at [64, 72 KB).
// Wave w of role A owns rows 32 (w % 4) .. +31 of q_nope and K quarter w / 4
// (of B: rows 128 + 32 (w % 2) and K eighth w / 2), each unit multiplied as in
// the GEMM body; a tile's K parts are added in K order and multiplied by
// 2^x_exp, by all threads (4 or 2 outputs each).  Role A then finds each token's q_nope exponent (as the absorb
// kernel does) and packs the scaled fp16 operand on waves 0-3 while every
// thread dequantises its share of W_UK (rows 2 lane and 2 lane + 1 of columns
// 32 wave .. +31, loaded with the q_b weights): one byte of each row (two
// columns) becomes two fp16 pairs (row 2 lane, row 2 lane + 1) with one byte
// permute, the nibble-under-exponent trick of the GEMM and one packed fma per
// pair.  Last, wave w multiplies columns 32w .. 32w + 31 for the 32 tokens
// with the W_UK columns as the M operand, so each lane holds four consecutive
// columns of one token per MFMA row group and stores them in one 8- or 16-byte
// write.  Role B rotates one (token, pair) per thread and stores it.
// ---------------------------------------------------------------------------
constexpr int kQaRows = 192, kQaMaxUnits = 12, kQaMaxC = 512;
constexpr uint32_t kQaPe = 65536u;                     // role B: q_pe fp32 [32][64]
constexpr uint32_t kQaAop = (uint32_t)kQaMaxC * 256u;  // the absorb's q operand (8 KB)
constexpr uint32_t kQaQf = kQaAop + 16384u;            // q_nope fp32 [32][128]
constexpr uint32_t kQaLds = kQaQf + 32u * 128u * 4u;   // 163840

// Byte offset in the W_UK area of the fp16 pair (n = 2np, 2np + 1) of column c.
__device__ __forceinline__ uint32_t qa_wt_off(uint32_t c, uint32_t np) {
  return c * 256u + (((np >> 2) ^ (c & 15u)) << 4) + ((np & 3u) << 2);
}

template <typename T>
__global__ void __launch_bounds__(1024) qb_absorb_kernel(GemmArgs g, AbsorbArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  MLA_LDS char* L = (MLA_LDS char*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)L;
  const int h = blockIdx.x, tile = blockIdx.y >> 1, b0 = tile * 32;
  const bool roleA = (blockIdx.y & 1) == 0;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int units = g.K >> 7;
  const int W = a.C + a.R;
  // this wave's q_b rows (of the head's 192) and K part
  const int nparts = roleA ? 4 : 8;
  const int t = roleA ? (wave & 3) : (wave & 1);
  const int part = roleA ? (wave >> 2) : (wave >> 1);
  const int per = (units + nparts - 1) / nparts;  // at most 3 (A) or 2 (B)
  const int ub = part * per;
  const int nu = units - ub < 0 ? 0 : (units - ub < per ? units - ub : per);
  const int row0 = roleA ? 32 * t : 128 + 32 * t;

  // role B's rope operands: token tid / 32, pair tid % 32
  int pos = 0;
  float invf = 0.f;
  if (!roleA) {
    const int bb = b0 + (tid >> 5);
    pos = a.positions[bb < a.B ? bb : a.B - 1];
    invf = a.inv_freq[tid & 31];
  }
  // The tile's packed activations are one contiguous run of units x 8 KB; copy
  // c (1 KB, c = wave + 16 k) lands at LDS byte 1024 c (M0 + 16 * lane).
  {
    const char* src = reinterpret_cast<const char*>(g.xp) + (size_t)tile * units * 8192;
    for (int c = wave; c < units * 8; c += 16) {
      const uint32_t m0 = lds0 + (uint32_t)c * 1024u, off = (uint32_t)c * 1024u + 16u * lane;
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                   :
                   : "v"(off), "s"(src), "s"(m0)
                   : "memory");
    }
  }
  // The copies first have the memory system to themselves.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (wave == 15 && lane < 32) {
    const int bb = b0 + lane;
    *(MLA_LDS int*)(L + kQaAop + 4u * lane) = bb < a.B ? g.x_exp[bb] : 0;
  }
  __syncthreads();  // the activations and x_exp are in LDS

  // q_b weights of the wave's units (offsets as in the GEMM body; a unit past
  // the wave's range re-reads its last one, or unit 0, and is never used)
  uint4 wq[3][2];
  uint16_t sc[3], bi[3];
  {
    const uint32_t wrow = (uint32_t)(h * kQaRows + row0 + l32);
    const bool tiled = g.w.dtype == MLA_Q4G64_T;
    const uint32_t tblk = (wrow >> 5) * (uint32_t)(g.w.cols >> 7), tlane = (wrow & 31u) + 32u * hh;
    const uint32_t woff = tiled ? tblk * 2048u + 16u * tlane : wrow * (uint32_t)(g.w.cols >> 1) + 32u * hh;
    const uint32_t soff = tiled ? tblk * 128u + 2u * tlane : wrow * (uint32_t)(g.w.cols >> 6) * 2u + 2u * hh;
    const uint32_t wstep = tiled ? 2048u : 64u, whalf = tiled ? 1024u : 16u, sstep = tiled ? 128u : 4u;
    const char* wbase = static_cast<const char*>(g.w.data);
    const char* sbase = reinterpret_cast<const char*>(g.w.scales);
    const char* bbase = reinterpret_cast<const char*>(g.w.biases);
    const int ulast = nu > 0 ? ub + nu - 1 : 0;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (!roleA && i == 2) break;
      const uint32_t uu = (uint32_t)(ub + i < ulast ? ub + i : ulast);
      sc[i] = *reinterpret_cast<const uint16_t*>(sbase + soff + sstep * uu);
      bi[i] = *reinterpret_cast<const uint16_t*>(bbase + soff + sstep * uu);
      wq[i][0] = *reinterpret_cast<const uint4*>(wbase + woff + wstep * uu);
      wq[i][1] = *reinterpret_cast<const uint4*>(wbase + woff + wstep * uu + whalf);
    }
  }
  // role A: W_UK, thread (np = lane, cq = wave) owns rows 2np, 2np + 1 of
  // columns 32 cq .. 32 cq + 31 (a wave past the latent re-reads the last ones)
  uint4 wv[2];
  uint16_t ws[2], wb[2];
  if (roleA) {
    const int cst = 32 * wave < a.C ? 32 * wave : a.C - 32;
    const int64_t wrow0 = (int64_t)h * (a.N + a.V);
    const bool tiled = a.kv_b.dtype == MLA_Q4G64_T;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int64_t row = wrow0 + 2 * lane + rr;
      int64_t wqi, gi;  // uint4 index of the 32 columns, index of their group's scale
      if (tiled) {
        const int64_t blk = (row >> 5) * (a.kv_b.cols >> 7) + (cst >> 7);
        const int64_t Ln = (row & 31) + 32 * ((cst >> 6) & 1);
        wqi = blk * 128 + ((cst >> 5) & 1) * 64 + Ln;
        gi = blk * 64 + Ln;
      } else {
        wqi = (row * (a.kv_b.cols >> 3) + (cst >> 3)) >> 2;
        gi = row * (a.kv_b.cols >> 6) + (cst >> 6);
      }
      ws[rr] = a.kv_b.scales[gi];
      wb[rr] = a.kv_b.biases[gi];
      wv[rr] = static_cast<const uint4*>(a.kv_b.data)[wqi];
    }
  }

  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i >= nu) break;
    const uint32_t ubase = (uint32_t)(ub + i) * 8192u + 16u * lane;
    // the empty asm keeps the conversions here, so that the compiler does
    // not wait for the scale loads right after issuing them
    uint32_t sr = sc[i], br = bi[i];
    asm volatile("" : "+v"(sr), "+v"(br));
    const _Float16 sh = (_Float16)bf16_to_f32((uint16_t)sr), bh = (_Float16)bf16_to_f32((uint16_t)br);
    const f16x2_t s2 = {sh, sh}, b2 = {bh, bh};
    const uint32_t words[8] = {wq[i][0].x, wq[i][0].y, wq[i][0].z, wq[i][0].w,
                               wq[i][1].x, wq[i][1].y, wq[i][1].z, wq[i][1].w};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const f16x8_t x = *(const MLA_LDS f16x8_t*)(L + ubase + 1024u * st);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, dequant8(words[st], s2, b2), acc, 0, 0, 0);
    }
  }
  __syncthreads();  // every product done: the activations are no longer read
  MLA_LDS float* red = (MLA_LDS float*)L;
  const int ntiles = roleA ? 4 : 2;
#pragma unroll
  for (int j = 0; j < 16; ++j) red[((part * ntiles + t) * 16 + j) * 64 + lane] = acc[j];
  __syncthreads();  // partial tiles written
  // q of the tile's tokens, K parts added in order, fp32: role A q_nope
  // [token][128] at kQaQf, role B q_pe [token][64] at kQaPe.  Output o of the
  // role's ntiles x 1024: tile o / 1024, then the MFMA tile's (j, lane).
  const MLA_LDS int* xe = (const MLA_LDS int*)(L + kQaAop);
  auto put_q = [&](int o, float v) {
    const int tt = o >> 10, ln = o & 63, j = (o >> 6) & 15;
    const int tok = (j >> 2) * 8 + (ln >> 5) * 4 + (j & 3);
    MLA_LDS float* q = roleA ? (MLA_LDS float*)(L + kQaQf) : (MLA_LDS float*)(L + kQaPe);
    const int pitch = roleA ? 128 : 64;
    q[tok * pitch + 32 * tt + (ln & 31)] = b0 + tok < a.B ? ldexpf(v, xe[tok]) : 0.f;
  };
  auto slot = [&](int p, int o) {  // part p's value of output o
    return red[(((p * ntiles + (o >> 10)) * 16 + ((o >> 6) & 15)) * 64) + (o & 63)];
  };
  if (roleA) {
    float v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 4; ++p) v[k][p] = slot(p, tid + 1024 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) put_q(tid + 1024 * k, ((v[k][0] + v[k][1]) + v[k][2]) + v[k][3]);
  } else {
    float v[2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int p = 0; p < 8; ++p) v[k][p] = slot(p, tid + 1024 * k);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float x = v[k][0];
#pragma unroll
      for (int p = 1; p < 8; ++p) x += v[k][p];
      put_q(tid + 1024 * k, x);
    }
  }
  __syncthreads();  // q complete; the activation and partial areas are free

  if (!roleA) {
    const int tt = tid >> 5, i = tid & 31, bb = b0 + tt;
    if (bb >= a.B) return;
    const float x = ((const MLA_LDS float*)(L + kQaPe))[tt * 64 + 2 * i];
    const float y = ((const MLA_LDS float*)(L + kQaPe))[tt * 64 + 2 * i + 1];
    float ox, oy;
    rope_pair(x, y, pos, invf, a.rope_mscale, &ox, &oy);
    char* dst = static_cast<char*>(a.q_abs) + (((size_t)bb * a.H + h) * W + a.C + 2 * i) * sizeof(T);
    if constexpr (std::is_same<T, float>::value)
      *reinterpret_cast<float2*>(dst) = float2{ox, oy};
    else
      *reinterpret_cast<uint32_t*>(dst) = f32_to_bf16(ox) | ((uint32_t)f32_to_bf16(oy) << 16);
    return;
  }

  if (wave < 4) {
    // token tt's q_nope n = 16 gq .. 16 gq + 15; the 8 threads of a token
    // are 8 consecutive lanes
    const int tt = tid >> 3, gq = tid & 7;
    const MLA_LDS f32x4_t* row = (const MLA_LDS f32x4_t*)(L + kQaQf + (uint32_t)(tt * 128 + 16 * gq) * 4u);
    f32x4_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = row[e];
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m = fmaxf(fmaxf(m, fmaxf(fabsf(v[e].x), fabsf(v[e].y))), fmaxf(fabsf(v[e].z), fabsf(v[e].w)));
    m = fmaxf(m, __shfl_xor(m, 4));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 1));
    const int qe = f16_range_exp(m);
    const float qsc = pow2f(-qe);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x4_t x0 = v[2 * e], x1 = v[2 * e + 1];
      const f16x8_t qa = {(_Float16)(x0.x * qsc), (_Float16)(x0.y * qsc), (_Float16)(x0.z * qsc),
                          (_Float16)(x0.w * qsc), (_Float16)(x1.x * qsc), (_Float16)(x1.y * qsc),
                          (_Float16)(x1.z * qsc), (_Float16)(x1.w * qsc)};
      const int st = 2 * (gq & 3) + e, hp = gq >> 2;  // n = 64 hp + 8 st + (0..7)
      *(MLA_LDS f16x8_t*)(L + kQaAop + (uint32_t)((st * 64 + 32 * hp + tt) * 16)) = qa;
    }
    // this thread alone read word 0 of the row, above
    if (gq == 0) *(MLA_LDS int*)(L + kQaQf + (uint32_t)(tt * 128) * 4u) = qe;
  }
  if (32 * wave < a.C) {
    const f16x2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    const f16x2_t k64 = {(_Float16)64.f, (_Float16)64.f};
    uint32_t r0 = ws[0], r1 = ws[1], r2 = wb[0], r3 = wb[1];
    asm volatile("" : "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3));
    const f16x2_t s2 = {(_Float16)bf16_to_f32((uint16_t)r0), (_Float16)bf16_to_f32((uint16_t)r1)};
    const f16x2_t b2 = {(_Float16)bf16_to_f32((uint16_t)r2), (_Float16)bf16_to_f32((uint16_t)r3)};
    const uint32_t w0[4] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w};
    const uint32_t w1[4] = {wv[1].x, wv[1].y, wv[1].z, wv[1].w};
#pragma unroll
    for (int kw = 0; kw < 4; ++kw)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        // bytes: row 2np's byte bb twice, then row 2np + 1's twice
        const uint32_t sel = (uint32_t)bb * 0x0101u + (uint32_t)(4 + bb) * 0x01010000u;
        const uint32_t p = __builtin_amdgcn_perm(w1[kw], w0[kw], sel);
        const f16x2_t e0 = __builtin_bit_cast(f16x2_t, and_or(p, 0x000F000Fu, 0x64006400u)) - k1024;
        const f16x2_t e1 = __builtin_bit_cast(f16x2_t, and_or(p, 0x00F000F0u, 0x54005400u)) - k64;
        const uint32_t c = (uint32_t)(32 * wave + 8 * kw + 2 * bb);
        *(MLA_LDS uint32_t*)(L + qa_wt_off(c, (uint32_t)lane)) =
            __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(e0, s2, b2));
        *(MLA_LDS uint32_t*)(L + qa_wt_off(c + 1u, (uint32_t)lane)) =
            __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(e1, s2, b2));
      }
  }
  __syncthreads();  // W_UK, the q operand and the exponents in LDS

  if (32 * wave >= a.C) return;
  // W_UK rows are the M operand and the tokens N, so a lane ends with 16
  // columns of its token l32: 32 wave + 8 (j / 4) + 4 hh + (j % 4).
  const uint32_t c = (uint32_t)(32 * wave + l32);
  acc = f32x16_t{};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const f16x8_t wa = *(const MLA_LDS f16x8_t*)(L + c * 256u + ((((uint32_t)(8 * hh + st)) ^ (c & 15u)) << 4));
    const f16x8_t qb8 = *(const MLA_LDS f16x8_t*)(L + kQaAop + (uint32_t)((st * 64 + lane) * 16));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa, qb8, acc, 0, 0, 0);
  }
  const int bb = b0 + l32;
  if (bb >= a.B) return;
  const int qe = *(const MLA_LDS int*)(L + kQaQf + (uint32_t)(l32 * 128) * 4u);
#pragma unroll
  for (int jg = 0; jg < 4; ++jg) {
    const float v0 = ldexpf(acc[4 * jg], qe), v1 = ldexpf(acc[4 * jg + 1], qe);
    const float v2 = ldexpf(acc[4 * jg + 2], qe), v3 = ldexpf(acc[4 * jg + 3], qe);
    char* dst = static_cast<char*>(a.q_abs) +
                (((size_t)bb * a.H + h) * W + 32 * wave + 8 * jg + 4 * hh) * sizeof(T);
    if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v0, v1, v2, v3};
    } else {
      const uint32_t lo = f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
      const uint32_t hi = f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16);
      *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
    }
  }
}

// ---------------------------------------------------------------------------
// The attention merge and W_UV of one head in two workgroups (the decode layer
// with more than one split, the MFMA kernel's fp16 partials, latent 512, 128
// heads, 4-bit W_UV of 128 rows per head feeding o_proj on the MFMA path).
// grid (128 heads, 2 x token tiles of 32: each tile's two halves of 16
// queries), 1024 threads, 96 KB of LDS:
//   [0, 32 KB)    the tile's merged v_combine of the head in fp16, in the
//                 packed MFMA layout W_UV reads (unit, step, lane, 8 values);
//                 the other half's 16 tokens are zeros
//   [32, 96 KB)   the 16 waves' W_UV partial tiles
// Wave w merges query b0 + 16 half + w exactly as the merge kernel does for
// one (query, head), also where that kernel gives a query of more
// than 8 splits W = 2 or 4 waves per head: here one wave forms the W sums in
// turn and adds them in the same order, so v_combine, lse and the fp16 values
// carry the same bits.  Then wave w = 4t + u multiplies row tile t of the
// head's W_UV by unit u of the packed values (its weights loaded before the
// merge), and the four unit sums are added in unit order, as the GEMM with one
// unit per wave adds its waves' tiles; the half's results go to o_proj's
// packed input (a token's row of the product does not depend on the others).
// Two workgroups per head halve the partial rows each one reads, which bound
// the merge; W_UV's 32 KB of weights per head are read twice.
// ---------------------------------------------------------------------------
constexpr uint32_t kMuvRed = 32768u, kMuvLds = kMuvRed + 16u * 4096u;

__global__ void __launch_bounds__(1024) merge_uv_kernel(AttnArgs a, GemmArgs g) {
  constexpr int kH = 128, kC = 512;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  MLA_LDS char* L = (MLA_LDS char*)smem;
  const int h = blockIdx.x, b0 = (blockIdx.y >> 1) * 32, half = blockIdx.y & 1;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = wave >> 2, u = wave & 3;
  const int tok = 16 * half + wave, b = b0 + tok;
  // the query's length (and the device plan's slots) first: loads complete in
  // issue order, so these do not wait behind the weights
  int len = 0, fr = 0;
  const int rows = a.auto_slots > 0 ? a.part_first[a.B] : a.split_rows;
  if (b < a.B) {
    len = a.seq_lens[b];
    fr = a.auto_slots > 0 ? a.part_first[b] : b * a.num_splits;
  }

  // W_UV weights of row tile t, unit u (offsets as in the GEMM body)
  uint4 wq[2];
  uint16_t sc, bi;
  {
    const uint32_t wrow = (uint32_t)(g.w_row0 + (int64_t)h * g.w_zrows + 32 * t + l32);
    const bool tiled = g.w.dtype == MLA_Q4G64_T;
    const uint32_t tblk = (wrow >> 5) * (uint32_t)(g.w.cols >> 7), tlane = (wrow & 31u) + 32u * hh;
    const uint32_t woff = tiled ? tblk * 2048u + 16u * tlane : wrow * (uint32_t)(g.w.cols >> 1) + 32u * hh;
    const uint32_t soff = tiled ? tblk * 128u + 2u * tlane : wrow * (uint32_t)(g.w.cols >> 6) * 2u + 2u * hh;
    const uint32_t wo = woff + (tiled ? 2048u : 64u) * u, so = soff + (tiled ? 128u : 4u) * u;
    const char* wbase = static_cast<const char*>(g.w.data);
    wq[0] = *reinterpret_cast<const uint4*>(wbase + wo);
    wq[1] = *reinterpret_cast<const uint4*>(wbase + wo + (tiled ? 1024u : 16u));
    sc = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(g.w.scales) + so);
    bi = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(g.w.biases) + so);
  }

  // this lane's 8 latent columns c = 8 lane sit in unit lane / 16, step lane % 8,
  // lane half (lane / 8) % 2 of the packed layout
  const uint32_t pk_off = (uint32_t)((((lane >> 4) * 8 + (lane & 7)) * 64 + 32 * ((lane >> 3) & 1)) * 16);
  // the other half's tokens enter W_UV as zeros
  *(MLA_LDS f16x8_t*)(L + pk_off + 16u * (16 * (1 - half) + wave)) = f16x8_t{};
  // Two memory round trips: the length, then the query's split lse,
  // exponents and first 8 partial rows.
  MLA_LDS f16x8_t* pk = (MLA_LDS f16x8_t*)(L + pk_off + 16u * tok);
  if (b >= a.B) {
    *pk = f16x8_t{};
  } else {
    len = len < a.max_len ? len : a.max_len;
    const int S = __builtin_amdgcn_readfirstlane(len > 0 ? (len + rows - 1) / rows : 0);
    const size_t first = (size_t)__builtin_amdgcn_readfirstlane(S > 0 ? fr : 0);
    const float ls0 = lane < S ? a.part_lse[(first + lane) * kH + h] : -INFINITY;
    const float ex0 = lane < S ? a.part_exp[(first + lane) * kH + h] : 0.f;
    const _Float16* src = a.part_oh + (first * kH + h) * kC + lane * 8;
    const size_t sstride = (size_t)kH * kC;
    f16x8_t v[8];  // batch 0, then the later batches in turn
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = j < S ? j : (S > 0 ? S - 1 : 0);  // uniform
      v[j] = *reinterpret_cast<const f16x8_t*>(src + (size_t)sj * sstride);
    }
    const int nb = (S + 7) / 8;
    const int W = nb <= 1 ? 1 : (nb == 2 ? 2 : 4);  // the merge kernel's waves per head
    const float* lse_s = a.part_lse + first * kH + h;
    const float* exp_s = a.part_exp + first * kH + h;
    float m = ls0;
    bool nan_lse = ls0 != ls0;
    for (int s = 64 + lane; s < S; s += 64) {
      const float l = lse_s[(size_t)s * kH];
      m = fmaxf(m, l);
      nan_lse |= l != l;
    }
    m = wave_max(m);
    if (__ballot(nan_lse) != 0) m = NAN;
    const bool empty = m == -INFINITY;
    float wsum = empty ? 1.f : expf(ls0 - m);
    if (!empty)
      for (int s = 64 + lane; s < S; s += 64) wsum += expf(lse_s[(size_t)s * kH] - m);
    wsum = wave_sum(wsum);
    const float inv = 1.0f / wsum;

    f32x4_t lo_t{0.f, 0.f, 0.f, 0.f}, hi_t{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < W && !empty; ++w) {
      f32x4_t lo{0.f, 0.f, 0.f, 0.f}, hi{0.f, 0.f, 0.f, 0.f};
      int chunk = -1;
      float wl = 0.f;
      for (int jb = w; jb < nb; jb += W) {
        if (jb > 0) {  // batch 0 came with the lse and is visited first
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int sj = 8 * jb + j < S ? 8 * jb + j : S - 1;  // uniform
            v[j] = *reinterpret_cast<const f16x8_t*>(src + (size_t)sj * sstride);
          }
        }
        const int s0 = 8 * jb;
        if (s0 / 64 != chunk) {
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
          const int sj = s0 + j;
          const float wj =
              sj < S ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), sj & 63)) : 0.f;
          const f32x4_t l4 = lo + wj * f32x4_t{(float)v[j][0], (float)v[j][1], (float)v[j][2], (float)v[j][3]};
          const f32x4_t h4 = hi + wj * f32x4_t{(float)v[j][4], (float)v[j][5], (float)v[j][6], (float)v[j][7]};
          const bool use = wj != 0.f;
          lo = use ? l4 : lo;
          hi = use ? h4 : hi;
        }
      }
      if (w == 0) {
        lo_t = lo;
        hi_t = hi;
      } else {
        lo_t = lo_t + lo;
        hi_t = hi_t + hi;
      }
    }
    float* dst = a.v_combine + ((size_t)b * kH + h) * kC + lane * 8;
    if (empty) {
      lo_t = f32x4_t{0.f, 0.f, 0.f, 0.f};
      hi_t = lo_t;
      if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = -INFINITY;
    } else {
      lo_t = lo_t * inv;
      hi_t = hi_t * inv;
      if (a.lse && lane == 0) a.lse[(size_t)b * kH + h] = m + logf(wsum);
    }
    *reinterpret_cast<f32x4_t*>(dst) = lo_t;
    *reinterpret_cast<f32x4_t*>(dst + 4) = hi_t;
    *pk = f16x8_t{(_Float16)lo_t[0], (_Float16)hi_t[0], (_Float16)lo_t[1], (_Float16)hi_t[1],
                  (_Float16)lo_t[2], (_Float16)hi_t[2], (_Float16)lo_t[3], (_Float16)hi_t[3]};
  }
  __syncthreads();  // the tile's packed v_combine is in LDS

  uint32_t sr = sc, br = bi;
  asm volatile("" : "+v"(sr), "+v"(br));
  const _Float16 sh = (_Float16)bf16_to_f32((uint16_t)sr), bh = (_Float16)bf16_to_f32((uint16_t)br);
  const f16x2_t s2 = {sh, sh}, b2 = {bh, bh};
  const uint32_t words[8] = {wq[0].x, wq[0].y, wq[0].z, wq[0].w, wq[1].x, wq[1].y, wq[1].z, wq[1].w};
  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const f16x8_t x = *(const MLA_LDS f16x8_t*)(L + (uint32_t)(((u * 8 + st) * 64 + lane) * 16));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, dequant8(words[st], s2, b2), acc, 0, 0, 0);
  }
  MLA_LDS float* red = (MLA_LDS float*)(L + kMuvRed);
#pragma unroll
  for (int j = 0; j < 16; ++j) red[((t * 4 + u) * 16 + j) * 64 + lane] = acc[j];
  __syncthreads();
  // Thread e < 256 adds the unit sums (in unit order, from 0) of rows 8 og ..
  // 8 og + 7 of the half's token tl and writes them as one 16-byte chunk of
  // o_proj's packed input (pair order k0 k4 k1 k5 k2 k6 k3 k7).
  if (tid < 256) {
    const int tl = 16 * half + (tid >> 4), og = tid & 15, tk = b0 + tl;
    if (tk < g.B) {
      const int tt = og >> 2, ln0 = 8 * (og & 3) + 32 * ((tl >> 2) & 1);
      const int j = (tl >> 3) * 4 + (tl & 3);
      f32x4_t lo{0.f, 0.f, 0.f, 0.f}, hi{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const MLA_LDS f32x4_t* rp = (const MLA_LDS f32x4_t*)(red + ((tt * 4 + uu) * 16 + j) * 64 + ln0);
        lo = lo + rp[0];
        hi = hi + rp[1];
      }
      const f16x8_t hv = {(_Float16)lo[0], (_Float16)hi[0], (_Float16)lo[1], (_Float16)hi[1],
                          (_Float16)lo[2], (_Float16)hi[2], (_Float16)lo[3], (_Float16)hi[3]};
      *reinterpret_cast<f16x8_t*>(g.yp + packed_index(0, tk, (int64_t)h * g.y_z + 32 * tt + 8 * (og & 3),
                                                      g.B, g.yp_K)) = hv;
    }
  }
}

}  // namespace

namespace {
// One 2 KB block of MLA_Q4G64_T per workgroup of 64 threads: thread L copies
// row 32 t + L % 32's two 16-byte pieces of columns 128 u + 64 (L / 32) ..
// +63 and that group's scale and bias.
__global__ void __launch_bounds__(64) repack_q4_kernel(WeightView w, uint8_t* od, uint16_t* osc,
                                                        uint16_t* obi) {
  const int64_t Un = w.cols >> 7, blk = blockIdx.x;
  const int64_t t = blk / Un, u = blk - t * Un;
  const int L = threadIdx.x;
  const int64_t row = 32 * t + (L & 31), g = row * (w.cols >> 6) + 2 * u + (L >> 5);
  const uint8_t* src = static_cast<const uint8_t*>(w.data) + row * (w.cols >> 1) + 64 * u + 32 * (L >> 5);
  uint8_t* dst = od + blk * 2048 + 16 * L;
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  *reinterpret_cast<uint4*>(dst + 1024) = *reinterpret_cast<const uint4*>(src + 16);
  osc[blk * 64 + L] = w.scales[g];
  obi[blk * 64 + L] = w.biases[g];
}
}  // namespace

hipError_t launch_repack_q4(const WeightView& src, void* data, uint16_t* scales, uint16_t* biases,
                            hipStream_t s) {
  if (src.dtype != MLA_Q4G64 || src.rows % 32 != 0 || src.cols % 128 != 0)
    return hipErrorInvalidValue;
  const int64_t blocks = (src.rows / 32) * (src.cols / 128);
  if (blocks <= 0) return hipSuccess;
  if (blocks > (1ll << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_q4_kernel, dim3((unsigned)blocks), dim3(64), 0, s, src,
                     static_cast<uint8_t*>(data), scales, biases);
  return hipGetLastError();
}

namespace {
constexpr int kMaxU = 16;

hipError_t launch_q4(const GemmArgs& a, int U, int nw, int S, hipStream_t s) {
  dim3 grid((a.O + 31) / 32, (a.B + 31) / 32, a.Z * S);
  const size_t lds = (size_t)nw * 16 * 64 * sizeof(float);
  if (a.w.dtype == MLA_Q8_0) {
    switch (U) {
      case 1: hipLaunchKernelGGL(gemm_q8_mfma_kernel<1>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
      case 2: hipLaunchKernelGGL(gemm_q8_mfma_kernel<2>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
      case 4: hipLaunchKernelGGL(gemm_q8_mfma_kernel<4>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
      case 8: hipLaunchKernelGGL(gemm_q8_mfma_kernel<8>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
      default: hipLaunchKernelGGL(gemm_q8_mfma_kernel<16>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
    }
    return hipGetLastError();
  }
  switch (U) {
    case 1: hipLaunchKernelGGL(gemm_q4_mfma_kernel<1>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
    case 2: hipLaunchKernelGGL(gemm_q4_mfma_kernel<2>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
    case 4: hipLaunchKernelGGL(gemm_q4_mfma_kernel<4>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
    case 8: hipLaunchKernelGGL(gemm_q4_mfma_kernel<8>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
    default: hipLaunchKernelGGL(gemm_q4_mfma_kernel<16>, grid, dim3(nw * 64), lds, s, a, nw, S); break;
  }
  return hipGetLastError();
}
}  // namespace

bool gemm_mfma_ok(const GemmArgs& a) {
  // 32-bit byte offsets inside the kernel: weights and packed activations under 2 GiB
  const bool q8 = a.w.dtype == MLA_Q8_0;
  const int64_t wbytes = q8 ? (int64_t)a.w.rows * (a.w.cols / 32) * 34 : (int64_t)a.w.rows * a.w.cols / 2;
  const int64_t xbytes = (int64_t)packed_bytes(a.Z, a.B, a.K);
  // Q8_0 blocks are read with aligned dword loads from a 4-byte aligned base
  if (q8 && (reinterpret_cast<uintptr_t>(a.w.data) & 3) != 0) return false;
  const bool tiled = a.w.dtype == MLA_Q4G64_T;
  return (a.w.dtype == MLA_Q4G64 || tiled || q8) && a.K > 0 && (a.K % 128) == 0 &&
         (a.w.cols % (q8 ? 32 : tiled ? 128 : 64)) == 0 && (!tiled || a.w.rows % 32 == 0) &&
         a.K <= a.w.cols && (a.K / 128) <= kQ4MaxWaves * kMaxU && wbytes < (1ll << 31) &&
         xbytes < (1ll << 31);
}

int gemm_max_splits(int64_t K) {
  const int64_t units = (K + 127) / 128;
  const int64_t s = (units + 7) / 8;
  return (int)(s < 1 ? 1 : (s > kMaxKSplits ? kMaxKSplits : s));
}

namespace {
// Shape of an MFMA-path launch over `units` 128-k units and `tiles` output
// tiles: U units per wave, nw waves, S K splits.  With few tiles K is spread
// over workgroups (the consumer adds the S partial sums).
void q4_shape(int units, int64_t tiles, int max_splits, bool packed_out, int* U, int* nw, int* S) {
  *U = 1;
  *S = 1;
  if (max_splits > kMaxKSplits) max_splits = kMaxKSplits;
  if (tiles >= 128 || max_splits <= 1 || packed_out) {
    while ((units + *U - 1) / *U > kQ4MaxWaves) *U *= 2;
    *nw = (units + *U - 1) / *U;
  } else {
    *nw = units < 8 ? units : 8;
    *S = (units + *nw - 1) / *nw;
    while (*S > max_splits) {
      *U *= 2;
      *S = (units + *nw * *U - 1) / (*nw * *U);
    }
  }
}

hipError_t launch_pair(const GemmArgs& a, const GemmArgs& b, int tiles_a, int tiles, int U, int nw,
                       int S, hipStream_t s) {
  constexpr bool kQ8 = false;  // kv_a and q_a take the 4-bit format only
  dim3 grid(tiles, (a.B + 31) / 32, S);
  const size_t lds = (size_t)nw * 16 * 64 * sizeof(float);
  const dim3 blk(nw * 64);
  switch (U) {
    case 1: hipLaunchKernelGGL((gemm_pair_mfma_kernel<1, kQ8>), grid, blk, lds, s, a, b, tiles_a, nw, S); break;
    case 2: hipLaunchKernelGGL((gemm_pair_mfma_kernel<2, kQ8>), grid, blk, lds, s, a, b, tiles_a, nw, S); break;
    case 4: hipLaunchKernelGGL((gemm_pair_mfma_kernel<4, kQ8>), grid, blk, lds, s, a, b, tiles_a, nw, S); break;
    case 8: hipLaunchKernelGGL((gemm_pair_mfma_kernel<8, kQ8>), grid, blk, lds, s, a, b, tiles_a, nw, S); break;
    default: hipLaunchKernelGGL((gemm_pair_mfma_kernel<16, kQ8>), grid, blk, lds, s, a, b, tiles_a, nw, S); break;
  }
  return hipGetLastError();
}

bool append_vec_ok(const AppendArgs& a) {
  const int W = a.C + a.R;
  const size_t elem = a.cache_dtype == MLA_F32 ? 4 : 2;
  return a.C % 8 == 0 && a.R % 8 == 0 && W <= 2048 &&
         (reinterpret_cast<uintptr_t>(a.kv_pre) & 15) == 0 && a.kv_split_stride % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.pool) & 15) == 0 && ((size_t)W * elem) % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(a.gamma.data) & 15) == 0;
}

bool qnorm_pack_ok(const float* part, int32_t S, int64_t split_stride, int32_t n, int64_t stride,
                   WeightView gamma, _Float16* yp) {
  return yp && n % 128 == 0 && n <= 8192 && S >= 1 && S <= kMaxKSplits &&
         (reinterpret_cast<uintptr_t>(part) & 15) == 0 && stride % 4 == 0 &&
         split_stride % 4 == 0 && (reinterpret_cast<uintptr_t>(gamma.data) & 15) == 0;
}
}  // namespace

namespace {
int64_t q4_tiles(const GemmArgs& a) { return (int64_t)((a.O + 31) / 32) * a.Z * ((a.B + 31) / 32); }
}  // namespace

// The pair also requires that both products would take the same K-split
// decision on their own, so each gets the shape (and the sums) of its own
// single launch.
bool gemm_pair_ok(const GemmArgs& a, const GemmArgs& b) {
  return a.O > 0 && b.O > 0 && a.B > 0 && a.Z == 1 && b.Z == 1 && a.K == b.K && a.B == b.B &&
         gemm_mfma_ok(a) && gemm_mfma_ok(b) && a.w.dtype != MLA_Q8_0 && b.w.dtype != MLA_Q8_0 &&
         a.xp && a.xp == b.xp &&
         !a.yp && !b.yp && a.y && b.y && (q4_tiles(a) >= 128) == (q4_tiles(b) >= 128);
}

hipError_t launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, int max_splits, int* splits,
                            hipStream_t s) {
  *splits = 1;
  if (!gemm_pair_ok(a, b)) return hipErrorInvalidValue;
  const int tiles_a = (a.O + 31) / 32, tiles = tiles_a + (b.O + 31) / 32;
  int U, nw, S;
  q4_shape(a.K / 128, q4_tiles(a), max_splits, false, &U, &nw, &S);
  *splits = S;
  return launch_pair(a, b, tiles_a, tiles, U, nw, S, s);
}

hipError_t launch_gemm_nt(const GemmArgs& a, int max_splits, int* splits, hipStream_t s) {
  *splits = 1;
  if (a.O <= 0 || a.B <= 0 || a.Z <= 0) return hipSuccess;
  if (a.yp && (a.yp_K % 128) != 0) return hipErrorInvalidValue;
  if (gemm_mfma_ok(a)) {
    if (!a.xp) return hipErrorInvalidValue;
    int U, nw, S;
    q4_shape(a.K / 128, q4_tiles(a), max_splits, a.yp != nullptr, &U, &nw, &S);
    *splits = S;
    return launch_q4(a, U, nw, S, s);
  }
  if (!a.x) return hipErrorInvalidValue;  // the fp32 path reads x
  dim3 grid((a.O + kTO - 1) / kTO, (a.B + kTB - 1) / kTB, a.Z);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_f16(const float* x, int64_t x_b, int64_t x_z, int32_t Z, int32_t B,
                           int32_t K, _Float16* xp, hipStream_t s) {
  if (Z <= 0 || B <= 0 || K <= 0) return hipSuccess;
  if (K % 128 != 0) return hipErrorInvalidValue;
  const bool vec = x_b % 4 == 0 && x_z % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  const int64_t zt = (int64_t)Z * ((B + 31) / 32);
  const int64_t per = (int64_t)(K / 128) * 512;  // chunks per (z, token tile)
  if (zt > (1ll << 31) - 1 || (per + 255) / 256 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_f16_kernel, dim3((unsigned)zt, (unsigned)((per + 255) / 256)), dim3(256), 0,
                     s, x, x_b, x_z, B, K, vec, xp);
  return hipGetLastError();
}

hipError_t launch_pack_scaled(const float* x, int64_t x_b, int32_t B, int32_t K, _Float16* xp,
                              int32_t* x_exp, hipStream_t s) {
  if (B <= 0 || K <= 0) return hipSuccess;
  if (K % 128 != 0 || !x_exp) return hipErrorInvalidValue;
  const bool vec = x_b % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  const int64_t slots = (int64_t)(B + 31) / 32 * 32;
  if (slots > (1ll << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_scaled_kernel, dim3((unsigned)slots), dim3(256), 0, s, x, x_b, B, K, vec,
                     xp, x_exp);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* part, int32_t S, int64_t split_stride, int32_t B,
                               int32_t n, int64_t stride, WeightView gamma, float eps, float* y,
                               _Float16* yp, int32_t* yexp, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (S < 1 || S > kMaxKSplits || (yp && n % 128 != 0)) return hipErrorInvalidValue;
  if (qnorm_pack_ok(part, S, split_stride, n, stride, gamma, yp)) {
    const int threads = ((n / 8) + 63) / 64 * 64;
    hipLaunchKernelGGL(rmsnorm_pack_kernel, dim3(B), dim3(threads), 0, s, part, S, split_stride,
                       B, n, stride, gamma, eps, yp, yexp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(B), dim3(256), 0, s, part, S, split_stride, B, n,
                     stride, gamma, eps, y, yp, yexp);
  return hipGetLastError();
}

bool append_qnorm_ok(const AppendArgs& a, const QNormArgs& q) {
  return append_vec_ok(a) && qnorm_pack_ok(q.part, q.S, q.split_stride, q.n, q.stride, q.gamma, q.yp);
}

hipError_t launch_append_qnorm(const AppendArgs& a, const QNormArgs& q, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (!append_qnorm_ok(a, q)) return hipErrorInvalidValue;
  const int ta = ((a.C + a.R) / 8 + 63) / 64 * 64, tq = (q.n / 8 + 63) / 64 * 64;
  const int threads = ta > tq ? ta : tq;
  if (a.cache_dtype == MLA_F32)
    hipLaunchKernelGGL(append_qnorm_kernel<float>, dim3(2 * a.B), dim3(threads), 0, s, a, q);
  else
    hipLaunchKernelGGL(append_qnorm_kernel<uint16_t>, dim3(2 * a.B), dim3(threads), 0, s, a, q);
  return hipGetLastError();
}

hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int W = a.C + a.R;
  if (append_vec_ok(a)) {
    const int threads = ((W / 8) + 63) / 64 * 64;
    if (a.cache_dtype == MLA_F32)
      hipLaunchKernelGGL(append_rows_vec_kernel<float>, dim3(a.B), dim3(threads), 0, s, a);
    else
      hipLaunchKernelGGL(append_rows_vec_kernel<uint16_t>, dim3(a.B), dim3(threads), 0, s, a);
    return hipGetLastError();
  }
  if (a.cache_dtype == MLA_F32)
    hipLaunchKernelGGL(append_rows_kernel<float>, dim3(a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_rows_kernel<uint16_t>, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const bool q8_ok = a.kv_b.dtype == MLA_Q8_0 && (reinterpret_cast<uintptr_t>(a.kv_b.data) & 1) == 0;
  const bool q4 = a.kv_b.dtype == MLA_Q4G64 ||
                  (a.kv_b.dtype == MLA_Q4G64_T && a.kv_b.rows % 32 == 0 && a.kv_b.cols % 128 == 0);
  if ((q4 || q8_ok) && a.N % kAbsN == 0 && a.C % 32 == 0) {
    dim3 grid(a.H, (a.C + 127) / 128, (a.B + 31) / 32);
    const bool q8 = a.kv_b.dtype == MLA_Q8_0;
    if (a.cache_dtype == MLA_F32) {
      if (q8) hipLaunchKernelGGL((absorb_mfma_kernel<float, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((absorb_mfma_kernel<float, false>), grid, dim3(256), 0, s, a);
    } else {
      if (q8) hipLaunchKernelGGL((absorb_mfma_kernel<uint16_t, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((absorb_mfma_kernel<uint16_t, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  dim3 grid(a.H, (a.C + kAbsC - 1) / kAbsC);
  const size_t smem = (size_t)kAbsB * a.N * sizeof(float);  // [N][32] token-minor
  if (a.cache_dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(kAbsC), smem, s, a);
  else
    hipLaunchKernelGGL(absorb_kernel<uint16_t>, grid, dim3(kAbsC), smem, s, a);
  return hipGetLastError();
}

bool qb_absorb_ok(const GemmArgs& g, const AbsorbArgs& a) {
  auto q4 = [](const WeightView& w) {
    return w.dtype == MLA_Q4G64 || (w.dtype == MLA_Q4G64_T && w.rows % 32 == 0 && w.cols % 128 == 0);
  };
  return q4(g.w) && q4(a.kv_b) && gemm_mfma_ok(g) && g.xp && g.x_exp && !g.yp && g.Z == 1 &&
         g.w_row0 == 0 && g.B == a.B && a.B > 0 && g.O == a.H * kQaRows && a.N == 128 &&
         a.R == 64 && a.C >= 32 && a.C <= kQaMaxC && a.C % 32 == 0 && a.kv_b.cols == a.C &&
         g.K >= 128 && g.K <= kQaMaxUnits * 128 && (reinterpret_cast<uintptr_t>(g.xp) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.kv_b.data) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.q_abs) & 15) == 0 &&
         (a.cache_dtype == MLA_F32 || a.cache_dtype == MLA_BF16);
}

hipError_t launch_qb_absorb(const GemmArgs& g, const AbsorbArgs& a, hipStream_t s) {
  if (!qb_absorb_ok(g, a)) return hipErrorInvalidValue;
  const bool f32 = a.cache_dtype == MLA_F32;
  const void* fn = f32 ? (const void*)qb_absorb_kernel<float> : (const void*)qb_absorb_kernel<uint16_t>;
  // The dynamic LDS limit is raised once per device and instantiation.
  static std::mutex mu;
  static bool attr_set[64][2] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (!attr_set[dev][f32]) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQaLds);
      if (e != hipSuccess) return e;
      attr_set[dev][f32] = true;
    }
  }
  const dim3 grid(a.H, 2 * ((a.B + 31) / 32));
  if (f32) hipLaunchKernelGGL(qb_absorb_kernel<float>, grid, dim3(1024), kQaLds, s, g, a);
  else hipLaunchKernelGGL(qb_absorb_kernel<uint16_t>, grid, dim3(1024), kQaLds, s, g, a);
  return hipGetLastError();
}

bool merge_uv_ok(const AttnArgs& a, const GemmArgs& g) {
  const bool q4 = g.w.dtype == MLA_Q4G64 ||
                  (g.w.dtype == MLA_Q4G64_T && g.w.rows % 32 == 0 && g.w.cols % 128 == 0);
  return q4 && a.part_oh && a.part_lse && a.part_exp && a.num_splits > 1 && a.H == 128 &&
         a.C == 512 && g.Z == 128 && g.O == 128 && g.K == 512 && g.B == a.B && a.B > 0 && g.yp &&
         g.xp && g.y_z == 128 && g.yp_K == 128 * 128 && gemm_mfma_ok(g);
}

hipError_t launch_merge_uv(const AttnArgs& a, const GemmArgs& g, hipStream_t s) {
  if (!merge_uv_ok(a, g)) return hipErrorInvalidValue;
  static std::mutex mu;
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lk(mu);
    if (!attr_set[dev]) {
      e = hipFuncSetAttribute((const void*)merge_uv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kMuvLds);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL(merge_uv_kernel, dim3(128, 2 * ((a.B + 31) / 32)), dim3(1024), kMuvLds, s, a, g);
  return hipGetLastError();
}
