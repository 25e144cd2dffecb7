// Device helpers shared by the MLA decode kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

#define MLA_LDS __attribute__((address_space(3)))

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // to nearest, ties to even
  const uint32_t quiet = (u >> 16) | 0x40u;                          // NaN: quieted, sign and payload kept
  return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

// Element loaders for the storage types a cache row / q_abs may have.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// One weight element W[r][k] of any storage type (fp32, bf16, 4-bit affine g64).
struct WeightView {
  int32_t dtype;
  int32_t rows, cols;
  const void* data;
  const uint16_t* scales;
  const uint16_t* biases;
};

__device__ __forceinline__ float weight_at(const WeightView& w, int64_t r, int64_t k) {
  if (w.dtype == MLA_F32) return static_cast<const float*>(w.data)[r * w.cols + k];
  if (w.dtype == MLA_BF16) return bf16_to_f32(static_cast<const uint16_t*>(w.data)[r * w.cols + k]);
  if (w.dtype == MLA_Q8_0) {  // 34-byte blocks: binary16 scale, 32 signed bytes
    const uint8_t* blk = static_cast<const uint8_t*>(w.data) + (r * (w.cols >> 5) + (k >> 5)) * 34;
    const uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    return (float)__builtin_bit_cast(_Float16, dbits) * (float)(int8_t)blk[2 + (k & 31)];
  }
  if (w.dtype == MLA_Q4G64_T) {  // 2 KB block per (row tile, 128-k unit), lane order
    const int64_t j = k & 63, L = (r & 31) + 32 * ((k >> 6) & 1);
    const int64_t blk = (r >> 5) * (w.cols >> 7) + (k >> 7);
    const uint32_t word = static_cast<const uint32_t*>(w.data)[blk * 512 + (j >> 5) * 256 + 4 * L +
                                                                ((j & 31) >> 3)];
    const float q = static_cast<float>((word >> (4 * (k & 7))) & 15u);
    const int64_t g = blk * 64 + L;
    return fmaf(bf16_to_f32(w.scales[g]), q, bf16_to_f32(w.biases[g]));
  }
  const uint32_t word = static_cast<const uint32_t*>(w.data)[r * (w.cols >> 3) + (k >> 3)];
  const float q = static_cast<float>((word >> (4 * (k & 7))) & 15u);
  const int64_t g = r * (w.cols >> 6) + (k >> 6);
  return fmaf(bf16_to_f32(w.scales[g]), q, bf16_to_f32(w.biases[g]));
}

// The two halves of a wave side by side: lo = x[lane % 32], hi = x[lane % 32 + 32]
// in every lane, by v_permlane32_swap (a VALU op; no LDS traffic, so it does
// not wait behind outstanding LDS reads the way a bpermute shuffle does).
__device__ __forceinline__ void wave_halves(float x, float* lo, float* hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  *lo = __uint_as_float(r[0]);
  *hi = __uint_as_float(r[1]);
}

// Exponent e that brings a block's largest magnitude amax into [2^14, 2^15)
// once the block is multiplied by 2^-e, so that binary16 holds it with full
// 11-bit significands and no overflow; clamped to [-100, 113] so that 2^-e
// and 2^e are normal floats.  0 for amax zero, infinite or NaN (those values
// pass through unscaled).  A power-of-two scale is exact in both directions.
__device__ __forceinline__ int f16_range_exp(float amax) {
  if (!(amax > 0.f) || !(amax <= 3.4028235e38f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 14;
  return e < -100 ? -100 : (e > 113 ? 113 : e);
}
// 2^k for k in [-126, 127], from the exponent bits.
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Launchers (defined in the kernel translation units, called by the C ABI layer).
struct AttnArgs {
  const void* q_abs;        // [B, H, W] cache dtype
  const void* pool;         // [num_blocks, block, W]
  const int32_t* table;     // [num_seqs, max_blocks]
  const int32_t* q_seq;     // [B] table row of query b, or null: row b
  const int32_t* seq_lens;  // [B] rows query b attends
  float* v_combine;         // [B, H, C]
  float* lse;               // [B, H] or null
  float* part_o;            // [B, S, H, C] fp32 partials (fp32 kernel, S > 1)
  _Float16* part_oh;        // [B*S slots, H, C] fp16 partials * 2^-part_exp (MFMA kernel, S > 1)
  float* part_exp;          // [B*S slots, H]    the exponent e of each fp16 partial
  float* part_lse;          // [B, S, H]   (S > 1)
  // MFMA kernel, S > 1: partials are kept in slots; part_first[b] is query b's
  // first slot and part_first[B] the rows per split the split kernel used
  int32_t* part_first;      // [B + 1]
  // or null: the merge of the MFMA kernel's partials also writes v_combine as
  // packed fp16 [H][B][C] (packed_index with z = head), the input layout of the
  // per-head W_UV product on the 4-bit path
  _Float16* vc_pk;
  int32_t B, H, C, R, block, max_blocks, num_blocks, num_seqs;
  int32_t max_len, split_rows, num_splits;
  int32_t auto_slots;       // > 0: the split kernel sizes the splits from the lengths,
                            // at most auto_slots non-empty splits in all (MFMA kernel)
  float scale_log2;         // softmax_scale * log2(e)
};

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_generic_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s);

// y[z][b][o] = sum_k W[z*w_zrows + w_row0 + o][k] * x[z*x_z + b*x_b + k], o < O, k < K.
//
// The 4-bit MFMA path reads its activations packed (xp, fp16, see packed_index);
// the fp32 path reads x.  The result goes to fp32 y or, for a following GEMM on
// the MFMA path, packed fp16 yp holding the logical matrix [b][z*y_z + o] with
// row length yp_K.  With K splits the partial sums of split s land at
// y + s * y_s and the consumer adds them.
struct GemmArgs {
  WeightView w;
  int64_t w_row0, w_zrows;
  const float* x;
  const _Float16* xp;
  int64_t x_b, x_z;
  float* y;
  _Float16* yp;
  int64_t y_b, y_z, y_s, yp_K;
  int32_t O, K, B, Z;
  // with xp: token b's packed activations hold x * 2^-x_exp[b] (or null: x);
  // the results are multiplied back by 2^x_exp[b]
  const int32_t* x_exp;
};

// Packed fp16 activations of a logical [Z][B][K] matrix (K % 128 == 0), laid
// out in the order the MFMA lanes read them: tiles of 32 tokens, then units of
// 128 k, then MFMA step st (8 k), lane half hh (64 k), token in tile, and 8
// values in pair order k0 k4 k1 k5 k2 k6 k3 k7.  One step of one unit is 1 KB
// contiguous for the 64 lanes.  Token slots past B are zero.
__host__ __device__ __forceinline__ int64_t packed_index(int64_t z, int64_t b, int64_t k,
                                                          int64_t B, int64_t K) {
  const int64_t tiles = (B + 31) >> 5;
  const int64_t unit = ((z * tiles + (b >> 5)) * (K >> 7) + (k >> 7));
  const int64_t lane = ((k >> 6) & 1) * 32 + (b & 31);
  return ((unit * 8 + ((k >> 3) & 7)) * 64 + lane) * 8 + ((k & 3) << 1) + ((k >> 2) & 1);
}
__host__ __device__ __forceinline__ size_t packed_bytes(int64_t Z, int64_t B, int64_t K) {
  return (size_t)Z * ((B + 31) / 32) * 32 * K * 2;
}

constexpr int kMaxKSplits = 16;

// True when the weight runs on the 4-bit MFMA path (which reads xp).
bool gemm_mfma_ok(const GemmArgs& a);
// Largest number of K splits the MFMA path may use for a depth K (workspace sizing).
int gemm_max_splits(int64_t K);
// Launches y = x W^T; *splits receives the number of K splits written (1 unless
// max_splits > 1 and y is fp32).
hipError_t launch_gemm_nt(const GemmArgs& a, int max_splits, int* splits, hipStream_t s);
// Packs fp32 x[z*x_z + b*x_b + k] into packed fp16 (packed_index) for the MFMA path.
hipError_t launch_pack_f16(const float* x, int64_t x_b, int64_t x_z, int32_t Z, int32_t B,
                           int32_t K, _Float16* xp, hipStream_t s);
// Packs fp32 x[b*x_b + k] (Z = 1) with a power-of-two scale per token: token
// b's values times 2^-x_exp[b] (f16_range_exp of its largest magnitude), so
// no value overflows binary16; the consuming GEMM gets x_exp.
hipError_t launch_pack_scaled(const float* x, int64_t x_b, int32_t B, int32_t K, _Float16* xp,
                              int32_t* x_exp, hipStream_t s);

// RMSNorm of rows b < B of the sum of S split partials part[s*split_stride +
// b*stride + i], i < n, with gamma (1 x n weight of F32/BF16), written to
// y[b*stride + i] (fp32; may alias part) or packed fp16 yp (n % 128 == 0),
// row b times 2^-yexp[b] (f16_range_exp of its largest magnitude).
hipError_t launch_rmsnorm_rows(const float* part, int32_t S, int64_t split_stride, int32_t B,
                               int32_t n, int64_t stride, WeightView gamma, float eps, float* y,
                               _Float16* yp, int32_t* yexp, hipStream_t s);

struct AppendArgs {
  const float* kv_pre;      // [S][B, W] fp32 partial sums of the pre-norm row
  int32_t kv_splits;        // S >= 1
  int64_t kv_split_stride;
  WeightView gamma;         // 1 x C
  const float* inv_freq;    // [R/2]
  float rope_mscale;
  const int32_t* positions; // [B]
  void* pool;
  const int32_t* table;     // [num_seqs, max_blocks]
  const int32_t* q_seq;     // [B] table row of token b, or null: row b
  int32_t* dev_status;
  int32_t B, C, R, block, max_blocks, num_blocks, cache_dtype, num_seqs;
  float eps;
};
hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s);
// MLA_Q4G64 [rows, cols] (rows % 32 == 0, cols % 128 == 0) -> MLA_Q4G64_T.
hipError_t launch_repack_q4(const WeightView& src, void* data, uint16_t* scales, uint16_t* biases,
                            hipStream_t s);

// RMSNorm of a q latent from its split partial sums, into the packed layout.
struct QNormArgs {
  const float* part;        // [S][B, n] fp32 partial sums
  int32_t S;
  int64_t split_stride;
  int32_t n;
  int64_t stride;           // between tokens inside a split
  WeightView gamma;         // 1 x n
  float eps;
  _Float16* yp;             // packed [B][n], token b times 2^-yexp[b]
  int32_t* yexp;            // [B]
};
// The append (token count a.B) and the q-latent norm of the same tokens in
// one launch; hipErrorInvalidValue (nothing launched) when either part does
// not fit its vector kernel.
hipError_t launch_append_qnorm(const AppendArgs& a, const QNormArgs& q, hipStream_t s);
bool append_qnorm_ok(const AppendArgs& a, const QNormArgs& q);
// y_a = x W_a^T and y_b = x W_b^T in one launch over the same packed x, with
// the K splits of the pair's combined tile count (*splits, for both);
// hipErrorInvalidValue (nothing launched) unless both are 4-bit weights on the
// MFMA path with the same depth and tokens, Z = 1, fp32 outputs and the same
// K-split decision as their own launches would take.
hipError_t launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, int max_splits, int* splits,
                            hipStream_t s);
bool gemm_pair_ok(const GemmArgs& a, const GemmArgs& b);

struct AbsorbArgs {
  const float* q;           // [B, H, N+R]
  WeightView kv_b;          // [H*(N+V), C]
  const float* inv_freq;
  float rope_mscale;
  const int32_t* positions;
  void* q_abs;              // [B, H, C+R] cache dtype
  int32_t B, H, N, R, V, C, cache_dtype;
};
hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s);
// q_b (g: the 4-bit product of the packed q latent) and the absorb (a, reading
// q from LDS instead of a.q) in one launch; qb_absorb_ok tells whether the
// shapes and formats take it (4-bit q_b and W_UK, N 128, R 64, C <= 512,
// q LoRA rank <= 1536).
bool qb_absorb_ok(const GemmArgs& g, const AbsorbArgs& a);
// The attention merge of the MFMA kernel's split partials (a) and W_UV (g, one
// unit of 128 k per wave, packed fp16 output for o_proj) in one launch, with
// the same results as the merge kernel followed by the W_UV GEMM.
bool merge_uv_ok(const AttnArgs& a, const GemmArgs& g);
hipError_t launch_merge_uv(const AttnArgs& a, const GemmArgs& g, hipStream_t s);
hipError_t launch_qb_absorb(const GemmArgs& g, const AbsorbArgs& a, hipStream_t s);
