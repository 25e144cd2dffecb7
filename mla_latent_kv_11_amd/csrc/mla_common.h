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
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
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
  const uint32_t word = static_cast<const uint32_t*>(w.data)[r * (w.cols >> 3) + (k >> 3)];
  const float q = static_cast<float>((word >> (4 * (k & 7))) & 15u);
  const int64_t g = r * (w.cols >> 6) + (k >> 6);
  return fmaf(bf16_to_f32(w.scales[g]), q, bf16_to_f32(w.biases[g]));
}

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
  const int32_t* table;     // [B, max_blocks]
  const int32_t* seq_lens;  // [B]
  float* v_combine;         // [B, H, C]
  float* lse;               // [B, H] or null
  float* part_o;            // [B, S, H, C] (S > 1)
  float* part_lse;          // [B, S, H]   (S > 1)
  int32_t B, H, C, R, block, max_blocks, num_blocks;
  int32_t max_len, split_rows, num_splits;
  float scale_log2;         // softmax_scale * log2(e)
};

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_generic_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs& a, hipStream_t s);

// y[z][b][o] = sum_k W[z*w_zrows + w_row0 + o][k] * x[z*x_z + b*x_b + k], o < O, k < K.
struct GemmArgs {
  WeightView w;
  int64_t w_row0, w_zrows;
  const float* x;
  int64_t x_b, x_z;
  float* y;
  int64_t y_b, y_z;
  int32_t O, K, B, Z;
};
// 4-bit weights with K % 512 == 0 run on MFMA and need a staging buffer of
// gemm_staging_bytes() for the fp16 copy of x; other weights ignore it.
bool gemm_uses_mfma(const GemmArgs& a);
size_t gemm_staging_bytes(const GemmArgs& a);
hipError_t launch_gemm_nt(const GemmArgs& a, void* staging, hipStream_t s);

// In-place RMSNorm of x[b][0..n) with gamma (1 x n weight of F32/BF16).
hipError_t launch_rmsnorm_rows(float* x, int32_t B, int32_t n, int64_t stride, WeightView gamma,
                               float eps, hipStream_t s);

struct AppendArgs {
  const float* kv_pre;      // [B, W] fp32, pre-norm row
  WeightView gamma;         // 1 x C
  const float* inv_freq;    // [R/2]
  float rope_mscale;
  const int32_t* positions; // [B]
  void* pool;
  const int32_t* table;
  int32_t* dev_status;
  int32_t B, C, R, block, max_blocks, num_blocks, cache_dtype;
  float eps;
};
hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s);

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
