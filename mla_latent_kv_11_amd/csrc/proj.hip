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
#include <math.h>

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
  float* y = a.y + (int64_t)z * a.y_z;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = o0 + 4 * to + i, bb = b0 + 2 * tb + j;
      if (o < a.O && bb < a.B) y[(int64_t)bb * a.y_b + o] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// 4-bit affine weights on MFMA: y[z][b][o] = sum_k W[row(z, o)][k] x[z][b][k].
// One workgroup = 32 outputs x 32 tokens; its 4 waves split K in quarters and
// reduce through LDS (deterministic).  Per 128-k chunk a lane dequantises one
// row's 64 consecutive k (8 packed words, one scale/bias group) into fp16 MFMA
// A operands and multiplies them by 64 fp16 activations of one token:
// v_mfma_f32_32x32x16_f16, k-slot j of lane-half h at step st <-> k = k0 + 64h
// + 8st + j (the same map on both operands).  fp32 accumulate.
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(256) to_f16_kernel(const float* x, int64_t x_b, int64_t x_z,
                                                     _Float16* y, int32_t B, int32_t K, int32_t Z) {
  const int64_t n = (int64_t)Z * B * K;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t k = i % K, zb = i / K;
    const int64_t bb = zb % B, z = zb / B;
    y[i] = (_Float16)x[z * x_z + bb * x_b + k];
  }
}

__global__ void __launch_bounds__(256) gemm_q4_mfma_kernel(GemmArgs a, const _Float16* xh) {
  __shared__ f32x16_t red[3][64];
  const int z = blockIdx.z;
  const int o0 = blockIdx.x * 32;
  const int b0 = blockIdx.y * 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int kq = a.K / 4;
  const int kbeg = wave * kq;

  int row = o0 + l32;
  row = row < a.O ? row : a.O - 1;  // rows past the end read a valid row; never stored
  const int64_t wrow = a.w_row0 + (int64_t)z * a.w_zrows + row;
  const uint32_t* wp = static_cast<const uint32_t*>(a.w.data) + wrow * (a.w.cols >> 3);
  const uint16_t* sp = a.w.scales + wrow * (a.w.cols >> 6);
  const uint16_t* bp = a.w.biases + wrow * (a.w.cols >> 6);
  const int tok = b0 + l32;
  const bool tok_ok = tok < a.B;
  const _Float16* xp = xh + ((int64_t)z * a.B + (tok_ok ? tok : 0)) * a.K;

  f32x16_t acc = f32x16_t{};
  for (int k0 = kbeg; k0 < kbeg + kq; k0 += 128) {
    const int kk = k0 + 64 * h;
    const uint4 w0 = *reinterpret_cast<const uint4*>(wp + (kk >> 3));
    const uint4 w1 = *reinterpret_cast<const uint4*>(wp + (kk >> 3) + 4);
    const float sc = bf16_to_f32(sp[kk >> 6]);
    const float bi = bf16_to_f32(bp[kk >> 6]);
    f16x8_t xf[8];
#pragma unroll
    for (int st = 0; st < 8; ++st)
      xf[st] = tok_ok ? *reinterpret_cast<const f16x8_t*>(xp + kk + 8 * st) : f16x8_t{};
    const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      f16x8_t wf;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wf[j] = (_Float16)fmaf((float)((words[st] >> (4 * j)) & 15u), sc, bi);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf, xf[st], acc, 0, 0, 0);
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0 || !tok_ok) return;
  acc += red[0][lane];
  acc += red[1][lane];
  acc += red[2][lane];
  float* y = a.y + (int64_t)z * a.y_z + (int64_t)tok * a.y_b;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int o = o0 + (j >> 2) * 8 + h * 4 + (j & 3);
    if (o < a.O) y[o] = acc[j];
  }
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

__device__ __forceinline__ float gamma_at(const WeightView& g, int i) {
  return g.dtype == MLA_F32 ? static_cast<const float*>(g.data)[i]
                            : bf16_to_f32(static_cast<const uint16_t*>(g.data)[i]);
}

__global__ void __launch_bounds__(256) rmsnorm_rows_kernel(float* x, int32_t n, int64_t stride,
                                                           WeightView gamma, float eps) {
  __shared__ float red[4];
  float* row = x + (int64_t)blockIdx.x * stride;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) ss = fmaf(row[i], row[i], ss);
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += 256) row[i] = row[i] * inv * gamma_at(gamma, i);
}

// (x, y) -> mscale * (x cos a - y sin a, x sin a + y cos a), a = pos * inv_freq,
// angle and rotation in fp64 (exact enough for positions in the millions).
__device__ __forceinline__ void rope_pair(float x, float y, int pos, float inv_freq, float mscale,
                                          float* ox, float* oy) {
  const double ang = (double)pos * (double)inv_freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  *ox = (float)((double)mscale * ((double)x * cs - (double)y * sn));
  *oy = (float)((double)mscale * ((double)x * sn + (double)y * cs));
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
  const int blk = a.table[(size_t)b * a.max_blocks + pos / a.block];
  if (blk < 0 || blk >= a.num_blocks) {
    if (a.dev_status && threadIdx.x == 0) atomicOr(a.dev_status, (int)MLA_DEV_BAD_BLOCK);
    return;
  }
  const float* src = a.kv_pre + (size_t)b * W;
  T* dst = static_cast<T*>(a.pool) + ((size_t)blk * a.block + pos % a.block) * W;
  float ss = 0.f;
  for (int i = threadIdx.x; i < a.C; i += 256) ss = fmaf(src[i], src[i], ss);
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / (float)a.C + a.eps);
  for (int i = threadIdx.x; i < a.C; i += 256)
    Elem<T>::store(dst, i, src[i] * inv * gamma_at(a.gamma, i));
  for (int i = threadIdx.x; i < a.R / 2; i += 256) {
    float ox, oy;
    rope_pair(src[a.C + 2 * i], src[a.C + 2 * i + 1], pos, a.inv_freq[i], a.rope_mscale, &ox, &oy);
    Elem<T>::store(dst, a.C + 2 * i, ox);
    Elem<T>::store(dst, a.C + 2 * i + 1, oy);
  }
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

}  // namespace

bool gemm_uses_mfma(const GemmArgs& a) {
  return a.w.dtype == MLA_Q4G64 && (a.K % 512) == 0 && (a.w.cols % 64) == 0 && a.K <= a.w.cols;
}

size_t gemm_staging_bytes(const GemmArgs& a) {
  return gemm_uses_mfma(a) ? (size_t)a.Z * a.B * a.K * sizeof(_Float16) : 0;
}

hipError_t launch_gemm_nt(const GemmArgs& a, void* staging, hipStream_t s) {
  if (a.O <= 0 || a.B <= 0 || a.Z <= 0) return hipSuccess;
  if (gemm_uses_mfma(a)) {
    _Float16* xh = static_cast<_Float16*>(staging);
    const int64_t n = (int64_t)a.Z * a.B * a.K;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(to_f16_kernel, dim3(blocks), dim3(256), 0, s, a.x, a.x_b, a.x_z, xh, a.B, a.K,
                       a.Z);
    dim3 grid((a.O + 31) / 32, (a.B + 31) / 32, a.Z);
    hipLaunchKernelGGL(gemm_q4_mfma_kernel, grid, dim3(256), 0, s, a, (const _Float16*)xh);
    return hipGetLastError();
  }
  dim3 grid((a.O + kTO - 1) / kTO, (a.B + kTB - 1) / kTB, a.Z);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(float* x, int32_t B, int32_t n, int64_t stride, WeightView gamma,
                               float eps, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(B), dim3(256), 0, s, x, n, stride, gamma, eps);
  return hipGetLastError();
}

hipError_t launch_append_rows(const AppendArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.cache_dtype == MLA_F32)
    hipLaunchKernelGGL(append_rows_kernel<float>, dim3(a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_rows_kernel<uint16_t>, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  dim3 grid(a.H, (a.C + kAbsC - 1) / kAbsC);
  const size_t smem = (size_t)kAbsB * a.N * sizeof(float);  // [N][32] token-minor
  if (a.cache_dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(kAbsC), smem, s, a);
  else
    hipLaunchKernelGGL(absorb_kernel<uint16_t>, grid, dim3(kAbsC), smem, s, a);
  return hipGetLastError();
}
