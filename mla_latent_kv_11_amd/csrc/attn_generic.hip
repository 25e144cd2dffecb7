// MLA decode attention for fp32 caches of any geometry (VALU, one wave per
// (split, head, sequence)).  Same math and the same split/partial layout as the
// bf16 MFMA kernel: scores over the full row [c_kv ; k_pe], online softmax in
// the exp2 domain, v_combine = sum_t p_t c_kv[t] (moeflux mla_attn_forward.rs,
// mla_sdpa_folded; turbospark deepseek2/attn.rs, encode_mla_attention_decode).
#include <math.h>

#include "mla_common.h"

namespace {

constexpr int kRows = 64;           // rows per tile = one per lane
constexpr int kMaxCPerLane = 16;    // C <= 1024
constexpr float kLn2 = 0.69314718055994530942f;

__global__ void __launch_bounds__(64) attn_generic_kernel(AttnArgs a) {
  extern __shared__ float sm[];
  const int W = a.C + a.R;
  float* qs = sm;              // [W]
  float* ps = sm + W;          // [kRows]
  int* phys_s = reinterpret_cast<int*>(ps + kRows);  // [kRows]

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;

  int len = a.seq_lens[b];
  len = len < a.max_len ? len : a.max_len;
  const int row_begin = split * a.split_rows;
  int row_end = row_begin + a.split_rows;
  row_end = row_end < len ? row_end : len;

  float* out_o;
  float* out_lse;
  if (a.num_splits == 1) {
    out_o = a.v_combine + ((size_t)b * a.H + h) * a.C;
    out_lse = a.lse ? a.lse + (size_t)b * a.H + h : nullptr;
  } else {
    const size_t bs = (size_t)b * a.num_splits + split;
    out_o = a.part_o + (bs * a.H + h) * a.C;
    out_lse = a.part_lse + bs * a.H + h;
  }
  if (row_begin >= row_end) {
    if (a.num_splits == 1)
      for (int c = lane; c < a.C; c += 64) out_o[c] = 0.f;
    if (out_lse && lane == 0) *out_lse = -INFINITY;
    return;
  }

  const float* q = static_cast<const float*>(a.q_abs) + ((size_t)b * a.H + h) * W;
  for (int k = lane; k < W; k += 64) qs[k] = q[k];
  __syncthreads();

  const float* pool = static_cast<const float*>(a.pool);
  const int sq = a.q_seq ? a.q_seq[b] : b;
  const bool seq_ok = sq >= 0 && sq < a.num_seqs;  // else every row reads as a bad entry
  const int32_t* trow = a.table + (size_t)(seq_ok ? sq : 0) * a.max_blocks;
  float o[kMaxCPerLane];
#pragma unroll
  for (int i = 0; i < kMaxCPerLane; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  bool bad = false;

  for (int t0 = row_begin; t0 < row_end; t0 += kRows) {
    const int t = t0 + lane;
    int phys = -1;
    float s = -INFINITY;
    if (t < row_end) {
      const int blk = seq_ok ? trow[t / a.block] : -1;
      if (blk >= 0 && blk < a.num_blocks) {
        phys = blk * a.block + t % a.block;
        const float* row = pool + (size_t)phys * W;
        float acc = 0.f;
        for (int k = 0; k < W; ++k) acc = fmaf(qs[k], row[k], acc);
        s = acc * a.scale_log2;
      } else {
        s = NAN;
      }
    }
    bad |= __ballot(s != s) != 0;
    const float mt = wave_max(s);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    const float p = (phys >= 0) ? exp2f(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    ps[lane] = p;
    phys_s[lane] = phys;
    __syncthreads();
    const int nr = (row_end - t0) < kRows ? (row_end - t0) : kRows;
#pragma unroll
    for (int i = 0; i < kMaxCPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < a.C) {
        float acc = o[i] * alpha;
        for (int r = 0; r < nr; ++r) {
          const int pr = phys_s[r];
          if (pr >= 0) acc = fmaf(ps[r], pool[(size_t)pr * W + c], acc);
        }
        o[i] = acc;
      }
    }
    __syncthreads();
  }

  const float inv_l = bad ? NAN : 1.0f / l_run;
#pragma unroll
  for (int i = 0; i < kMaxCPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < a.C) out_o[c] = o[i] * inv_l;
  }
  if (out_lse && lane == 0) *out_lse = bad ? NAN : (m_run + log2f(l_run)) * kLn2;
}

}  // namespace

hipError_t launch_attn_generic_f32(const AttnArgs& a, hipStream_t s) {
  const size_t smem = (a.C + a.R + 2 * kRows) * sizeof(float);
  hipLaunchKernelGGL(attn_generic_kernel, dim3(a.num_splits, a.H, a.B), dim3(64), smem, s, a);
  return hipGetLastError();
}
