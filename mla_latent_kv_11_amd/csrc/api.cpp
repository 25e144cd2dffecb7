// C ABI of the MLA decode library: host-side validation, workspace layout,
// split-K planning and kernel launches.  Nothing here allocates or
// synchronises; every check runs before the first launch
// (turbospark deepseek2/attn.rs, validate_q8_0_matrix: validate before any
// kernel receives a raw offset; moeflux mla_attn_forward.rs,
// MlaForwardGpuError: the error taxonomy).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "mla_common.h"

int attn_mfma_max_split_rows();

// Scratch of mla_decode_attn_noalloc: the split partials live in this static
// device array instead of a caller workspace.  Each device holds its own copy
// at its own address, found once per device with hipGetSymbolAddress; host
// code only ever passes that address (the array's name is a host-side
// stand-in).  Calls on one device share it, so overlapping calls race.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
// Smallest automatic split: 128 rows (4 tiles).  Shorter splits cost a query
// load and a partial write each; on one 4096-row context 64-, 128-, 256- and
// 512-row splits took 35.9, 34.0, 38.0 and 50.0 us.
constexpr int64_t kMinSplitRows = 128;
constexpr int kMaxDim = 1 << 16;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dims_ok(const mla_dims* d) {
  if (!d) return false;
  if (d->num_heads < 1 || d->qk_nope < 0 || d->qk_rope < 2 || (d->qk_rope & 1) ||
      d->v_head < 1 || d->kv_lora < 1 || d->hidden < 0 || d->q_lora < 0 || d->block_size < 1)
    return false;
  if (d->num_heads > kMaxDim || d->qk_nope > kMaxDim || d->qk_rope > kMaxDim ||
      d->v_head > kMaxDim || d->kv_lora > kMaxDim || d->hidden > (1 << 20) ||
      d->q_lora > (1 << 20) || d->block_size > (1 << 20))
    return false;
  if (d->cache_dtype != MLA_F32 && d->cache_dtype != MLA_BF16) return false;
  if (!(d->rms_eps >= 0.f) || !isfinite(d->rms_eps)) return false;
  return true;
}

int dims_status(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->cache_dtype != MLA_F32 && d->cache_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  return dims_ok(d) ? MLA_OK : MLA_ERR_DIMS;
}

// A weight must be non-null, of an accepted dtype, and exactly [rows, cols].
// allow_q4: the 4-bit affine format, row-major or tiled; allow_q8: Q8_0
// (kv_b only).
int check_weight(const mla_weight* w, int64_t rows, int64_t cols, bool allow_q4,
                 bool allow_q8 = false) {
  if (!w || !w->data) return MLA_ERR_NULL;
  const bool q4 = w->dtype == MLA_Q4G64 || w->dtype == MLA_Q4G64_T;
  if (w->dtype != MLA_F32 && w->dtype != MLA_BF16 && !(allow_q4 && q4) &&
      !(allow_q8 && w->dtype == MLA_Q8_0))
    return MLA_ERR_DTYPE;
  if (w->rows != rows || w->cols != cols) return MLA_ERR_DIMS;
  if (q4) {
    if (cols % 64 != 0) return MLA_ERR_DIMS;
    if (w->dtype == MLA_Q4G64_T && (cols % 128 != 0 || rows % 32 != 0)) return MLA_ERR_DIMS;
    if (!w->scales || !w->biases) return MLA_ERR_NULL;
  }
  if (w->dtype == MLA_Q8_0 && (cols % 32 != 0 || cols <= 0)) return MLA_ERR_DIMS;
  return MLA_OK;
}

WeightView view(const mla_weight* w) {
  return WeightView{w->dtype, w->rows, w->cols, w->data, w->scales, w->biases};
}

int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int max_split_rows(const mla_dims* d) {
  return d->cache_dtype == MLA_BF16 ? attn_mfma_max_split_rows() : (1 << 30);
}

// Rows per split and splits per sequence.  Automatic: about one workgroup per
// compute unit over batch * max_seq_len rows, at least kMinSplitRows per split: each
// split also reads the sequence's 147 KB query and writes a 128 KB partial, so
// shorter splits cost more in overhead than they gain in parallelism.
int plan(const mla_dims* d, int32_t batch, int32_t max_len, int32_t req, int32_t* rows,
         int32_t* splits) {
  if (max_len < 0 || batch < 0) return MLA_ERR_DIMS;
  if (req < 0 || (req % 64) != 0) return MLA_ERR_DIMS;
  const int64_t cap = max_split_rows(d);
  int64_t r;
  if (req > 0) {
    if (req > cap) return MLA_ERR_DIMS;
    r = req;
  } else {
    const int64_t total = (int64_t)(batch > 0 ? batch : 1) * (max_len > 0 ? max_len : 1);
    const int64_t cus = device_cus();
    r = (total + cus - 1) / cus;
    r = (r + 63) / 64 * 64;
    if (r < kMinSplitRows) r = kMinSplitRows;
    if (r > cap) r = cap / 64 * 64;
  }
  int64_t s = max_len > 0 ? (max_len + r - 1) / r : 1;
  if (s < 1) s = 1;
  if (s > (1 << 20)) return MLA_ERR_DIMS;
  *rows = (int32_t)r;
  *splits = (int32_t)s;
  return MLA_OK;
}

// Workspace regions of the projection calls (each 256-byte aligned); "packed"
// is the fp16 activation layout of the 4-bit MFMA path (packed_index):
//   append : x packed [B][hidden]; kv_a partial sums [S][B][W] fp32; the
//            packed tokens' exponents [B] int32
//   absorb : x packed [B][hidden]; q_a partial sums [S][B][q_lora] fp32;
//            normalised q latent packed [B][q_lora]; q [B][H][N+R] fp32; the
//            exponents of the packed x and q latent, [B] int32 each
//   out    : v_combine packed [H][B][C]; per-head W_UV outputs [B][H*V]
//            (packed fp16 for a 4-bit o_proj, else fp32)
size_t ws_append(const mla_dims* d, int32_t B) {
  if (d->hidden <= 0) return 0;
  return align_up(packed_bytes(1, B, d->hidden)) +
         align_up((size_t)gemm_max_splits(d->hidden) * B * (d->kv_lora + d->qk_rope) * 4) +
         align_up((size_t)B * 4);
}
size_t ws_q_part(const mla_dims* d, int32_t B) {
  return align_up((size_t)gemm_max_splits(d->hidden) * B * d->q_lora * 4);
}
size_t ws_absorb(const mla_dims* d, int32_t B) {
  if (d->q_lora <= 0) return 0;
  return align_up(packed_bytes(1, B, d->hidden)) + ws_q_part(d, B) +
         align_up(packed_bytes(1, B, d->q_lora)) +
         align_up((size_t)B * d->num_heads * (d->qk_nope + d->qk_rope) * 4) +
         2 * align_up((size_t)B * 4);
}
// Split partials: fp16 values plus a power-of-two exponent per (sequence,
// split, head) for a bf16 cache, fp32 values for an fp32 cache; and the lse.
size_t ws_attn_o(const mla_dims* d, int32_t B, int32_t splits) {
  const size_t elem = d->cache_dtype == MLA_BF16 ? 2 : 4;
  return align_up((size_t)B * splits * d->num_heads * d->kv_lora * elem);
}
// For a bf16 cache also the slot table (first partial slot of each query and
// the rows per split the kernel chose).
size_t ws_attn(const mla_dims* d, int32_t B, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t lse = align_up((size_t)B * splits * d->num_heads * 4);
  if (d->cache_dtype != MLA_BF16) return ws_attn_o(d, B, splits) + lse;
  return ws_attn_o(d, B, splits) + 2 * lse + align_up(((size_t)B + 1) * 4);
}
// mla_decode_layer: the regions of the four calls side by side (append,
// absorb, attention, out), each a multiple of kAlign.
size_t ws_layer(const mla_dims* d, int32_t B, int32_t splits);
size_t ws_out(const mla_dims* d, int32_t B) {
  const size_t vc = align_up(packed_bytes(d->num_heads, B, d->kv_lora));
  return vc + (d->hidden > 0 ? align_up((size_t)((B + 31) / 32) * 32 * d->num_heads * d->v_head * 4) : 0);
}

size_t ws_layer(const mla_dims* d, int32_t B, int32_t splits) {
  return ws_append(d, B) + ws_absorb(d, B) + ws_attn(d, B, splits) + ws_out(d, B);
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Device address of this device's scratch, or nullptr if it cannot be found.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

double yarn_get(double s, double m) { return s <= 1.0 ? 1.0 : 0.1 * m * log(s) + 1.0; }

}  // namespace

extern "C" {

int mla_validate_q8_0_kv_b(int32_t dtype, int64_t rows, int64_t cols, int64_t size_bytes,
                           int32_t heads, int32_t nope, int32_t kv_lora, int32_t v_head) {
  if (dtype != MLA_Q8_0) return MLA_ERR_DTYPE;
  if (heads < 1 || nope < 0 || v_head < 0 || kv_lora < 1) return MLA_ERR_DIMS;
  const int64_t expect_rows = (int64_t)heads * ((int64_t)nope + v_head);  // no overflow in int64
  if (rows != expect_rows || cols != kv_lora) return MLA_ERR_DIMS;
  if (kv_lora % 32 != 0) return MLA_ERR_DIMS;
  const int64_t row_bytes = (int64_t)(kv_lora / 32) * 34;
  if (rows > INT64_MAX / row_bytes) return MLA_ERR_DIMS;
  if (size_bytes != rows * row_bytes) return MLA_ERR_DIMS;
  return MLA_OK;
}

int mla_repack_q4g64(const mla_weight* src, void* data, uint16_t* scales, uint16_t* biases,
                     void* stream) {
  if (!src || !src->data || !src->scales || !src->biases || !data || !scales || !biases)
    return MLA_ERR_NULL;
  if (src->dtype != MLA_Q4G64) return MLA_ERR_DTYPE;
  if (src->rows < 0 || src->cols < 0 || src->rows % 32 != 0 || src->cols % 128 != 0)
    return MLA_ERR_DIMS;
  return hip_status(launch_repack_q4(view(src), data, scales, biases, (hipStream_t)stream));
}

const char* mla_status_str(int st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DIMS: return "inconsistent or out-of-range dimensions";
    case MLA_ERR_DTYPE: return "unsupported element type";
    case MLA_ERR_UNSUPPORTED: return "no kernel for these dimensions";
    case MLA_ERR_CAPACITY: return "max_seq_len exceeds the block table capacity";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int mla_yarn_tables(const mla_yarn* p, int32_t R, int32_t qk_head_dim, float* inv_freq,
                    float* rope_mscale, float* softmax_scale) {
  if (!p) return MLA_ERR_NULL;
  if (R < 2 || (R & 1) || R > kMaxDim || qk_head_dim < 1 || !(p->theta > 1.0) ||
      !(p->factor > 0.0) || !(p->original_max_pos > 0.0) || !(p->beta_fast > 0.0) ||
      !(p->beta_slow > 0.0))
    return MLA_ERR_DIMS;
  if (inv_freq) {
    // Correction dimension: the pair index whose rotation count over the
    // original context equals r.
    const double two_pi = 6.283185307179586476925;
    auto corr = [&](double r) {
      return (double)R * log(p->original_max_pos / (r * two_pi)) / (2.0 * log(p->theta));
    };
    double lo = floor(corr(p->beta_fast));
    double hi = ceil(corr(p->beta_slow));
    if (lo < 0) lo = 0;
    if (hi > R - 1) hi = R - 1;
    if (lo == hi) hi += 0.001;
    for (int i = 0; i < R / 2; ++i) {
      const double base = pow(p->theta, -2.0 * i / (double)R);
      double ramp = (i - lo) / (hi - lo);
      ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
      inv_freq[i] = (float)(base * (1.0 - ramp) + (base / p->factor) * ramp);
    }
  }
  const double m = yarn_get(p->factor, p->mscale);
  const double m_all = yarn_get(p->factor, p->mscale_all_dim);
  if (rope_mscale) *rope_mscale = (float)(m / m_all);
  if (softmax_scale) *softmax_scale = (float)(m_all * m_all / sqrt((double)qk_head_dim));
  return MLA_OK;
}

size_t mla_workspace_bytes(const mla_dims* d, int32_t B, int32_t max_len, int32_t split_rows) {
  if (!dims_ok(d) || B < 0) return 0;
  int32_t rows = 0, splits = 1;
  if (plan(d, B, max_len, split_rows, &rows, &splits) != MLA_OK) return 0;
  size_t w = ws_append(d, B);
  w = w > ws_absorb(d, B) ? w : ws_absorb(d, B);
  w = w > ws_attn(d, B, splits) ? w : ws_attn(d, B, splits);
  w = w > ws_out(d, B) ? w : ws_out(d, B);
  return w + kAlign;
}

int mla_attn_plan(const mla_dims* d, int32_t B, int32_t max_len, int32_t split_rows,
                  int32_t* rows_per_split, int32_t* num_splits) {
  int st = dims_status(d);
  if (st) return st;
  if (!rows_per_split || !num_splits) return MLA_ERR_NULL;
  return plan(d, B, max_len, split_rows, rows_per_split, num_splits);
}

// Split plan from the lengths themselves (host copies): the smallest split
// (a multiple of 64, at least kMinSplitRows) whose non-empty workgroups,
// sum_b ceil(len_b / rows), fit one per compute unit, so that a ragged batch
// runs as one wave of workgroups of about equal size instead of splits sized
// for its longest sequence.  If even the largest split needs more workgroups
// than there are compute units, the automatic plan for the longest length.
int mla_attn_plan_lens(const mla_dims* d, int32_t B, const int32_t* host_lens,
                       int32_t* rows_per_split, int32_t* num_splits) {
  int st = dims_status(d);
  if (st) return st;
  if (!rows_per_split || !num_splits || (B > 0 && !host_lens)) return MLA_ERR_NULL;
  if (B < 0) return MLA_ERR_DIMS;
  int32_t max_len = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (host_lens[b] < 0) return MLA_ERR_DIMS;
    max_len = host_lens[b] > max_len ? host_lens[b] : max_len;
  }
  const int64_t cus = device_cus();
  auto workgroups = [&](int64_t r) {
    int64_t n = 0;
    for (int32_t b = 0; b < B; ++b) n += (host_lens[b] + r - 1) / r;
    return n;
  };
  int64_t lo = kMinSplitRows / 64, hi = max_split_rows(d) / 64;  // in units of 64 rows
  if (hi > 1 << 24) hi = 1 << 24;
  if (max_len == 0 || workgroups(hi * 64) > cus) return plan(d, B, max_len, 0, rows_per_split, num_splits);
  while (lo < hi) {  // smallest r with workgroups(r) <= cus (monotone in r)
    const int64_t mid = (lo + hi) / 2;
    if (workgroups(mid * 64) <= cus) hi = mid; else lo = mid + 1;
  }
  return plan(d, B, max_len, (int32_t)(lo * 64), rows_per_split, num_splits);
}

// Arguments of the append kernels for pre-norm rows given as S partial sums.
static AppendArgs append_args(const mla_dims* d, int32_t B, const float* kv_pre, int kv_splits,
                              const mla_weight* kv_a_norm, const mla_rope* rope,
                              const int32_t* positions, const int32_t* token_seq, int32_t num_seqs,
                              const mla_cache* cache, int32_t* dev_status) {
  AppendArgs a{};
  a.kv_pre = kv_pre;
  a.kv_splits = kv_splits;
  a.kv_split_stride = (int64_t)B * (d->kv_lora + d->qk_rope);
  a.gamma = view(kv_a_norm);
  a.inv_freq = rope->inv_freq;
  a.rope_mscale = rope->mscale;
  a.positions = positions;
  a.pool = cache->pool;
  a.table = cache->block_table;
  a.q_seq = token_seq;
  a.num_seqs = num_seqs;
  a.dev_status = dev_status;
  a.B = B;
  a.C = d->kv_lora;
  a.R = d->qk_rope;
  a.block = d->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.cache_dtype = d->cache_dtype;
  a.eps = d->rms_eps;
  return a;
}

// token_seq null: token b owns table row b (num_seqs = B).  dry: validate only.
static int cache_append_impl(const mla_dims* d, int32_t B, const float* x, const mla_weight* kv_a,
                             const mla_weight* kv_a_norm, const mla_rope* rope,
                             const int32_t* positions, const int32_t* token_seq, int32_t num_seqs,
                             const mla_cache* cache, int32_t* dev_status, void* ws,
                             size_t ws_bytes, void* stream, bool dry) {
  int st = dims_status(d);
  if (st) return st;
  if (B < 0) return MLA_ERR_DIMS;
  if (B > 0 && num_seqs < 1) return MLA_ERR_DIMS;
  const int W = d->kv_lora + d->qk_rope;
  if (!x || !rope || !rope->inv_freq || !positions || !cache || !cache->pool ||
      !cache->block_table)
    return MLA_ERR_NULL;
  if (cache->num_blocks < 1 || cache->max_blocks_per_seq < 1) return MLA_ERR_DIMS;
  if ((st = check_weight(kv_a_norm, 1, d->kv_lora, false))) return st;
  if (d->hidden > 0 && (st = check_weight(kv_a, W, d->hidden, true))) return st;
  const size_t need = ws_append(d, B);
  if (need && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (dry || B == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const float* kv_pre = x;
  int kv_splits = 1;
  if (d->hidden > 0) {
    char* base = static_cast<char*>(ws);
    GemmArgs g{};
    g.w = view(kv_a);
    g.x = x;
    g.x_b = d->hidden;
    g.y = reinterpret_cast<float*>(base + align_up(packed_bytes(1, B, d->hidden)));
    g.y_b = W;
    g.y_s = (int64_t)B * W;
    g.O = W;
    g.K = d->hidden;
    g.B = B;
    g.Z = 1;
    if (gemm_mfma_ok(g)) {
      g.xp = reinterpret_cast<_Float16*>(base);
      int32_t* x_exp = reinterpret_cast<int32_t*>(
          base + align_up(packed_bytes(1, B, d->hidden)) +
          align_up((size_t)gemm_max_splits(d->hidden) * B * W * 4));
      g.x_exp = x_exp;
      if ((st = hip_status(launch_pack_scaled(x, d->hidden, B, d->hidden,
                                              reinterpret_cast<_Float16*>(base), x_exp, s))))
        return st;
    }
    if ((st = hip_status(launch_gemm_nt(g, gemm_max_splits(d->hidden), &kv_splits, s)))) return st;
    kv_pre = g.y;
  }
  const AppendArgs a = append_args(d, B, kv_pre, kv_splits, kv_a_norm, rope, positions, token_seq,
                                   num_seqs, cache, dev_status);
  return hip_status(launch_append_rows(a, s));
}

int mla_cache_append(const mla_dims* d, int32_t B, const float* x, const mla_weight* kv_a,
                     const mla_weight* kv_a_norm, const mla_rope* rope, const int32_t* positions,
                     const mla_cache* cache, int32_t* dev_status, void* ws, size_t ws_bytes,
                     void* stream) {
  return cache_append_impl(d, B, x, kv_a, kv_a_norm, rope, positions, nullptr, B, cache,
                           dev_status, ws, ws_bytes, stream, false);
}

int mla_cache_append_tokens(const mla_dims* d, int32_t n_tokens, const float* x,
                            const mla_weight* kv_a, const mla_weight* kv_a_norm,
                            const mla_rope* rope, const int32_t* positions,
                            const int32_t* token_seq, int32_t num_seqs, const mla_cache* cache,
                            int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  if (!token_seq) return MLA_ERR_NULL;
  return cache_append_impl(d, n_tokens, x, kv_a, kv_a_norm, rope, positions, token_seq, num_seqs,
                           cache, dev_status, ws, ws_bytes, stream, false);
}

static AbsorbArgs absorb_args(const mla_dims* d, int32_t B, const float* q, const mla_weight* kv_b,
                              const mla_rope* rope, const int32_t* positions, void* q_abs) {
  AbsorbArgs a{};
  a.q = q;
  a.kv_b = view(kv_b);
  a.inv_freq = rope->inv_freq;
  a.rope_mscale = rope->mscale;
  a.positions = positions;
  a.q_abs = q_abs;
  a.B = B;
  a.H = d->num_heads;
  a.N = d->qk_nope;
  a.R = d->qk_rope;
  a.V = d->v_head;
  a.C = d->kv_lora;
  a.cache_dtype = d->cache_dtype;
  return a;
}

// Workspace regions of the q chain (mla_absorb_q): x packed, q_a partial sums,
// q latent packed, q fp32.
struct AbsorbWs {
  _Float16* x_pk;
  float* q_part;
  _Float16* q_lat_pk;
  float* q_full;
  int32_t* x_exp;
  int32_t* q_lat_exp;
};
static AbsorbWs absorb_ws(const mla_dims* d, int32_t B, void* ws) {
  char* base = static_cast<char*>(ws);
  AbsorbWs r{};
  r.x_pk = reinterpret_cast<_Float16*>(base);
  base += align_up(packed_bytes(1, B, d->hidden));
  r.q_part = reinterpret_cast<float*>(base);
  base += ws_q_part(d, B);
  r.q_lat_pk = reinterpret_cast<_Float16*>(base);
  base += align_up(packed_bytes(1, B, d->q_lora));
  r.q_full = reinterpret_cast<float*>(base);
  base += align_up((size_t)B * d->num_heads * (d->qk_nope + d->qk_rope) * 4);
  r.x_exp = reinterpret_cast<int32_t*>(base);
  r.q_lat_exp = reinterpret_cast<int32_t*>(base + align_up((size_t)B * 4));
  return r;
}

// q_b of the q chain: q latent (packed on the MFMA path, else the normalised
// fp32 partials in place) -> q fp32 [B, H, N+R].
static GemmArgs q_b_gemm(const mla_dims* d, int32_t B, const mla_weight* q_b, const AbsorbWs& r) {
  GemmArgs g2{};
  g2.w = view(q_b);
  g2.x = r.q_part;  // normalised in place on the fp32 path
  g2.x_b = d->q_lora;
  g2.y = r.q_full;
  g2.y_b = (int64_t)d->num_heads * (d->qk_nope + d->qk_rope);
  g2.O = d->num_heads * (d->qk_nope + d->qk_rope);
  g2.K = d->q_lora;
  g2.B = B;
  g2.Z = 1;
  if (gemm_mfma_ok(g2)) {
    g2.xp = r.q_lat_pk;
    g2.x_exp = r.q_lat_exp;
  }
  return g2;
}

// dry: validate only.
static int absorb_impl(const mla_dims* d, int32_t B, const float* q_in, const mla_weight* q_a,
                       const mla_weight* q_a_norm, const mla_weight* q_b, const mla_weight* kv_b,
                       const mla_rope* rope, const int32_t* positions, void* q_abs, void* ws,
                       size_t ws_bytes, void* stream, bool dry) {
  int st = dims_status(d);
  if (st) return st;
  if (B < 0) return MLA_ERR_DIMS;
  const int H = d->num_heads, N = d->qk_nope, R = d->qk_rope, V = d->v_head, C = d->kv_lora;
  if (N < 1 || N > 4096) return MLA_ERR_DIMS;
  if (!q_in || !rope || !rope->inv_freq || !positions || !q_abs) return MLA_ERR_NULL;
  if ((st = check_weight(kv_b, (int64_t)H * (N + V), C, true, true))) return st;
  if (q_a) {
    if (d->q_lora < 1 || d->hidden < 1) return MLA_ERR_DIMS;
    if ((st = check_weight(q_a, d->q_lora, d->hidden, true))) return st;
    if ((st = check_weight(q_a_norm, 1, d->q_lora, false))) return st;
    if ((st = check_weight(q_b, (int64_t)H * (N + R), d->q_lora, true))) return st;
    const size_t need = ws_absorb(d, B);
    if (!ws || ws_bytes < need) return MLA_ERR_WORKSPACE;
  } else if (q_b) {
    return MLA_ERR_DIMS;  // q_b without q_a
  }
  if (dry || B == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const float* q = q_in;
  if (q_a) {
    const AbsorbWs r = absorb_ws(d, B, ws);
    GemmArgs g{};
    g.w = view(q_a);
    g.x = q_in;
    g.x_b = d->hidden;
    g.y = r.q_part;
    g.y_b = d->q_lora;
    g.y_s = (int64_t)B * d->q_lora;
    g.O = d->q_lora;
    g.K = d->hidden;
    g.B = B;
    g.Z = 1;
    const GemmArgs g2 = q_b_gemm(d, B, q_b, r);
    if (gemm_mfma_ok(g)) {
      g.xp = r.x_pk;
      g.x_exp = r.x_exp;
      if ((st = hip_status(launch_pack_scaled(q_in, d->hidden, B, d->hidden, r.x_pk, r.x_exp, s))))
        return st;
    }
    int splits = 1;
    if ((st = hip_status(launch_gemm_nt(g, gemm_max_splits(d->hidden), &splits, s)))) return st;
    if ((st = hip_status(launch_rmsnorm_rows(r.q_part, splits, g.y_s, B, d->q_lora, d->q_lora,
                                             view(q_a_norm), d->rms_eps,
                                             g2.xp ? nullptr : r.q_part,
                                             g2.xp ? r.q_lat_pk : nullptr,
                                             g2.xp ? r.q_lat_exp : nullptr, s))))
      return st;
    const AbsorbArgs ab = absorb_args(d, B, r.q_full, kv_b, rope, positions, q_abs);
    if (qb_absorb_ok(g2, ab)) return hip_status(launch_qb_absorb(g2, ab, s));
    if ((st = hip_status(launch_gemm_nt(g2, 1, &splits, s)))) return st;
    q = r.q_full;
  }
  return hip_status(launch_absorb(absorb_args(d, B, q, kv_b, rope, positions, q_abs), s));
}

int mla_absorb_q(const mla_dims* d, int32_t B, const float* q_in, const mla_weight* q_a,
                 const mla_weight* q_a_norm, const mla_weight* q_b, const mla_weight* kv_b,
                 const mla_rope* rope, const int32_t* positions, void* q_abs, void* ws,
                 size_t ws_bytes, void* stream) {
  return absorb_impl(d, B, q_in, q_a, q_a_norm, q_b, kv_b, rope, positions, q_abs, ws, ws_bytes,
                     stream, false);
}

// token_seq null: query b reads table row b (num_seqs = B).  dry: validate
// only.  vc_pk: where the merge of the MFMA kernel's split partials also
// writes v_combine in the packed fp16 layout of W_UV's input (*vc_written
// says whether it did: only with more than one split on a bf16 cache).  uv:
// W_UV of the step, which the merge then applies itself where the shapes
// allow (*uv_done).
static int attn_impl(const mla_dims* d, int32_t B, const void* q_abs, const mla_cache* cache,
                     const int32_t* token_seq, int32_t num_seqs, const int32_t* seq_lens,
                     int32_t max_len, float softmax_scale, int32_t split_rows, float* v_combine,
                     float* lse, void* ws, size_t ws_bytes, void* stream, bool dry,
                     _Float16* vc_pk = nullptr, bool* vc_written = nullptr,
                     const GemmArgs* uv = nullptr, bool* uv_done = nullptr) {
  if (vc_written) *vc_written = false;
  if (uv_done) *uv_done = false;
  int st = dims_status(d);
  if (st) return st;
  if (B < 0 || max_len < 0) return MLA_ERR_DIMS;
  if (B > 0 && num_seqs < 1) return MLA_ERR_DIMS;
  if (!q_abs || !cache || !cache->pool || !cache->block_table || !seq_lens || !v_combine)
    return MLA_ERR_NULL;
  if (cache->num_blocks < 1 || cache->max_blocks_per_seq < 1) return MLA_ERR_DIMS;
  if (!isfinite(softmax_scale)) return MLA_ERR_DIMS;
  if ((int64_t)max_len > (int64_t)cache->max_blocks_per_seq * d->block_size) return MLA_ERR_CAPACITY;
  const bool bf16 = d->cache_dtype == MLA_BF16;
  if (bf16) {
    if (d->num_heads != 128 || d->kv_lora != 512 || d->qk_rope != 64 || (d->block_size % 32) != 0)
      return MLA_ERR_UNSUPPORTED;
  } else {
    if (d->kv_lora > 1024 || d->kv_lora + d->qk_rope > 8192 || (d->kv_lora % 4) != 0)
      return MLA_ERR_UNSUPPORTED;
  }
  int32_t rows = 0, splits = 1;
  if ((st = plan(d, B, max_len, split_rows, &rows, &splits))) return st;
  const size_t need = ws_attn(d, B, splits);
  if (need && (!ws || ws_bytes < need)) return MLA_ERR_WORKSPACE;
  if (dry || B == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);

  AttnArgs a{};
  a.q_abs = q_abs;
  a.pool = cache->pool;
  a.table = cache->block_table;
  a.q_seq = token_seq;
  a.num_seqs = num_seqs;
  a.seq_lens = seq_lens;
  a.v_combine = v_combine;
  a.lse = lse;
  if (splits > 1) {
    char* base = static_cast<char*>(ws);
    if (bf16) a.part_oh = reinterpret_cast<_Float16*>(base);
    else a.part_o = reinterpret_cast<float*>(base);
    base += ws_attn_o(d, B, splits);
    a.part_lse = reinterpret_cast<float*>(base);
    if (bf16) {
      const size_t lse = align_up((size_t)B * splits * d->num_heads * 4);
      a.part_exp = reinterpret_cast<float*>(base + lse);
      a.part_first = reinterpret_cast<int32_t*>(base + 2 * lse);
      // automatic plan, packed grid, more than one query: the kernel sizes the
      // splits from the lengths, with at most one non-empty split per compute
      // unit (and never more than the slots the workspace holds)
      if (split_rows == 0 && B >= 2 && B <= 4096) {
        const int64_t slots = (int64_t)B * splits, cus = device_cus();
        a.auto_slots = (int32_t)(slots < cus ? slots : cus);
      }
      a.vc_pk = vc_pk;
      if (vc_written) *vc_written = vc_pk != nullptr;
    }
  }
  a.B = B;
  a.H = d->num_heads;
  a.C = d->kv_lora;
  a.R = d->qk_rope;
  a.block = d->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  a.max_len = max_len;
  a.split_rows = rows;
  a.num_splits = splits;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  st = hip_status(bf16 ? launch_attn_mfma_bf16(a, s) : launch_attn_generic_f32(a, s));
  if (st) return st;
  if (splits > 1) {
    if (uv && uv_done && merge_uv_ok(a, *uv)) {
      st = hip_status(launch_merge_uv(a, *uv, s));
      *uv_done = st == MLA_OK;
    } else {
      st = hip_status(launch_attn_combine(a, s));
    }
  }
  return st;
}

int mla_decode_attn(const mla_dims* d, int32_t B, const void* q_abs, const mla_cache* cache,
                    const int32_t* seq_lens, int32_t max_len, float softmax_scale,
                    int32_t split_rows, float* v_combine, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  return attn_impl(d, B, q_abs, cache, nullptr, B, seq_lens, max_len, softmax_scale, split_rows,
                   v_combine, lse, ws, ws_bytes, stream, false);
}

int mla_decode_attn_noalloc(const mla_dims* d, int32_t B, const void* q_abs,
                            const mla_cache* cache, const int32_t* seq_lens, int32_t max_len,
                            float softmax_scale, int32_t split_rows, float* v_combine, float* lse,
                            void* stream) {
  int st = dims_status(d);
  if (st) return st;
  if (B < 0 || max_len < 0) return MLA_ERR_DIMS;
  int32_t rows = 0, splits = 1;
  if ((st = plan(d, B, max_len, split_rows, &rows, &splits))) return st;
  if (ws_attn(d, B, splits) > kScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (splits > 1 && !(ws = scratch_ptr())) return MLA_ERR_HIP;
  return attn_impl(d, B, q_abs, cache, nullptr, B, seq_lens, max_len, softmax_scale, split_rows,
                   v_combine, lse, ws, ws ? kScratchBytes : 0, stream, false);
}

int mla_attn_tokens(const mla_dims* d, int32_t n_tokens, const void* q_abs,
                    const mla_cache* cache, const int32_t* token_seq, int32_t num_seqs,
                    const int32_t* seq_lens, int32_t max_len, float softmax_scale,
                    int32_t split_rows, float* v_combine, float* lse, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!token_seq) return MLA_ERR_NULL;
  return attn_impl(d, n_tokens, q_abs, cache, token_seq, num_seqs, seq_lens, max_len,
                   softmax_scale, split_rows, v_combine, lse, ws, ws_bytes, stream, false);
}

// W_UV (per head, z = head) and the optional o_proj of mla_out_proj over the
// workspace at base (may be null when nothing runs on the MFMA path): v_combine
// packed at the start, then the per-head outputs.
static void out_gemms(const mla_dims* d, int32_t B, const float* v_combine, const mla_weight* kv_b,
                      const mla_weight* o_proj, float* out, char* base, GemmArgs* pg, GemmArgs* pg2) {
  const int H = d->num_heads, N = d->qk_nope, V = d->v_head, C = d->kv_lora;
  _Float16* vc_pk = reinterpret_cast<_Float16*>(base);
  void* heads = base ? base + align_up(packed_bytes(H, B, C)) : nullptr;
  GemmArgs g{};
  g.w = view(kv_b);
  g.w_row0 = N;
  g.w_zrows = N + V;
  g.x = v_combine;
  g.x_b = (int64_t)H * C;
  g.x_z = C;
  g.y = out;
  g.y_b = (int64_t)H * V;
  g.y_z = V;
  g.O = V;
  g.K = C;
  g.B = B;
  g.Z = H;
  GemmArgs g2{};
  if (o_proj) {
    g2.w = view(o_proj);
    g2.x = static_cast<const float*>(heads);
    g2.x_b = (int64_t)H * V;
    g2.y = out;
    g2.y_b = d->hidden;
    g2.O = d->hidden;
    g2.K = H * V;
    g2.B = B;
    g2.Z = 1;
    g.y = static_cast<float*>(heads);
    if (gemm_mfma_ok(g2)) {  // W_UV writes packed fp16 straight for the MFMA path
      g2.xp = static_cast<const _Float16*>(heads);
      g.y = nullptr;
      g.yp = static_cast<_Float16*>(heads);
      g.yp_K = (int64_t)H * V;
    }
  }
  if (gemm_mfma_ok(g)) g.xp = vc_pk;
  *pg = g;
  *pg2 = g2;
}

// dry: validate only.  vc_ready: the packed v_combine is already at the start
// of the workspace (written by the attention merge); uv_done: so are W_UV's
// outputs, and only o_proj runs.
static int out_proj_impl(const mla_dims* d, int32_t B, const float* v_combine,
                         const mla_weight* kv_b, const mla_weight* o_proj, float* out, void* ws,
                         size_t ws_bytes, void* stream, bool dry, bool vc_ready,
                         bool uv_done = false) {
  int st = dims_status(d);
  if (st) return st;
  if (B < 0) return MLA_ERR_DIMS;
  const int H = d->num_heads, N = d->qk_nope, V = d->v_head, C = d->kv_lora;
  if (!v_combine || !out) return MLA_ERR_NULL;
  if ((st = check_weight(kv_b, (int64_t)H * (N + V), C, true, true))) return st;
  if (o_proj) {
    if (d->hidden < 1) return MLA_ERR_DIMS;
    if ((st = check_weight(o_proj, d->hidden, (int64_t)H * V, true))) return st;
    if (!ws || ws_bytes < ws_out(d, B)) return MLA_ERR_WORKSPACE;
  }
  if (B == 0) return MLA_OK;
  GemmArgs g, g2;
  out_gemms(d, B, v_combine, kv_b, o_proj, out, static_cast<char*>(ws), &g, &g2);
  const bool mfma = gemm_mfma_ok(g);
  if (mfma && (!ws || ws_bytes < ws_out(d, B))) return MLA_ERR_WORKSPACE;
  if (dry) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma && !vc_ready && !uv_done) {
    if ((st = hip_status(launch_pack_f16(v_combine, (int64_t)H * C, C, H, B, C,
                                         const_cast<_Float16*>(g.xp), s))))
      return st;
  }
  int splits = 1;
  if (!uv_done && (st = hip_status(launch_gemm_nt(g, 1, &splits, s)))) return st;
  if (o_proj) st = hip_status(launch_gemm_nt(g2, 1, &splits, s));
  return st;
}

int mla_out_proj(const mla_dims* d, int32_t B, const float* v_combine, const mla_weight* kv_b,
                 const mla_weight* o_proj, float* out, void* ws, size_t ws_bytes, void* stream) {
  return out_proj_impl(d, B, v_combine, kv_b, o_proj, out, ws, ws_bytes, stream, false, false);
}

// Front of mla_decode_layer when both projections of x run on the MFMA path
// with one weight type: x is packed once, kv_a and q_a run in one launch, the
// append and the q-latent RMSNorm in one launch, then q_b and the absorb as in
// mla_absorb_q.  Every launch computes what the separate calls compute, in the
// same arithmetic.  Returns kNotFused, having launched nothing, when the shapes
// do not allow it.  ws_a / ws_b: the append and absorb regions.
constexpr int kNotFused = 1;
static int layer_front_fused(const mla_dims* d, int32_t B, const float* x, const mla_layer* w,
                             const int32_t* positions, const mla_cache* cache,
                             int32_t* dev_status, void* q_abs, char* ws_a, char* ws_b,
                             hipStream_t s) {
  if (d->hidden <= 0 || !w->q_a || B <= 0) return kNotFused;
  const int W = d->kv_lora + d->qk_rope;
  _Float16* x_pk = reinterpret_cast<_Float16*>(ws_a);
  float* kv_part = reinterpret_cast<float*>(ws_a + align_up(packed_bytes(1, B, d->hidden)));
  int32_t* x_exp = reinterpret_cast<int32_t*>(
      ws_a + align_up(packed_bytes(1, B, d->hidden)) +
      align_up((size_t)gemm_max_splits(d->hidden) * B * W * 4));
  const AbsorbWs r = absorb_ws(d, B, ws_b);
  GemmArgs ga{};  // kv_a, as in mla_cache_append
  ga.w = view(w->kv_a);
  ga.x = x;
  ga.xp = x_pk;
  ga.x_exp = x_exp;
  ga.x_b = d->hidden;
  ga.y = kv_part;
  ga.y_b = W;
  ga.y_s = (int64_t)B * W;
  ga.O = W;
  ga.K = d->hidden;
  ga.B = B;
  ga.Z = 1;
  GemmArgs gq{};  // q_a, as in mla_absorb_q
  gq.w = view(w->q_a);
  gq.x = x;
  gq.xp = x_pk;
  gq.x_exp = x_exp;
  gq.x_b = d->hidden;
  gq.y = r.q_part;
  gq.y_b = d->q_lora;
  gq.y_s = (int64_t)B * d->q_lora;
  gq.O = d->q_lora;
  gq.K = d->hidden;
  gq.B = B;
  gq.Z = 1;
  const GemmArgs g2 = q_b_gemm(d, B, w->q_b, r);
  AppendArgs a = append_args(d, B, kv_part, 1, w->kv_a_norm, w->rope, positions, nullptr, B, cache,
                             dev_status);
  QNormArgs qn{};
  qn.part = r.q_part;
  qn.S = 1;
  qn.split_stride = gq.y_s;
  qn.n = d->q_lora;
  qn.stride = d->q_lora;
  qn.gamma = view(w->q_a_norm);
  qn.eps = d->rms_eps;
  qn.yp = g2.xp ? r.q_lat_pk : nullptr;
  qn.yexp = r.q_lat_exp;
  if (!gemm_pair_ok(ga, gq) || !g2.xp || !append_qnorm_ok(a, qn)) return kNotFused;
  int st;
  if ((st = hip_status(launch_pack_scaled(x, d->hidden, B, d->hidden, x_pk, x_exp, s)))) return st;
  int splits = 1;
  if ((st = hip_status(launch_gemm_pair(ga, gq, gemm_max_splits(d->hidden), &splits, s)))) return st;
  a.kv_splits = splits;
  qn.S = splits;
  if ((st = hip_status(launch_append_qnorm(a, qn, s)))) return st;
  const AbsorbArgs ab = absorb_args(d, B, r.q_full, w->kv_b, w->rope, positions, q_abs);
  if (qb_absorb_ok(g2, ab)) return hip_status(launch_qb_absorb(g2, ab, s));
  if ((st = hip_status(launch_gemm_nt(g2, 1, &splits, s)))) return st;
  return hip_status(launch_absorb(ab, s));
}

size_t mla_layer_workspace_bytes(const mla_dims* d, int32_t B, int32_t max_len, int32_t split_rows) {
  if (!dims_ok(d) || B < 0) return 0;
  int32_t rows = 0, splits = 1;
  if (plan(d, B, max_len, split_rows, &rows, &splits) != MLA_OK) return 0;
  return ws_layer(d, B, splits) + kAlign;
}

int mla_decode_layer(const mla_dims* d, int32_t B, const float* x, const float* q_in,
                     const mla_layer* w, const int32_t* positions, const mla_cache* cache,
                     const int32_t* seq_lens, int32_t max_len, float softmax_scale,
                     int32_t split_rows, void* q_abs, float* v_combine, float* lse, float* out,
                     int32_t* dev_status, void* ws, size_t ws_bytes, void* stream) {
  int st = dims_status(d);
  if (st) return st;
  if (!w) return MLA_ERR_NULL;
  if (B < 0 || max_len < 0) return MLA_ERR_DIMS;
  int32_t rows = 0, splits = 1;
  if ((st = plan(d, B, max_len, split_rows, &rows, &splits))) return st;
  const size_t wa = ws_append(d, B), wb = ws_absorb(d, B), wc = ws_attn(d, B, splits);
  const size_t wo = ws_out(d, B);
  if (wa + wb + wc + wo > 0 && (!ws || ws_bytes < wa + wb + wc + wo)) return MLA_ERR_WORKSPACE;
  char* ws_a = static_cast<char*>(ws);
  char* ws_b = ws_a ? ws_a + wa : nullptr;
  char* ws_c = ws_a ? ws_b + wb : nullptr;
  char* ws_o = ws_a ? ws_c + wc : nullptr;
  const float* qx = w->q_a ? x : q_in;
  // every step's arguments are checked before anything is enqueued
  if ((st = cache_append_impl(d, B, x, w->kv_a, w->kv_a_norm, w->rope, positions, nullptr, B, cache,
                              dev_status, ws_a, wa, stream, true)))
    return st;
  if ((st = absorb_impl(d, B, qx, w->q_a, w->q_a_norm, w->q_b, w->kv_b, w->rope, positions, q_abs,
                        ws_b, wb, stream, true)))
    return st;
  if ((st = attn_impl(d, B, q_abs, cache, nullptr, B, seq_lens, max_len, softmax_scale, split_rows,
                      v_combine, lse, ws_c, wc, stream, true)))
    return st;
  if ((st = out_proj_impl(d, B, v_combine, w->kv_b, w->o_proj, out, ws_o, wo, stream, true, false)))
    return st;
  if (B == 0) return MLA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = layer_front_fused(d, B, x, w, positions, cache, dev_status, q_abs, ws_a, ws_b, s);
  if (st == kNotFused) {
    st = cache_append_impl(d, B, x, w->kv_a, w->kv_a_norm, w->rope, positions, nullptr, B, cache,
                           dev_status, ws_a, wa, stream, false);
    if (!st)
      st = absorb_impl(d, B, qx, w->q_a, w->q_a_norm, w->q_b, w->kv_b, w->rope, positions, q_abs,
                       ws_b, wb, stream, false);
  }
  if (st) return st;
  // the merge writes W_UV's packed input itself when W_UV runs on the MFMA path,
  // and applies W_UV too where merge_uv_ok allows
  GemmArgs g, g2;
  out_gemms(d, B, v_combine, w->kv_b, w->o_proj, out, ws_o, &g, &g2);
  _Float16* vc_pk = gemm_mfma_ok(g) ? const_cast<_Float16*>(g.xp) : nullptr;
  bool packed = false, uv_done = false;
  if ((st = attn_impl(d, B, q_abs, cache, nullptr, B, seq_lens, max_len, softmax_scale, split_rows,
                      v_combine, lse, ws_c, wc, stream, false, vc_pk, &packed, &g, &uv_done)))
    return st;
  return out_proj_impl(d, B, v_combine, w->kv_b, w->o_proj, out, ws_o, wo, stream, false, packed,
                       uv_done);
}

}  // extern "C"
