/*
 * mla.h -- C ABI of the MLA latent-KV decode library (MI355X / gfx950).
 *
 * Single-token decode of Multi-head Latent Attention with weight absorption,
 * split into the four calls the source pages' per-layer flow is made of:
 *
 *   mla_cache_append  kv_a projection -> RMSNorm of the latent half -> YaRN
 *                     RoPE of k_pe (consecutive pairs) -> one rounded row
 *                     written into a paged cache slot.
 *   mla_absorb_q      optional q chain (q_a -> RMSNorm -> q_b), then
 *                     q' = W_UK^T q_nope per head and RoPE of q_pe, packed
 *                     as q_abs = [q' ; q_pe] rows.
 *   mla_decode_attn   scores of q_abs against every cached row [c_kv ; k_pe],
 *                     scaled softmax, v_combine = sum_t p_t c_kv[t]; split-K
 *                     over rows with an online-softmax combine.
 *   mla_out_proj      out_h = W_UV_h v_combine_h, then optionally o_proj.
 *
 * Sources (page title and item):
 *   moeflux 0.1.0-pre.3, src/riir/attn/mla_attn_forward.rs --
 *     mla_attn_layer_forward_gpu (the step order, one command buffer, the
 *     caller owns the pre-norm and the residual, len bumped after append),
 *     MlaForwardGpuError (error taxonomy), MlaYarnTables (YaRN table + mscale).
 *   turbospark-runtime 0.3.0, src/families/deepseek2/attn.rs --
 *     encode_mla_attention_block (fused cache row [latent ; k_pe], in-place
 *     norm and rope, absorb into fused q_abs rows, MQA decode over pos+1 rows,
 *     v-combine, o_proj), validate_q8_0_matrix (validate before any kernel
 *     receives a raw offset).
 *   moeflux 0.1.0-pre.3, src/riir/backend/gpu/gpu_matvec.rs -- MatvecSpec
 *     (4-bit affine weights: packed nibbles, bf16 scales and biases, group 64;
 *     caller-owned input/output buffers).
 *
 * Conventions for every call
 *   - Pointers marked "device" are HIP device addresses; "host" are CPU
 *     addresses read before the call returns.  The caller owns every buffer
 *     (inputs, outputs, the cache pool, block table, lengths and workspace);
 *     the library allocates nothing, keeps no state and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Device buffers must stay valid until that work completes.
 *   - Every argument is validated on the host first.  On any error the call
 *     returns a negative MLA_ERR_* code and enqueues nothing, except
 *     MLA_ERR_HIP, which reports a launch failure after validation passed.
 *   - Layouts are row-major and dense.  bf16 values are raw 16-bit patterns.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (MlaForwardGpuError, mapped to integers) ---- */
enum {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL (CacheNotReady, MissingTensor) */
  MLA_ERR_DIMS = -2,        /* inconsistent or out-of-range sizes (shape checks) */
  MLA_ERR_DTYPE = -3,       /* a dtype code this call does not take */
  MLA_ERR_UNSUPPORTED = -4, /* valid dims with no compiled kernel (NotMlaVariant) */
  MLA_ERR_CAPACITY = -5,    /* max_seq_len exceeds the block table (CacheFull) */
  MLA_ERR_WORKSPACE = -6,   /* workspace pointer NULL or smaller than required */
  MLA_ERR_HIP = -7          /* a kernel launch failed */
};

/* ---- element types ---- */
enum {
  MLA_F32 = 0,   /* IEEE float32 */
  MLA_BF16 = 1,  /* bfloat16 bit patterns (uint16) */
  MLA_Q4G64 = 2, /* 4-bit affine, group 64 along the input dim (weights only) */
  MLA_Q8_0 = 3,  /* 8-bit blocks of 32 with a binary16 scale (kv_b only) */
  MLA_Q4G64_T = 4 /* MLA_Q4G64 repacked in MFMA fragment order (mla_repack_q4g64) */
};

/* ---- device status flags OR-ed by mla_cache_append (dev_status) ---- */
enum {
  MLA_DEV_POS_RANGE = 1,  /* positions[b] < 0 or >= max_blocks_per_seq * block_size */
  MLA_DEV_BAD_BLOCK = 2,  /* block_table entry for that row is < 0 or >= num_blocks */
  MLA_DEV_BAD_SEQ = 4     /* mla_cache_append_tokens: token_seq[t] < 0 or >= num_seqs */
};

/* Model geometry.  W = kv_lora + qk_rope is the cache row width. */
typedef struct mla_dims {
  int32_t num_heads;   /* H: query heads */
  int32_t qk_nope;     /* N: per-head no-position query/key dims */
  int32_t qk_rope;     /* R: rotary dims (even) */
  int32_t v_head;      /* V: per-head value dims */
  int32_t kv_lora;     /* C: latent (compressed KV) dims */
  int32_t hidden;      /* model width; 0 = the projections are not used */
  int32_t q_lora;      /* q LoRA rank; 0 = q is given directly */
  int32_t block_size;  /* rows per cache block (paged pool) */
  int32_t cache_dtype; /* MLA_F32 or MLA_BF16: cache rows and q_abs */
  float rms_eps;       /* RMSNorm epsilon */
} mla_dims;

/* A weight matrix [rows (outputs), cols (inputs)], row-major.
 *   MLA_F32 : data = float [rows, cols]
 *   MLA_BF16: data = uint16 [rows, cols]
 *   MLA_Q4G64: data = uint32 [rows, cols/8]; element k of a row sits in word
 *     k/8 at bits 4*(k%8)..+3 (low nibble first); scales, biases = bf16
 *     [rows, cols/64]; w = scale * nibble + bias.  Products with a Q4G64
 *     weight whose depth is a multiple of 128 run on fp16 MFMA: w and the
 *     activations are rounded to fp16 (11-bit significands), sums are fp32.
 *     The hidden state and the normalised q latent are first scaled per
 *     token by a power of two that brings their largest magnitude into
 *     [2^14, 2^15) (undone exactly on the fp32 results), as is each token's
 *     q_nope per head before the W_UK product, so no value overflows fp16 or
 *     falls into its subnormals.  v_combine and the per-head W_UV outputs
 *     enter W_UV and o_proj unscaled: they are bounded by the cache latents
 *     (|c| <= sqrt(C) max|kv_a_norm gamma|) times the weights.
 *   MLA_Q4G64_T: the same values as MLA_Q4G64, repacked by mla_repack_q4g64
 *     (rows a multiple of 32, cols of 128) so that the 4-bit MFMA products
 *     read them in whole lines: for row tile t = r/32 and unit u = k/128, a
 *     2048-byte block at (t * cols/128 + u) * 2048 holds two 1 KB parts; lane
 *     L = r%32 + 32*h (h = (k%128)/64) owns 16 bytes at part*1024 + 16*L,
 *     part = (k%64)/32, with the row-major format's nibble order inside (the
 *     32 elements 64h + 32*part .. +31 of the unit, low nibble first).
 *     scales and biases: bf16 at (t * cols/128 + u) * 64 + L (group 2u + h of
 *     row r).  Accepted wherever MLA_Q4G64 is; it changes the reads, not the
 *     arithmetic (results equal bit for bit).
 *   MLA_Q8_0: data = bytes, [rows][cols/32] blocks of 34: a little-endian
 *     binary16 scale d, then 32 signed bytes q; element = d * q (turbospark
 *     deepseek2/attn.rs, validate_q8_0_matrix: kv_b read in place; the byte
 *     layout is GGUF's Q8_0).  cols must be a multiple of 32; scales and
 *     biases are unused.  Accepted for kv_b only; products with it run on
 *     the VALU kernels in fp32.
 * A norm weight (gamma) is passed as a 1 x n matrix of MLA_F32 or MLA_BF16.
 * All pointers are device pointers. */
typedef struct mla_weight {
  int32_t dtype;
  int32_t rows;
  int32_t cols;
  const void* data;
  const uint16_t* scales;
  const uint16_t* biases;
} mla_weight;

/* RoPE table: inv_freq = device float [qk_rope/2]; the rotation is
 * multiplied by mscale. */
typedef struct mla_rope {
  const float* inv_freq;
  float mscale;
} mla_rope;

/* Paged latent cache.  pool = device [num_blocks, block_size, W] of
 * cache_dtype; block_table = device int32 [batch, max_blocks_per_seq]:
 * logical row t of sequence b lives at pool[block_table[b][t / block_size]]
 * [t % block_size].  A contiguous cache is the identity table. */
typedef struct mla_cache {
  void* pool;
  const int32_t* block_table;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
} mla_cache;

/* YaRN parameters (MlaYarnTables): theta, scaling factor, original context,
 * beta_fast, beta_slow, mscale, mscale_all_dim. */
typedef struct mla_yarn {
  double theta;
  double factor;
  double original_max_pos;
  double beta_fast;
  double beta_slow;
  double mscale;
  double mscale_all_dim;
} mla_yarn;

/* mla_yarn_tables -- host helper: the YaRN inverse frequencies and scalars
 * (moeflux mla_attn_forward.rs, MlaYarnTables::new; turbospark gptoss/attn.rs
 * module doc, the ramp between two correction dimensions; turbospark
 * deepseek2/attn.rs, the softmax scale (1 + 0.1 mscale ln factor)^2 /
 * sqrt(key_dim)).
 *   inv_freq_host  host float [qk_rope/2], written
 *   rope_mscale    host float, written: get(factor, mscale)/get(factor, mscale_all_dim)
 *   softmax_scale  host float, written: get(factor, mscale_all_dim)^2 / sqrt(qk_head_dim)
 * where get(s, m) = 1 + 0.1 m ln s for s > 1, else 1.  Any output may be NULL.
 * Errors: MLA_ERR_NULL (p), MLA_ERR_DIMS (qk_rope odd or < 2, qk_head_dim < 1,
 * theta <= 1, factor <= 0, original_max_pos <= 0, beta_fast/beta_slow <= 0). */
int mla_yarn_tables(const mla_yarn* p, int32_t qk_rope, int32_t qk_head_dim,
                    float* inv_freq_host, float* rope_mscale, float* softmax_scale);

/* mla_cache_append -- write the new row of each sequence into its slot
 * (moeflux mla_attn_forward.rs: KV-A chain, kv_a_layernorm, YaRN rope on
 * k_pe, mla_kv_cache_append; turbospark deepseek2/attn.rs: kv_a writes the
 * fused row, then in-place latent norm and windowed k_pe rope).
 *   x          device float [batch, hidden]; when dims->hidden == 0 it is the
 *              pre-norm row itself, float [batch, W]
 *   kv_a       [W, hidden] weight (F32, BF16 or Q4G64); ignored if hidden == 0
 *   kv_a_norm  1 x C gamma (F32 or BF16)
 *   rope       k_pe rotation table and multiplier
 *   positions  device int32 [batch]: the row written for sequence b
 *   cache      pool and block table (written: one row per sequence)
 *   dev_status device int32, may be NULL: rows whose position or block is
 *              out of range are skipped and MLA_DEV_* flags OR-ed in
 *   ws         device workspace of at least mla_workspace_bytes() bytes
 * The row is y = [gamma * c / sqrt(mean(c^2) + eps) ; mscale * RoPE(k_pe, pos)]
 * with [c ; k_pe] = W_kva x, computed in fp32 (angles in fp64) and rounded
 * once to cache_dtype (round to nearest even).  The caller advances its
 * sequence lengths afterwards.
 * Errors: NULL, DIMS (batch < 0, shapes, block_size < 1), DTYPE, WORKSPACE. */
int mla_cache_append(const mla_dims* dims, int32_t batch, const float* x,
                     const mla_weight* kv_a, const mla_weight* kv_a_norm,
                     const mla_rope* rope, const int32_t* positions,
                     const mla_cache* cache, int32_t* dev_status,
                     void* ws, size_t ws_bytes, void* stream);

/* mla_absorb_q -- fused latent query rows (moeflux mla_attn_forward.rs: Q
 * chain, mla_q_prime_4bit; turbospark deepseek2/attn.rs: q_pe roped before
 * encode_mla_absorb_q gathers [q' ; q_pe]).
 *   q_in       device float: [batch, H, N+R] when q_a is NULL, else the
 *              pre-norm hidden state [batch, hidden]
 *   q_a        [q_lora, hidden] Q-LoRA down projection or NULL
 *   q_a_norm   1 x q_lora gamma (required with q_a)
 *   q_b        [H*(N+R), q_lora] up projection (required with q_a)
 *   kv_b       [H*(N+V), C]: head h owns rows h*(N+V)..+N-1 (W_UK) then V
 *              rows (W_UV); F32, BF16, Q4G64 or Q8_0
 *   positions  device int32 [batch]: rotation position of each query
 *   q_abs      device [batch, H, W] of cache_dtype, written:
 *              q_abs[b,h,:C] = sum_n W_UK[h,n,:] q_nope[b,h,n] (fp32
 *              accumulate), q_abs[b,h,C:] = mscale * RoPE(q_pe[b,h], pos)
 * Errors: NULL, DIMS, DTYPE, WORKSPACE. */
int mla_absorb_q(const mla_dims* dims, int32_t batch, const float* q_in,
                 const mla_weight* q_a, const mla_weight* q_a_norm,
                 const mla_weight* q_b, const mla_weight* kv_b,
                 const mla_rope* rope, const int32_t* positions, void* q_abs,
                 void* ws, size_t ws_bytes, void* stream);

/* mla_decode_attn -- MQA decode over the compressed rows (moeflux
 * mla_attn_forward.rs: mla_sdpa_folded; turbospark deepseek2/attn.rs:
 * encode_mla_attention_decode, V = the row's first C values).
 *   q_abs        device [batch, H, W] of cache_dtype
 *   cache        pool + block table (read only)
 *   seq_lens     device int32 [batch]: rows attended per sequence (after
 *                the append); 0 gives v_combine = 0 and lse = -inf
 *   max_seq_len  host: upper bound of seq_lens (sizes the split grid);
 *                values above it are clamped to it on the device
 *   softmax_scale  multiplies the fp32 scores
 *   split_rows   rows per split-K partition (multiple of 64; at most 32768
 *                on a bf16 cache), 0 = automatic: on a bf16 cache with 2 to
 *                4096 queries the split kernel sizes the splits from the
 *                lengths on the device (about one non-empty split per compute
 *                unit, within the host plan's workspace), else the host plan
 *                over batch * max_seq_len rows
 *   v_combine    device float [batch, H, C], written
 *   lse          device float [batch, H] or NULL: natural-log sum of exp of
 *                the scaled scores
 * bf16 caches run on the MFMA kernel (H = 128, C = 512, R = 64, block_size a
 * multiple of 32); f32 caches on a VALU kernel of any shape.  With more than
 * one split the bf16 kernel keeps each split's normalised partial in fp16
 * times a power-of-two scale per head that brings the head's largest
 * magnitude into [2^14, 2^15) (2^-11 relative rounding before the fp32
 * merge, at any magnitude); the f32 kernel keeps fp32 partials.
 * Errors: NULL, DIMS (max_seq_len < 0, split_rows), UNSUPPORTED, CAPACITY
 * (max_seq_len > max_blocks_per_seq * block_size), WORKSPACE. */
int mla_decode_attn(const mla_dims* dims, int32_t batch, const void* q_abs,
                    const mla_cache* cache, const int32_t* seq_lens,
                    int32_t max_seq_len, float softmax_scale, int32_t split_rows,
                    float* v_combine, float* lse, void* ws, size_t ws_bytes,
                    void* stream);

/* mla_out_proj -- per-head expansion and output projection (moeflux
 * mla_attn_forward.rs: mla_out_per_head_4bit then o_proj; turbospark
 * deepseek2/attn.rs: encode_mla_v_combine then O_PROJ; the caller adds the
 * residual).
 *   v_combine  device float [batch, H, C]
 *   kv_b       as in mla_absorb_q (W_UV rows are read)
 *   o_proj     [hidden, H*V] or NULL
 *   out        device float: [batch, H, V] when o_proj is NULL, else
 *              [batch, hidden]
 * Errors: NULL, DIMS, DTYPE, WORKSPACE. */
int mla_out_proj(const mla_dims* dims, int32_t batch, const float* v_combine,
                 const mla_weight* kv_b, const mla_weight* o_proj, float* out,
                 void* ws, size_t ws_bytes, void* stream);

/* The weights of one MLA attention layer for mla_decode_layer. */
typedef struct mla_layer {
  const mla_weight* kv_a;       /* as in mla_cache_append (ignored if hidden == 0) */
  const mla_weight* kv_a_norm;  /* as in mla_cache_append */
  const mla_weight* q_a;        /* as in mla_absorb_q, or NULL */
  const mla_weight* q_a_norm;   /* with q_a */
  const mla_weight* q_b;        /* with q_a */
  const mla_weight* kv_b;       /* as in mla_absorb_q and mla_out_proj */
  const mla_weight* o_proj;     /* as in mla_out_proj, or NULL */
  const mla_rope* rope;         /* shared by the k_pe and q_pe rotations */
} mla_layer;

/* mla_decode_layer -- the whole decode step of one layer in one call, the
 * forward the pages encode as a single command buffer (moeflux
 * mla_attn_forward.rs, mla_attn_layer_forward_gpu: kv append, Q chain,
 * absorb, SDPA over the latent cache, per-head W_UV, o_proj, one commit;
 * turbospark deepseek2/attn.rs, encode_mla_attention_block).  Its results are
 * those of mla_cache_append, mla_absorb_q, mla_decode_attn and mla_out_proj
 * called in that order on `stream` with the same arguments:
 *   x          as mla_cache_append's x; with q_a it is also mla_absorb_q's
 *              q_in (the hidden state)
 *   q_in       mla_absorb_q's q_in when layer->q_a is NULL (per-head q
 *              [batch, H, N+R]); ignored otherwise
 *   seq_lens   lengths after this step's append (positions[b] + 1 for a
 *              sequence decoding at positions[b])
 *   q_abs      device [batch, H, W] of cache_dtype, written (the latent query)
 *   v_combine, lse, out   written as by mla_decode_attn and mla_out_proj
 *   ws         device workspace of mla_layer_workspace_bytes() bytes
 * All kernels go on the one stream, with no host synchronisation, so the call
 * can be captured into a HIP graph.  With 4-bit kv_a and q_a of one type
 * (hidden > 0, q_a given) the front runs fused: one fp16 pack of x, kv_a and
 * q_a in one launch, the append and the q-latent RMSNorm in one launch; and
 * when W_UV (4-bit, 128 rows per head) runs on the MFMA path with more than
 * one split, the attention merge and W_UV run as one launch.  On the 4-bit
 * DeepSeek-V3 layer that is 7 kernels: pack, kv_a + q_a, append + norm,
 * q_b + absorb (as in mla_absorb_q), attention, merge + W_UV, o_proj.  Each
 * fused launch does the same arithmetic as the separate calls, so the results
 * equal theirs bit for bit.
 * Errors: those of the four calls, all checked before anything is enqueued. */
int mla_decode_layer(const mla_dims* dims, int32_t batch, const float* x, const float* q_in,
                     const mla_layer* layer, const int32_t* positions, const mla_cache* cache,
                     const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                     int32_t split_rows, void* q_abs, float* v_combine, float* lse, float* out,
                     int32_t* dev_status, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of mla_decode_layer for this geometry, batch, max_seq_len
 * and split_rows (0 = automatic).  Returns 0 for invalid dims. */
size_t mla_layer_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_seq_len,
                                 int32_t split_rows);

/* mla_repack_q4g64 -- a MLA_Q4G64 weight repacked into MLA_Q4G64_T (see
 * mla_weight), once, for the faster 4-bit products: the 4-bit MFMA kernels
 * read a row-major weight in 16 bytes per row for 32 rows per load
 * instruction, the repacked one in 1 KB contiguous per instruction (o_proj
 * at batch 32: the whole out_proj call 29.7 against 39.3 us with the weights
 * in the last-level cache, 50.8 against 63.8 us from HBM).  The tiled format
 * is this library's; the sources' 4-bit format (gpu_matvec.rs MatvecSpec) is
 * the row-major MLA_Q4G64, which stays the input.
 *   src       a MLA_Q4G64 weight, rows a multiple of 32, cols of 128
 *   data      device, rows * cols / 2 bytes, written
 *   scales, biases  device bf16 [rows * cols / 64] each, written
 * The caller then passes {MLA_Q4G64_T, rows, cols, data, scales, biases}.
 * Errors: NULL, DTYPE (src not MLA_Q4G64), DIMS (rows, cols). */
int mla_repack_q4g64(const mla_weight* src, void* data, uint16_t* scales, uint16_t* biases,
                     void* stream);

/* mla_decode_attn_noalloc -- mla_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and arguments, with the
 * split partials kept in a static device array of MLA_NOALLOC_SCRATCH_BYTES
 * that each device holds from the library's load until the process ends,
 * instead of a caller workspace.  The call allocates and frees nothing.
 *   Arguments: as mla_decode_attn, without ws / ws_bytes.
 *   Limit: the split plan's partials (mla_workspace_bytes of an attention-only
 *   geometry, i.e. batch * splits * H * (C * 2 + 8) bytes on a bf16 cache) must
 *   fit the array, else MLA_ERR_WORKSPACE and nothing is enqueued.  The
 *   automatic plan at H = 128, C = 512 needs at most about (256 + batch)
 *   partials of 129 KB while batch < 256, and none from batch 256 up.
 *   Concurrency: every call on one device uses the same array, so calls that
 *   overlap in time on one device (other streams, other threads) race; order
 *   them on one stream.
 * Errors: as mla_decode_attn; WORKSPACE when the plan exceeds the array;
 * HIP when the array's device address cannot be obtained. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int mla_decode_attn_noalloc(const mla_dims* dims, int32_t batch, const void* q_abs,
                            const mla_cache* cache, const int32_t* seq_lens,
                            int32_t max_seq_len, float softmax_scale, int32_t split_rows,
                            float* v_combine, float* lse, void* stream);

/* ---- several tokens per sequence (chunked prefill, multi-token decode) ----
 * moeflux gpu_matvec.rs, encode_matvec_n_tokens: one weight matrix is applied
 * to stacked tokens, each token's arithmetic unchanged.  mla_absorb_q and
 * mla_out_proj already take a batch of tokens (batch = tokens, positions per
 * token); the two calls below add the token -> sequence map that the cache
 * needs.  The pages do not describe attention over several new tokens; the
 * reading taken: every new row is appended first, then the token at position
 * p attends rows 0..p of its sequence (seq_lens[t] = positions[t] + 1), which
 * is what the same tokens give one decode step at a time. */

/* mla_cache_append_tokens -- mla_cache_append for n_tokens tokens that may
 * share sequences: token t's row goes to position positions[t] of
 * block-table row token_seq[t].
 *   token_seq  device int32 [n_tokens], values in [0, num_seqs)
 *   num_seqs   rows of cache->block_table (>= 1 when n_tokens > 0)
 * Other arguments, and the row's arithmetic, are those of mla_cache_append
 * with batch = n_tokens.  A token whose token_seq is out of range is skipped
 * and MLA_DEV_BAD_SEQ is OR-ed into dev_status.  Two tokens naming the same
 * (sequence, position) race.
 * Errors: as mla_cache_append; DIMS also for num_seqs < 1 with tokens. */
int mla_cache_append_tokens(const mla_dims* dims, int32_t n_tokens, const float* x,
                            const mla_weight* kv_a, const mla_weight* kv_a_norm,
                            const mla_rope* rope, const int32_t* positions,
                            const int32_t* token_seq, int32_t num_seqs,
                            const mla_cache* cache, int32_t* dev_status,
                            void* ws, size_t ws_bytes, void* stream);

/* mla_attn_tokens -- mla_decode_attn for n_tokens queries that may share
 * sequences: query t attends the first seq_lens[t] rows of block-table row
 * token_seq[t] (a causal chunk sets seq_lens[t] = positions[t] + 1).
 *   q_abs      device [n_tokens, H, W] of cache_dtype
 *   token_seq  device int32 [n_tokens], values in [0, num_seqs)
 *   num_seqs   rows of cache->block_table (>= 1 when n_tokens > 0)
 *   seq_lens   device int32 [n_tokens]
 *   v_combine  device float [n_tokens, H, C]; lse device float
 *              [n_tokens, H] or NULL
 * Other arguments as mla_decode_attn with batch = n_tokens, and the
 * workspace is mla_workspace_bytes(dims, n_tokens, max_seq_len, split_rows).
 * A query whose token_seq is out of range gets NaN outputs, as a bad
 * block-table entry does.  Each query is its own workgroups' work, as in
 * decode; queries of one sequence read the same rows, mostly from L2.
 * Errors: as mla_decode_attn; DIMS also for num_seqs < 1 with tokens. */
int mla_attn_tokens(const mla_dims* dims, int32_t n_tokens, const void* q_abs,
                    const mla_cache* cache, const int32_t* token_seq, int32_t num_seqs,
                    const int32_t* seq_lens, int32_t max_seq_len, float softmax_scale,
                    int32_t split_rows, float* v_combine, float* lse, void* ws,
                    size_t ws_bytes, void* stream);

/* mla_validate_q8_0_kv_b -- host-side check of a Q8_0 kv_b tensor before it
 * is wrapped as an mla_weight (turbospark deepseek2/attn.rs,
 * validate_q8_0_matrix and its unit test): the dtype must be MLA_Q8_0, the
 * shape (rows, cols) must equal (heads * (nope + v_head), kv_lora), kv_lora
 * must be a positive multiple of 32, and size_bytes must equal
 * rows * (kv_lora / 32) * 34.  Host values only; touches no device.
 * Errors: DTYPE (wrong dtype), DIMS (shape, width, size or an overflow). */
int mla_validate_q8_0_kv_b(int32_t dtype, int64_t rows, int64_t cols, int64_t size_bytes,
                           int32_t heads, int32_t nope, int32_t kv_lora, int32_t v_head);

/* Bytes of workspace that covers every call above for this geometry, batch,
 * max_seq_len and split_rows (0 = automatic).  Returns 0 for invalid dims. */
size_t mla_workspace_bytes(const mla_dims* dims, int32_t batch,
                           int32_t max_seq_len, int32_t split_rows);

/* The split-K plan mla_decode_attn would use: rows per split and splits per
 * sequence.  Returns MLA_OK or an error code. */
int mla_attn_plan(const mla_dims* dims, int32_t batch, int32_t max_seq_len,
                  int32_t split_rows, int32_t* rows_per_split,
                  int32_t* num_splits);

/* A split-K plan for a batch whose lengths the caller knows on the host
 * (host_lens, int32 [batch], each >= 0): the smallest split (a multiple of 64
 * rows, at least 128) whose non-empty workgroups fit one per compute unit of
 * the current device.  Pass *rows_per_split as split_rows to mla_decode_attn
 * or mla_attn_tokens (and to mla_workspace_bytes).  A ragged batch then runs
 * as one wave of workgroups of nearly equal size (the automatic plan of a
 * bf16 cache does the same on the device; the f32 kernel's sizes every split
 * for the longest sequence).  Falls back to the automatic plan of the longest
 * length when no split fits.  The flash-decoding split itself is
 * the long-context step of the pages' MLA decode (turbospark deepseek2
 * attn.rs; moeflux mla_attn_forward.rs, SDPA over the latent cache).
 * Errors: NULL, DIMS (a negative length), UNSUPPORTED. */
int mla_attn_plan_lens(const mla_dims* dims, int32_t batch, const int32_t* host_lens,
                       int32_t* rows_per_split, int32_t* num_splits);

/* Human-readable text for a status code (static storage). */
const char* mla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
