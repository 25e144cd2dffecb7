"""CPU oracle for single-token MLA decode with weight absorption -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and must never sit on the product path.

It is a plain, slow, obviously correct float64 implementation written from the
source pages, which are host-side Rust that drives GPU kernels whose bodies are
not shown:

  [moeflux/forward]  moeflux 0.1.0-pre.3, ``src/riir/attn/mla_attn_forward.rs``
  [ts/deepseek2]     turbospark-runtime 0.3.0, ``src/families/deepseek2/attn.rs``
  [moeflux/matvec]   moeflux 0.1.0-pre.3, ``src/riir/backend/gpu/gpu_matvec.rs``
  [ts/gptoss]        turbospark-runtime 0.3.0, ``src/families/gptoss/attn.rs``

Every input is widened exactly to float64 from its stored bits (fp32, bf16, or
4-bit nibbles with bf16 scale/bias); all arithmetic is float64; values are
rounded only where the method stores them (the cache row, and ``q_abs`` when
the chain is modelled), with round-to-nearest-even.

Readings of points the pages leave open:
  * YaRN inverse frequencies: the ramp between two correction dimensions
    ([ts/gptoss] module doc, item 2; parameter list of ``MlaYarnTables::new``
    in [moeflux/forward]) is taken from the YaRN paper (Peng et al., 2023):
    correction dim d(r) = R ln(L_orig / (2 pi r)) / (2 ln theta); low =
    floor(d(beta_fast)) >= 0, high = ceil(d(beta_slow)) <= R-1; a linear ramp
    over the pair index between them blends theta^(-2i/R) (kept) with
    theta^(-2i/R)/factor (interpolated).
  * Two YaRN scalars, get(s, m) = 1 + 0.1 m ln s (1 for s <= 1): the rotation
    is multiplied by get(s, mscale)/get(s, mscale_all_dim) and the softmax
    scale is get(s, mscale_all_dim)^2 / sqrt(N+R)  ([ts/deepseek2]
    ``encode_mla_attention_block`` keeps ``rope_mscale`` apart from the scale
    folded at repack; [moeflux/forward] multiplies the scale by mscale^2).
  * RoPE rotates consecutive pairs (2i, 2i+1) ([ts/deepseek2], the comment on
    the k_pe rope) as (x, y) -> (x cos a - y sin a, x sin a + y cos a) with
    a = pos * inv_freq[i].
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma over the latent half only
    ([moeflux/forward] module doc item 2; [ts/deepseek2] ``encode_mla_kv_norm``).
  * The finished cache row [norm(c) ; rope(k_pe)] is rounded once to the cache
    dtype; q_abs is stored in the cache dtype; the softmax scale multiplies the
    scores (it is not folded into q).
  * kv_b rows: head h owns rows h*(N+V) .. h*(N+V)+N-1 (W_UK) then the next V
    rows (W_UV) ([moeflux/forward] ``kv_b_per_head``).
  * 4-bit affine weights: w = scale * q + bias per 64-wide input group
    ([moeflux/matvec] ``MatvecSpec``, ``encode_matvec``); nibble k of a row sits
    in word k//8 at bits 4*(k%8) (low nibble first) -- parity unpinned by the
    pages, a storage convention.
  * Paging: logical row t of sequence b lives at pool[table[b][t // block],
    t % block].
  * Q8_0 kv_b ([ts/deepseek2] ``validate_q8_0_matrix`` and its unit test: the
    row width must tile whole blocks, and a 64-wide row holds two, so a block
    is 32 values): the pages name the format without its byte layout; it is
    read as GGUF's Q8_0, each block a little-endian binary16 scale d followed
    by 32 signed 8-bit q, element = d * q (34 bytes per block).
  * Several tokens per sequence in one step (chunked prefill, multi-token
    decode): [moeflux/matvec] ``encode_matvec_n_tokens`` applies each
    projection to stacked tokens with per-token arithmetic unchanged; the
    pages say nothing about attention over several new tokens.  Read plainly:
    every new row is appended first, and the token at position p attends rows
    0..p of its own sequence, so a chunk gives what the same tokens give one
    decode step at a time.  ``token_seq[t]`` names the block-table row of
    token t; without it token t owns row t.
"""
from __future__ import annotations

import math

import numpy as np

F32, BF16, Q4G64, Q8_0 = 0, 1, 2, 3
Q8_0_BLOCK, Q8_0_BLOCK_BYTES = 32, 34


# ----------------------------------------------------------------------------
# storage types
# ----------------------------------------------------------------------------
def widen(arr, dtype: int) -> np.ndarray:
    """Stored bits -> float64, exactly.  bf16 is a uint16 bit pattern."""
    if dtype == F32:
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        b = np.ascontiguousarray(np.asarray(arr, dtype=np.uint16))
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), returned as uint16 bits.

    Written directly on the float64 value (no detour through float32, so there
    is no double rounding): bf16 keeps 8 significant bits for normals and a
    fixed quantum of 2^-133 below 2^-126.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    a = np.abs(x)
    small = a < 2.0 ** -126
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    out[~small] = np.ldexp(np.rint(np.ldexp(m[~small], 8)), e[~small] - 8)
    out[small] = np.rint(x[small] * 2.0 ** 133) * 2.0 ** -133
    big = np.abs(out) > 3.3895313892515355e38   # largest finite bf16
    out[big] = np.copysign(np.inf, x[big])
    out[np.isnan(x)] = np.nan
    bits = (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(x)] = 0x7FC0
    return bits


def round_to(x, dtype: int):
    """Round float64 values to a storage dtype; returns the stored form."""
    if dtype == F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == BF16:
        return round_bf16(x)
    raise ValueError(dtype)


def dequant_q4(packed, scales, biases, rows: int, cols: int, group: int = 64) -> np.ndarray:
    """4-bit affine weight -> float64 [rows, cols]: w = scale * q + bias.

    [moeflux/matvec] ``MatvecSpec`` (packed weight, bf16 scales, bf16 biases),
    ``encode_matvec`` (group size); [moeflux/forward] ``resolve_proj``.
    """
    packed = np.asarray(packed, dtype=np.uint32).reshape(rows, cols // 8)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    q = ((packed[:, :, None] >> shifts[None, None, :]) & np.uint32(15)).reshape(rows, cols)
    s = widen(scales, BF16).reshape(rows, cols // group)
    b = widen(biases, BF16).reshape(rows, cols // group)
    return q.astype(np.float64) * np.repeat(s, group, axis=1) + np.repeat(b, group, axis=1)


def dequant_q8_0(blocks, rows: int, cols: int) -> np.ndarray:
    """Q8_0 weight (uint8 bytes, [rows][cols/32] blocks of 34) -> float64 [rows, cols].

    Element k of a row is d * q[k % 32] of block k // 32, with d the block's
    little-endian binary16 scale and q its signed bytes ([ts/deepseek2]
    ``validate_q8_0_matrix``; the byte layout is GGUF's Q8_0).
    """
    raw = np.asarray(blocks, dtype=np.uint8).reshape(rows, cols // Q8_0_BLOCK, Q8_0_BLOCK_BYTES)
    d = raw[:, :, :2].copy().view("<f2")[..., 0].astype(np.float64)
    q = raw[:, :, 2:].view(np.int8).astype(np.float64)
    return (d[:, :, None] * q).reshape(rows, cols)


def weight_f64(w, dtype: int, rows: int, cols: int) -> np.ndarray:
    """Any stored weight (fp32, bf16 bits, Q8_0 bytes, or an object with
    packed/scales/biases) -> float64."""
    if dtype == Q4G64:
        return dequant_q4(w.packed, w.scales, w.biases, rows, cols)
    if dtype == Q8_0:
        return dequant_q8_0(w, rows, cols)
    return widen(w, dtype).reshape(rows, cols)


# ----------------------------------------------------------------------------
# YaRN tables  ([moeflux/forward] ``MlaYarnTables::new``)
# ----------------------------------------------------------------------------
def yarn_get_mscale(scale: float, mscale: float = 1.0) -> float:
    """Attention-temperature factor 1 + 0.1 m ln s of YaRN (1 when s <= 1)."""
    if scale <= 1.0:
        return 1.0
    return 0.1 * mscale * math.log(scale) + 1.0


def yarn_correction_range(R: int, theta: float, orig_max_pos: float,
                          beta_fast: float, beta_slow: float):
    """The two correction dimensions (low, high) bounding the YaRN ramp.

    A pair i turns orig_max_pos * theta^(-2i/R) / (2 pi) times over the original
    context; d(r) solves that count = r for i.  low = floor(d(beta_fast)),
    high = ceil(d(beta_slow)), clamped to [0, R-1].
    """
    def d(r):
        return R * math.log(orig_max_pos / (r * 2.0 * math.pi)) / (2.0 * math.log(theta))
    low = max(math.floor(d(beta_fast)), 0)
    high = min(math.ceil(d(beta_slow)), R - 1)
    return low, high


def yarn_inv_freq(R: int, theta: float, factor: float, orig_max_pos: float,
                  beta_fast: float, beta_slow: float) -> np.ndarray:
    """YaRN inverse frequencies for the R/2 rotated pairs, float64.

    Pairs below ``low`` keep theta^(-2i/R); pairs above ``high`` are divided by
    ``factor``; in between a linear ramp in the pair index blends the two.
    """
    i = np.arange(R // 2, dtype=np.float64)
    extra = theta ** (-2.0 * i / R)
    inter = extra / factor
    low, high = yarn_correction_range(R, theta, orig_max_pos, beta_fast, beta_slow)
    if low == high:
        high = high + 0.001
    ramp = np.clip((i - low) / (high - low), 0.0, 1.0)
    return extra * (1.0 - ramp) + inter * ramp


def yarn_scalars(factor: float, mscale: float, mscale_all_dim: float, qk_head_dim: int):
    """(rope_mscale, softmax_scale) under the two-scalar reading."""
    m = yarn_get_mscale(factor, mscale)
    m_all = yarn_get_mscale(factor, mscale_all_dim)
    return m / m_all, m_all * m_all / math.sqrt(qk_head_dim)


# ----------------------------------------------------------------------------
# the elementwise steps
# ----------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma over the last axis.

    [moeflux/forward] ``encode_rms_norm_bf16_into`` on q_lat and kv_lat;
    [ts/deepseek2] ``encode_mla_kv_norm`` (latent half of the row only).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_consecutive(x, pos, inv_freq, mscale: float = 1.0) -> np.ndarray:
    """Rotate consecutive pairs (2i, 2i+1) of the last axis by pos * inv_freq[i].

    ``pos`` broadcasts against the leading axes of ``x``.
    [ts/deepseek2] ``encode_mla_attention_block``: q_pe and the k_pe tail of the
    cache row go through the same windowed rope with consecutive pairing;
    [moeflux/forward] ``encode_yarn_rope_apply`` scales by the YaRN mscale.
    """
    x = np.asarray(x, dtype=np.float64)
    inv_freq = np.asarray(inv_freq, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq      # [..., R/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = mscale * (a * c - b * s)
    out[..., 1::2] = mscale * (a * s + b * c)
    return out


def matvec(W, x) -> np.ndarray:
    """y[..., o] = sum_k W[o, k] x[..., k]  ([moeflux/matvec] ``encode_matvec``)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def kv_b_split(kv_b64: np.ndarray, H: int, N: int, V: int):
    """kv_b [H*(N+V), C] -> (W_UK [H, N, C], W_UV [H, V, C])."""
    w = kv_b64.reshape(H, N + V, -1)
    return w[:, :N, :], w[:, N:, :]


# ----------------------------------------------------------------------------
# paged cache addressing  (integer work; reproduced exactly)
# ----------------------------------------------------------------------------
def slot(table, b: int, pos: int, block: int) -> tuple:
    """(physical block, row in block) of logical row ``pos`` of sequence ``b``."""
    return int(table[b][pos // block]), pos % block


def gather_rows(pool, table, b: int, length: int, block: int) -> np.ndarray:
    """Logical rows 0..length-1 of sequence b, in the pool's stored form."""
    nb = (length + block - 1) // block
    blocks = np.asarray(table[b][:nb], dtype=np.int64)
    return np.asarray(pool)[blocks].reshape(nb * block, -1)[:length]


# ----------------------------------------------------------------------------
# the four calls
# ----------------------------------------------------------------------------
def cache_append(dims, x, kv_a, kv_a_dtype, kv_a_norm, norm_dtype, inv_freq, rope_mscale,
                 positions, pool, table, token_seq=None):
    """kv_a projection -> RMSNorm of the latent half -> RoPE of k_pe -> one rounded row.

    [moeflux/forward] ``mla_attn_layer_forward_gpu``: KV-A chain, split,
    ``kv_a_layernorm``, YaRN rope on k_pe, ``mla_kv_cache_append`` into row[pos];
    [ts/deepseek2]: kv_a writes the fused row ``[latent ; k_pe]``, then norm and
    rope run on it.  With ``dims.hidden == 0`` the row before the norm is ``x``.
    Token b writes into sequence ``token_seq[b]`` (``b`` when it is None).
    Returns (new pool, the appended rows as float64 before rounding).
    """
    C, R, W, blk = dims.kv_lora, dims.qk_rope, dims.width, dims.block_size
    x64 = np.asarray(x, dtype=np.float64).reshape(len(positions), -1)
    if dims.hidden:
        Wk = weight_f64(kv_a, kv_a_dtype, W, dims.hidden)
        kv_pre = matvec(Wk, x64)
    else:
        kv_pre = x64
    gamma = widen(kv_a_norm, norm_dtype)
    c = rmsnorm(kv_pre[:, :C], gamma, dims.rms_eps)
    k_pe = rope_consecutive(kv_pre[:, C:], np.asarray(positions), inv_freq, rope_mscale)
    rows = np.concatenate([c, k_pe], axis=1)
    out = np.array(pool, copy=True)
    stored = round_to(rows, dims.cache_dtype)
    for b, pos in enumerate(positions):
        seq = b if token_seq is None else int(token_seq[b])
        pb, r = slot(table, seq, int(pos), blk)
        out[pb, r] = stored[b]
    return out, rows


def q_chain(dims, x, q_a, q_a_norm, q_b):
    """q = W_qb RMSNorm_qa(W_qa x), split per head into [nope ; rope].

    [moeflux/forward]: ``q_a_proj`` -> ``q_a_layernorm`` (one norm over q_lora,
    as the code does; the module doc's "per-head" wording is not followed) ->
    ``q_b_proj``.
    """
    H, N, R = dims.num_heads, dims.qk_nope, dims.qk_rope
    Wa = weight_f64(q_a, Q4G64, dims.q_lora, dims.hidden)
    Wb = weight_f64(q_b, Q4G64, H * (N + R), dims.q_lora)
    q_lat = rmsnorm(matvec(Wa, x), widen(q_a_norm, BF16), dims.rms_eps)
    return matvec(Wb, q_lat).reshape(-1, H, N + R)


def absorb_q(dims, q, kv_b64, inv_freq, rope_mscale, positions) -> np.ndarray:
    """q_abs[b, h] = [W_UK_h^T q_nope[b, h] ; RoPE(q_pe[b, h])]  (float64, unrounded).

    [moeflux/forward] ``mla_q_prime_4bit`` (q' = W_UK^T q_nope per head);
    [ts/deepseek2] ``encode_mla_absorb_q`` (fused ``[q' ; q_pe]`` rows, q_pe
    roped before the absorb gathers it).
    """
    H, N, V = dims.num_heads, dims.qk_nope, dims.v_head
    q = np.asarray(q, dtype=np.float64)
    W_UK, _ = kv_b_split(kv_b64, H, N, V)
    qp = np.einsum("bhn,hnc->bhc", q[:, :, :N], W_UK)
    pos = np.asarray(positions, dtype=np.float64)[:, None]           # [B, 1] -> heads
    qpe = rope_consecutive(q[:, :, N:], pos, inv_freq, rope_mscale)
    return np.concatenate([qp, qpe], axis=2)


def attention_latent(dims, q_abs64, pool, table, lens, scale: float, token_seq=None):
    """Latent-form decode attention: the absorbed path.

    s[t] = scale * q_abs_h . row_t over the full row [c_kv ; k_pe]; p = softmax
    over t < len (max-subtracted); v_combine_h = sum_t p[t] c_kv[t]; lse_h =
    log sum_t exp(s[t]).  [moeflux/forward] ``mla_sdpa_folded``;
    [ts/deepseek2] ``encode_mla_attention_decode`` (V is the row's first C).
    Returns (v_combine [B, H, C], lse [B, H], list of p [H, len] per query).
    A query that sees 0 rows gives v_combine = 0 and lse = -inf.  Query b reads
    the rows of sequence ``token_seq[b]`` (``b`` when it is None).
    """
    C, blk = dims.kv_lora, dims.block_size
    B, H = q_abs64.shape[0], q_abs64.shape[1]
    vc = np.zeros((B, H, C))
    lse = np.full((B, H), -np.inf)
    ps = []
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            ps.append(np.zeros((H, 0)))
            continue
        seq = b if token_seq is None else int(token_seq[b])
        rows = widen(gather_rows(pool, table, seq, L, blk), dims.cache_dtype)  # [L, W]
        s = scale * (q_abs64[b] @ rows.T)                                    # [H, L]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        p = e / z
        vc[b] = p @ rows[:, :C]
        lse[b] = (m + np.log(z))[:, 0]
        ps.append(p)
    return vc, lse, ps


def attention_unabsorbed(dims, q64, kv_b64, pool, table, lens, scale, inv_freq, rope_mscale,
                         positions, heads=None, seqs=None):
    """The unabsorbed definition: decompress per-head K and V, then plain attention.

    For head h and row t: K_h[t] = [W_UK_h c_t ; k_pe_t], V_h[t] = W_UV_h c_t;
    q_h = [q_nope_h ; RoPE(q_pe_h)]; o_h = softmax_t(scale q_h . K_h[t]) V_h.
    This is what weight absorption must reproduce ([moeflux/forward] module doc,
    "folded SDPA"; [ts/deepseek2] module doc).  Rows are the stored cache values.
    Returns o [len(seqs), len(heads), V] and lse.
    """
    H, N, R, V, C, blk = (dims.num_heads, dims.qk_nope, dims.qk_rope, dims.v_head,
                          dims.kv_lora, dims.block_size)
    heads = range(H) if heads is None else heads
    seqs = range(q64.shape[0]) if seqs is None else seqs
    W_UK, W_UV = kv_b_split(kv_b64, H, N, V)
    o = np.zeros((len(seqs), len(heads), V))
    lse = np.zeros((len(seqs), len(heads)))
    for i, b in enumerate(seqs):
        L = int(lens[b])
        rows = widen(gather_rows(pool, table, b, L, blk), dims.cache_dtype)
        c, kpe = rows[:, :C], rows[:, C:]
        qpe = rope_consecutive(q64[b, :, N:], float(positions[b]), inv_freq, rope_mscale)
        for j, h in enumerate(heads):
            K = np.concatenate([c @ W_UK[h].T, kpe], axis=1)        # [L, N+R]
            Vh = c @ W_UV[h].T                                       # [L, V]
            qh = np.concatenate([q64[b, h, :N], qpe[h]])
            s = scale * (K @ qh)
            m = s.max()
            e = np.exp(s - m)
            o[i, j] = (e / e.sum()) @ Vh
            lse[i, j] = m + np.log(e.sum())
    return o, lse


def out_proj(dims, v_combine64, kv_b64, o_proj64=None) -> np.ndarray:
    """out[b, h] = W_UV_h v_combine[b, h]; then y = W_o concat_h(out) if o_proj is given.

    [moeflux/forward] ``mla_out_per_head_4bit`` then the ``o_proj`` matvec;
    [ts/deepseek2] ``encode_mla_v_combine`` then ``O_PROJ``.
    """
    H, N, V = dims.num_heads, dims.qk_nope, dims.v_head
    _, W_UV = kv_b_split(kv_b64, H, N, V)
    out = np.einsum("hvc,bhc->bhv", W_UV, np.asarray(v_combine64, dtype=np.float64))
    if o_proj64 is None:
        return out
    return matvec(o_proj64, out.reshape(out.shape[0], H * V))


# ----------------------------------------------------------------------------
# a whole decode step on one synthetic case
# ----------------------------------------------------------------------------
def weight_dtype(w) -> int:
    if hasattr(w, "packed"):
        return Q4G64
    dt = np.asarray(w).dtype
    if dt == np.uint8:
        return Q8_0
    return BF16 if dt == np.uint16 else F32


def tables_for(case):
    """(inv_freq as stored float32 bits widened, rope_mscale, softmax_scale)."""
    d, y = case.dims, case.yarn
    inv = yarn_inv_freq(d.qk_rope, y.theta, y.factor, y.original_max_pos, y.beta_fast, y.beta_slow)
    inv32 = inv.astype(np.float32).astype(np.float64)     # the table the library is given
    rm, sc = yarn_scalars(y.factor, y.mscale, y.mscale_all_dim, d.qk_nope + d.qk_rope)
    if case.softmax_scale is not None:
        sc = float(case.softmax_scale)
    return inv32, float(np.float32(rm)), float(np.float32(sc))


def attention_query(case, res=None, model_q_abs_storage=True) -> np.ndarray:
    """The absorbed query the latent attention of ``decode_step`` consumes:
    q_abs as given, or q (given, else the q chain) absorbed through W_UK with
    its rope part rotated.  Intermediates go into ``res`` when one is passed."""
    d = case.dims
    res = {} if res is None else res
    if case.q_abs is not None:
        res["q_abs_stored"] = case.q_abs
        return widen(case.q_abs, d.cache_dtype)
    inv, rm, _ = tables_for(case)
    kvb_dt = weight_dtype(case.kv_b)
    kv_b64 = weight_f64(case.kv_b, kvb_dt, d.num_heads * (d.qk_nope + d.v_head), d.kv_lora)
    res["kv_b64"] = kv_b64
    if case.q is not None:
        q = widen(case.q, F32)
    else:
        q = q_chain(d, case.x, case.q_a, case.q_a_norm, case.q_b)
    res["q"] = q
    q_abs64 = absorb_q(d, q, kv_b64, inv, rm, case.positions)
    res["q_abs64"] = q_abs64
    stored = round_to(q_abs64, d.cache_dtype)
    res["q_abs_stored"] = stored
    return widen(stored, d.cache_dtype) if model_q_abs_storage else q_abs64


def decode_step(case, *, model_q_abs_storage=True):
    """Run append -> absorb (q chain) -> latent attention -> out_proj on a case.

    A case with ``token_seq`` holds several tokens per sequence: all their rows
    are appended, then token t attends its sequence's first ``lens[t]`` rows.

    Returns a dict with the new pool, q (float64), q_abs (float64, and its
    stored form), v_combine, lse and out.  With ``model_q_abs_storage`` the
    attention consumes q_abs rounded to the cache dtype, as the library stores it.
    """
    d = case.dims
    inv, rm, sc = tables_for(case)
    res = {"inv_freq": inv, "rope_mscale": rm, "softmax_scale": sc}
    pool = case.pool
    tseq = getattr(case, "token_seq", None)
    if case.appended:
        kdt = weight_dtype(case.kv_a) if case.kv_a is not None else F32
        ndt = weight_dtype(case.kv_a_norm)
        pool, rows = cache_append(d, case.x, case.kv_a, kdt, case.kv_a_norm, ndt, inv, rm,
                                  case.positions, case.pool, case.table, tseq)
        res["appended_rows"] = rows
    res["pool"] = pool
    q_abs64 = attention_query(case, res, model_q_abs_storage)
    vc, lse, ps = attention_latent(d, q_abs64, pool, case.table, case.lens, sc, tseq)
    res.update(v_combine=vc, lse=lse, p=ps)
    if case.kv_b is not None:
        o64 = None
        if case.o_proj is not None:
            o64 = weight_f64(case.o_proj, weight_dtype(case.o_proj), d.hidden,
                             d.num_heads * d.v_head)
        res["out"] = out_proj(d, vc, res["kv_b64"], o64)
    return res
