"""Seeded synthetic inputs for MLA latent-KV decode.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds no arithmetic of the method: it only draws seeded random
numbers, rounds them to their storage type (fp32, bf16 bit patterns, packed
4-bit nibbles with bf16 scale/bias) and lays them out in the shapes the C ABI
takes. Everything derived from these inputs (YaRN tables, norms, projections,
attention) is computed elsewhere: by the oracle on the CPU, or by the library.

Shapes follow DeepSeek-V3-style MLA as described by the pages
(moeflux ``mla_attn_forward.rs`` -- ``MlaForwardBuffers``; turbospark-runtime
``deepseek2/attn.rs`` -- the fused cache row ``[latent ; k_pe]``).

Storage conventions (these are layouts, not arithmetic):
  * bf16 tensors are ``numpy.uint16`` bit patterns.
  * 4-bit affine weights (``Q4G64``): ``packed`` uint32 [rows, cols/8], element
    k of a row lives in word k//8 at bits 4*(k%8)..4*(k%8)+3 (low nibble first);
    ``scales`` and ``biases`` are bf16 bits [rows, cols/64].
  * the paged cache pool is [num_blocks, block, C+R] in the cache dtype; the
    block table is int32 [B, max_blocks] padded with -1.

Random draws use ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order
per configuration; the order is listed in each ``make_*`` function.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32, BF16, Q4G64 = 0, 1, 2
BLOCK = 64
BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# storage rounding (input preparation only)
# ----------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even from float32) and return the bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    # finite values cannot overflow 32 bits here; NaNs are patched below
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Q4Weight:
    packed: np.ndarray   # uint32 [rows, cols // 8]
    scales: np.ndarray   # uint16 (bf16) [rows, cols // 64]
    biases: np.ndarray   # uint16 (bf16) [rows, cols // 64]
    rows: int
    cols: int


def draw_q4(rng: np.random.Generator, rows: int, cols: int, std: float = 0.02) -> Q4Weight:
    """Draw a 4-bit affine weight whose dequantised values spread like N(0, std^2).

    Draw order: nibbles (rows*cols standard normals, float32), then per-group
    scale jitter (uniform), then per-group bias jitter (normal).
    Nibbles are clip(round(7.5 + 3 z), 0, 15); scale ~ (std/3)*U(0.9, 1.1);
    bias ~ -7.5*scale*(1 + 0.05 z'). These only shape the synthetic
    distribution; the dequantisation itself is the method's and lives elsewhere.
    """
    assert cols % 64 == 0
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    q = np.clip(np.rint(7.5 + 3.0 * z), 0, 15).astype(np.uint32)
    del z
    q = q.reshape(rows, cols // 8, 8)
    packed = np.zeros((rows, cols // 8), dtype=np.uint32)
    for j in range(8):
        packed |= q[:, :, j] << np.uint32(4 * j)
    del q
    g = cols // 64
    s = (std / 3.0) * rng.uniform(0.9, 1.1, size=(rows, g))
    b = -7.5 * s * (1.0 + 0.05 * rng.standard_normal((rows, g)))
    return Q4Weight(packed, to_bf16_bits(s), to_bf16_bits(b), rows, cols)


@dataclasses.dataclass
class Dims:
    num_heads: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora: int
    hidden: int = 0
    q_lora: int = 0
    block_size: int = BLOCK
    cache_dtype: int = BF16
    rms_eps: float = 1e-6

    @property
    def width(self) -> int:
        return self.kv_lora + self.qk_rope


@dataclasses.dataclass
class Yarn:
    theta: float = 10000.0
    factor: float = 40.0
    original_max_pos: float = 4096.0
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 1.0


DEEPSEEK_V3 = dict(num_heads=128, qk_nope=128, qk_rope=64, v_head=128, kv_lora=512)


@dataclasses.dataclass
class Case:
    """One synthetic decode step.  ``None`` fields are absent for this case."""
    name: str
    dims: Dims
    yarn: Yarn
    batch: int
    lens: np.ndarray                 # int32 [B], sequence lengths AFTER the append
    pool: np.ndarray                 # [num_blocks, block, W] float32 or uint16 (bf16)
    table: np.ndarray                # int32 [B, max_blocks], -1 padded
    # softmax scale: a fixed number, or None = the YaRN rule (computed by the consumer)
    softmax_scale: Optional[float]
    x: Optional[np.ndarray] = None   # fp32 [B, hidden] (or [B, W] when hidden == 0)
    kv_a: object = None              # fp32 [W, hidden] | Q4Weight | None (hidden == 0)
    kv_a_norm: Optional[np.ndarray] = None   # [C] fp32 or bf16 bits
    q: Optional[np.ndarray] = None   # fp32 [B, H, N+R] (q given directly)
    q_a: object = None               # Q4Weight [q_lora, hidden] (q chain)
    q_a_norm: Optional[np.ndarray] = None    # bf16 bits [q_lora]
    q_b: object = None               # Q4Weight [H*(N+R), q_lora]
    kv_b: object = None              # [H*(N+V), C] fp32 | bf16 bits | Q4Weight
    o_proj: object = None            # [hidden, H*V] fp32 | Q4Weight | None
    q_abs: Optional[np.ndarray] = None       # [B, H, W] in cache dtype (attention-only cases)
    appended: bool = True            # row at position lens-1 is written by the append step
    # several tokens per sequence: token t belongs to table row token_seq[t] and
    # sees its first lens[t] rows (batch, lens, x, q, q_abs are per token)
    token_seq: Optional[np.ndarray] = None

    @property
    def positions(self) -> np.ndarray:
        return (self.lens - 1).astype(np.int32)


def _cache_values(rng, shape, std, dtype):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v if dtype == F32 else to_bf16_bits(v)


def _store(v, dtype):
    return np.asarray(v, dtype=np.float32) if dtype == F32 else to_bf16_bits(v)


def build_pool(rng, dims: Dims, lens, *, std=1.0, paged=False, appended=True, fresh=None):
    """Allocate the paged pool, the block table and fill the prior rows per sequence.

    Draw order: (if paged) one permutation of all blocks; then per sequence, in
    order, the values of its allocated blocks (block-major, standard normals
    scaled by ``std``).  Rows past the last valid row inside allocated blocks
    are set to NaN so that any read of them shows up in the output.  With
    ``appended`` the row at ``len - 1`` is NaN too: it is the append target;
    ``fresh`` (per sequence) sets how many trailing rows are append targets.
    """
    W, blk = dims.width, dims.block_size
    lens = np.asarray(lens, dtype=np.int64)
    nblk = (lens + blk - 1) // blk
    total = int(nblk.sum())
    maxb = int(nblk.max())
    order = rng.permutation(total).astype(np.int32) if paged else np.arange(total, dtype=np.int32)
    table = np.full((len(lens), maxb), -1, dtype=np.int32)
    dt = np.float32 if dims.cache_dtype == F32 else np.uint16
    pool = np.empty((total, blk, W), dtype=dt)
    k = 0
    for b, nb in enumerate(nblk):
        ids = order[k:k + nb]
        k += nb
        table[b, :nb] = ids
        vals = _cache_values(rng, (int(nb), blk, W), std, dims.cache_dtype)
        pool[ids] = vals
        nf = (1 if appended else 0) if fresh is None else int(np.broadcast_to(fresh, lens.shape)[b])
        first_unset = int(lens[b]) - nf
        if first_unset < nb * blk:
            flat = pool[ids].reshape(-1, W)
            flat[first_unset:] = np.nan if dims.cache_dtype == F32 else BF16_NAN
            pool[ids] = flat.reshape(int(nb), blk, W)
    return pool, table


def to_q8_0(w) -> np.ndarray:
    """float [rows, cols] -> Q8_0 bytes, rows x cols/32 blocks of 34 (input generation).

    Per block of 32: scale d = max|w| / 127 stored as binary16 (little
    endian), then q = round(w / d) clipped to [-127, 127] as signed bytes.
    """
    w = np.asarray(w, dtype=np.float64)
    rows, cols = w.shape
    blk = w.reshape(rows, cols // 32, 32)
    d16 = (np.abs(blk).max(axis=2) / 127.0).astype("<f2")
    d = d16.astype(np.float64)
    safe = np.where(d > 0, d, 1.0)
    q = np.clip(np.rint(blk / safe[..., None]), -127, 127)
    q = np.where(d[..., None] > 0, q, 0).astype(np.int8)
    out = np.empty((rows, cols // 32, 34), dtype=np.uint8)
    out[:, :, :2] = d16.view(np.uint8).reshape(rows, cols // 32, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(-1)


def with_q8_0_kv_b(case: "Case", seed: int = 808) -> "Case":
    """The same case with kv_b stored as Q8_0: quantised from its current values
    (fp32 or bf16), or, for a 4-bit kv_b, from a fresh draw of N(0, 0.02^2)."""
    import copy
    d = case.dims
    rows, cols = d.num_heads * (d.qk_nope + d.v_head), d.kv_lora
    if isinstance(case.kv_b, Q4Weight):
        vals = np.random.default_rng(seed).normal(0.0, 0.02, size=(rows, cols))
    else:
        kv = np.asarray(case.kv_b)
        vals = bf16_bits_to_f32(kv) if kv.dtype == np.uint16 else kv.astype(np.float32)
    out = copy.copy(case)
    out.kv_b = to_q8_0(vals.reshape(rows, cols))
    out.name = case.name + "_q8_0kvb"
    return out


def _pool_for(rng, d: Dims, L, token_seq, *, std, paged, appended=True):
    """Pool and table for per-sequence ``L`` or, with ``token_seq``, for the
    sequences the tokens belong to: a sequence's length is the largest
    ``L[t]`` of its tokens, and each of its tokens leaves one row to append."""
    if token_seq is None:
        return build_pool(rng, d, L, std=std, paged=paged, appended=appended)
    ns = int(np.max(token_seq)) + 1
    final = np.zeros(ns, dtype=np.int64)
    fresh = np.zeros(ns, dtype=np.int64)
    for t, sq in enumerate(token_seq):
        final[sq] = max(final[sq], int(L[t]))
        fresh[sq] += 1
    return build_pool(rng, d, final, std=std, paged=paged, fresh=fresh if appended else 0)


def make_chunk_case(cfg: int, prior, chunk, *, seed: Optional[int] = None,
                    paged: Optional[bool] = None) -> Case:
    """Several new tokens per sequence in one step (chunked prefill, multi-token decode).

    Sequence s holds ``prior[s]`` rows and gains ``chunk[s]`` tokens at positions
    prior[s] .. prior[s] + chunk[s] - 1, stacked sequence by sequence; token t
    sees ``lens[t]`` = its position + 1 rows.  The draws are those of
    ``make_case(cfg)`` with one x / q (or q_abs) per token; the pool holds every
    sequence's prior rows and NaN in the rows its tokens append.
    """
    prior = np.asarray(prior, dtype=np.int64)
    chunk = np.broadcast_to(np.asarray(chunk, dtype=np.int64), prior.shape)
    token_seq = np.repeat(np.arange(len(prior)), chunk).astype(np.int32)
    lens = np.concatenate([p + 1 + np.arange(c) for p, c in zip(prior, chunk)]).astype(np.int32)
    case = make_case(cfg, lens=lens, seed=seed, paged=paged, token_seq=token_seq)
    case.name += "_chunk"
    return case


def make_case(cfg: int, *, batch: Optional[int] = None, lens=None, seed: Optional[int] = None,
              paged: Optional[bool] = None, sharp: bool = False, token_seq=None) -> Case:
    """Build configuration ``cfg`` (1..5) with optional size overrides.

    The five configurations, in the storage forms the library takes:
      1  tiny fp32 decode, 1 sequence: H16/N32/R16/V32/C64, hidden 256, L 128,
         append at 127 through kv_a; two blocks mapped by table [1, 0];
         q, c_kv, k_pe, W_UK, W_UV, W_kva, W_o ~ N(0, 0.02^2); x ~ N(0, 1);
         gamma = 1 + 0.1 N(0, 1); softmax scale by the YaRN rule.
         ``sharp=True`` draws the cache rows and q with std 1.
      2  DeepSeek-V3 shapes, batch 1, L 4096, bf16 cache and bf16 kv_b;
         append at 4095 with the pre-norm row given directly (hidden 0);
         q ~ N(0, 1), rows ~ N(0, 1), kv_b ~ N(0, 0.02^2), scale 1/sqrt(192).
      3  as 2 with 64 sequences, lengths uniform in [1024, 8192], paged pool
         with a random block permutation.
      4  batch 4, L 131072, attention only: q_abs ~ N(0, 1) (bf16) given in
         latent form, rows ~ N(0, 1), scale 1/sqrt(192).
      5  full layer, batch 32, L 16384: hidden 7168, q_lora 1536, all five
         projections 4-bit affine group 64, bf16 norms; YaRN softmax scale.
    With ``token_seq`` the batch is of tokens (see ``make_chunk_case``).
    """
    seed = 1000 + cfg if seed is None else seed
    if lens is not None and batch is None:
        batch = len(lens)
    rng = np.random.default_rng(seed)
    yarn = Yarn()
    if cfg == 1:
        d = Dims(num_heads=16, qk_nope=32, qk_rope=16, v_head=32, kv_lora=64, hidden=256,
                 q_lora=0, cache_dtype=F32)
        B = 1 if batch is None else batch
        L = np.full(B, 128, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
        std = 1.0 if sharp else 0.02
        if paged is None and B == 1 and lens is None and token_seq is None:
            # the fixed two-block layout: logical block 0 -> physical 1, 1 -> 0
            pool, table = build_pool(rng, d, L, std=std, paged=False)
            pool = pool[::-1].copy()
            table = np.array([[1, 0]], dtype=np.int32)
        else:
            pool, table = _pool_for(rng, d, L, token_seq, std=std, paged=bool(paged))
        H, N, R, V, C, W = 16, 32, 16, 32, 64, 80
        x = rng.standard_normal((B, d.hidden))
        kv_a = rng.standard_normal((W, d.hidden)) * 0.02
        gamma = 1.0 + 0.1 * rng.standard_normal(C)
        q = rng.standard_normal((B, H, N + R)) * std
        kv_b = rng.standard_normal((H * (N + V), C)) * 0.02
        o_proj = rng.standard_normal((d.hidden, H * V)) * 0.02
        return Case("cfg1" + ("_sharp" if sharp else ""), d, yarn, B, L, pool, table, None,
                    x=_store(x, F32), kv_a=_store(kv_a, F32), kv_a_norm=_store(gamma, F32),
                    q=_store(q, F32), kv_b=_store(kv_b, F32), o_proj=_store(o_proj, F32),
                    token_seq=token_seq)
    if cfg in (2, 3):
        d = Dims(**DEEPSEEK_V3, hidden=0, q_lora=0, cache_dtype=BF16)
        if cfg == 2:
            B = 1 if batch is None else batch
            L = np.full(B, 4096, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
            pg = False if paged is None else paged
        else:
            B = 64 if batch is None else batch
            L = (rng.integers(1024, 8192, size=B, endpoint=True).astype(np.int32)
                 if lens is None else np.asarray(lens, dtype=np.int32))
            pg = True if paged is None else paged
        pool, table = _pool_for(rng, d, L, token_seq, std=1.0, paged=pg)
        H, N, R, V, C, W = 128, 128, 64, 128, 512, 576
        x = rng.standard_normal((B, W))
        gamma = 1.0 + 0.1 * rng.standard_normal(C)
        q = rng.standard_normal((B, H, N + R))
        kv_b = rng.standard_normal((H * (N + V), C)) * 0.02
        return Case(f"cfg{cfg}", d, yarn, B, L, pool, table, 1.0 / np.sqrt(192.0),
                    x=_store(x, F32), kv_a=None, kv_a_norm=to_bf16_bits(gamma),
                    q=_store(q, F32), kv_b=to_bf16_bits(kv_b), token_seq=token_seq)
    if cfg == 4:
        d = Dims(**DEEPSEEK_V3, hidden=0, q_lora=0, cache_dtype=BF16)
        B = 4 if batch is None else batch
        L = np.full(B, 131072, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
        pool, table = _pool_for(rng, d, L, token_seq, std=1.0, paged=bool(paged), appended=False)
        q_abs = to_bf16_bits(rng.standard_normal((B, 128, 576), dtype=np.float32))
        return Case("cfg4", d, yarn, B, L, pool, table, 1.0 / np.sqrt(192.0),
                    q_abs=q_abs, appended=False, token_seq=token_seq)
    if cfg == 5:
        d = Dims(**DEEPSEEK_V3, hidden=7168, q_lora=1536, cache_dtype=BF16)
        B = 32 if batch is None else batch
        L = np.full(B, 16384, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
        pool, table = _pool_for(rng, d, L, token_seq, std=1.0, paged=bool(paged))
        H, N, R, V, C, W = 128, 128, 64, 128, 512, 576
        x = rng.standard_normal((B, d.hidden), dtype=np.float32)
        q_a = draw_q4(rng, d.q_lora, d.hidden)
        q_a_norm = to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d.q_lora))
        q_b = draw_q4(rng, H * (N + R), d.q_lora)
        kv_a = draw_q4(rng, W, d.hidden)
        kv_a_norm = to_bf16_bits(1.0 + 0.1 * rng.standard_normal(C))
        kv_b = draw_q4(rng, H * (N + V), C)
        o_proj = draw_q4(rng, d.hidden, H * V)
        return Case("cfg5", d, yarn, B, L, pool, table, None,
                    x=x, kv_a=kv_a, kv_a_norm=kv_a_norm, q_a=q_a, q_a_norm=q_a_norm, q_b=q_b,
                    kv_b=kv_b, o_proj=o_proj, token_seq=token_seq)
    raise ValueError(f"unknown configuration {cfg}")
