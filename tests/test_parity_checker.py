"""CPU test of the attention parity checker itself (tests/parity.py).

At the long-context size (one sequence of 131072 rows, DeepSeek-V3 shapes, the
inputs of the long-context workload) the checker must
  * reject the oracle's own result with rows missing: one 32-row tile (first,
    middle) or one 2048-row split (first, middle);
  * accept a model of the kernel's rounding: per 2048-row split, numerators
    rounded to bf16 against the split's own maximum, the denominator summed
    from the unrounded values, the normalised partial stored as fp16, then
    merged by weights exp(lse_s - lse).
Everything here runs on the oracle (fp64) and numpy; no GPU.
"""
import numpy as np
import pytest

import mla_synth as S
from oracle import mla_oracle as O

from parity import attn_check

L = 131072
SPLIT = 2048


@pytest.fixture(scope="module")
def long_case():
    case = S.make_case(4, batch=1, lens=[L])
    q64 = O.widen(case.q_abs, case.dims.cache_dtype)
    scale = float(np.float32(case.softmax_scale))
    rvc, rlse, _ = O.attention_latent(case.dims, q64, case.pool, case.table, case.lens, scale)
    return case, q64, scale, rvc, rlse


def without_rows(case, start, count):
    """The sequence with logical rows [start, start + count) removed, as a
    contiguous pool (NaN padding after the last row)."""
    d = case.dims
    rows = O.gather_rows(case.pool, case.table, 0, L, d.block_size)
    keep = np.concatenate([rows[:start], rows[start + count:]])
    n = len(keep)
    nb = (n + d.block_size - 1) // d.block_size
    flat = np.full((nb * d.block_size, d.width), S.BF16_NAN, dtype=np.uint16)
    flat[:n] = keep
    table = np.arange(nb, dtype=np.int32)[None, :]
    return flat.reshape(nb, d.block_size, d.width), table, np.array([n], dtype=np.int32)


@pytest.mark.parametrize("start,count", [(0, 32), (L // 2, 32), (0, SPLIT), (L // 2 - SPLIT, SPLIT)],
                         ids=["first-tile", "middle-tile", "first-split", "middle-split"])
def test_checker_rejects_missing_rows(long_case, start, count):
    case, q64, scale, rvc, rlse = long_case
    pool, table, lens = without_rows(case, start, count)
    vc, lse, _ = O.attention_latent(case.dims, q64, pool, table, lens, scale)
    with pytest.raises(AssertionError):
        attn_check(vc, lse, rvc, rlse, f"{count} rows from {start} removed")


def bf16_round(x):
    return O.widen(O.round_bf16(x), O.BF16)


def test_checker_accepts_kernel_rounding_model(long_case):
    case, q64, scale, rvc, rlse = long_case
    d = case.dims
    C = d.kv_lora
    rows = O.widen(O.gather_rows(case.pool, case.table, 0, L, d.block_size), d.cache_dtype)
    s = scale * (q64[0] @ rows.T)                                   # [H, L]
    parts, lses = [], []
    for r0 in range(0, L, SPLIT):
        ss = s[:, r0:r0 + SPLIT]
        m = ss.max(axis=1, keepdims=True)
        e = np.exp(ss - m)
        l_s = e.sum(axis=1, keepdims=True)
        o = (bf16_round(e) @ rows[r0:r0 + SPLIT, :C]) / l_s
        parts.append(o.astype(np.float16).astype(np.float64))
        lses.append((m + np.log(l_s))[:, 0])
    lses = np.stack(lses)                                            # [S, H]
    top = lses.max(axis=0)
    w = np.exp(lses - top)
    vc = np.einsum("sh,shc->hc", w, np.stack(parts)) / w.sum(axis=0)[:, None]
    lse = top + np.log(w.sum(axis=0))
    attn_check(vc[None], lse[None], rvc, rlse, "kernel rounding model")
