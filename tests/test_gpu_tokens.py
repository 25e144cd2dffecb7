"""GPU parity of the several-tokens-per-sequence calls (chunked prefill,
multi-token decode): ``mla_cache_append_tokens`` and ``mla_attn_tokens``, with
``mla_absorb_q`` / ``mla_out_proj`` taking the stacked tokens as their batch.

Reading under test (the pages give the batched projections, not the
attention): all new rows are appended first, and the token at position p
attends rows 0..p of its own sequence.  Tolerances as in test_gpu_parity,
with the tight per-query attention checks of ``tests/parity.py``.
"""
import copy

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import attn_check, close_bf16, close_f32
from test_gpu_parity import attn_on_oracle_query, host, sync

pytestmark = pytest.mark.gpu


def _close(dtype, got, ref, what):
    (close_f32 if dtype == O.F32 else close_bf16)(got, ref, what)


CHUNKS = [
    (1, [5, 70], [4, 3], None),             # fp32 cache, VALU attention, fp32 projections
    (2, [1000, 37], [3, 5], None),          # bf16 MFMA attention, tokens crossing a block edge
    (3, [1024, 1500, 2049], 2, True),       # ragged, paged with a random block order
    (5, [300, 1100], [4, 2], None),         # the whole layer with 4-bit projections
]


@pytest.mark.parametrize("cfg,prior,chunk,paged", CHUNKS)
def test_chunk_step(cfg, prior, chunk, paged):
    case = S.make_chunk_case(cfg, prior, chunk, paged=paged)
    print(f"[chunk] cfg {cfg} prior {prior} chunk {chunk} tokens {case.batch}", flush=True)
    ns = D.stage(case)
    D.run_step(case, ns)
    sync()
    res = O.decode_step(case)
    d = case.dims
    assert int(host(ns.status)[0]) == 0
    pool = host(ns.pool)
    for t, pos in enumerate(case.positions):
        pb, r = O.slot(case.table, int(case.token_seq[t]), int(pos), d.block_size)
        _close(d.cache_dtype, O.widen(pool[pb, r], d.cache_dtype),
               O.widen(res["pool"][pb, r], d.cache_dtype), f"row of token {t}")
    _close(d.cache_dtype, host(ns.v_combine), res["v_combine"], "v_combine")
    _close(d.cache_dtype, host(ns.out), res["out"].reshape(case.batch, -1), "out")
    if d.cache_dtype != O.F32:
        attn_on_oracle_query(case, ns, res, f"chunk cfg {cfg}")


def test_attn_tokens_equals_decode_on_an_expanded_table():
    """Query t through the sequence map reads what decode attention reads with
    a block table whose row t is the row of token t's sequence: bit for bit."""
    case = S.make_chunk_case(4, [3000, 777, 4100], [2, 3, 1], paged=True)
    ns = D.stage(case)
    ws = D.workspace(ns, 512)
    mla.attn_tokens(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.token_seq, ns.lens, ns.max_len,
                    ns.softmax_scale, ns.v_combine, ns.lse, 512, ws)
    wide = D.t(np.ascontiguousarray(case.table[case.token_seq]))
    vc2, lse2 = torch.empty_like(ns.v_combine), torch.empty_like(ns.lse)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, wide, ns.lens, ns.max_len,
                    ns.softmax_scale, vc2, lse2, 512, ws)
    sync()
    assert np.array_equal(host(ns.v_combine), host(vc2))
    assert np.array_equal(host(ns.lse), host(lse2))
    res = O.decode_step(case)
    attn_check(host(ns.v_combine), host(ns.lse), res["v_combine"], res["lse"], "tokens")


def _token_view(ns, t):
    """Token t of a staged chunk as a one-token step on the same pool and weights."""
    v = copy.copy(ns)
    sl = slice(t, t + 1)
    for f in ("x", "q", "positions", "token_seq", "lens", "q_abs_given"):
        a = getattr(ns, f)
        if a is not None:
            setattr(v, f, a[sl])
    v.q_abs = torch.empty_like(ns.q_abs[sl])
    v.v_combine = torch.empty_like(ns.v_combine[sl])
    v.lse = torch.empty_like(ns.lse[sl])
    v.out = torch.empty_like(ns.out[sl])
    return v


@pytest.mark.parametrize("cfg,prior,chunk", [(2, [500, 90], [3, 2]), (5, [300, 1100], [3, 2])])
def test_chunk_equals_token_by_token_bitwise(cfg, prior, chunk):
    """The stacked tokens (fewer than one 32-token tile) give, bit for bit,
    what the same tokens give one step at a time in position order, as the
    pages state for their n-token projections; the attention grid is fixed by
    passing the same split size and bound."""
    case = S.make_chunk_case(cfg, prior, chunk)
    ns, ns1 = D.stage(case), D.stage(case)
    D.run_step(case, ns, split_rows=256)
    outs, vcs = [], []
    for t in range(case.batch):                 # one token per step, sharing ns1's pool
        v = _token_view(ns1, t)
        D.run_step(case, v, split_rows=256)
        sync()
        outs.append(host(v.out)[0])
        vcs.append(host(v.v_combine)[0])
    assert np.array_equal(host(ns.pool), host(ns1.pool))
    assert np.array_equal(np.stack(vcs), host(ns.v_combine))
    assert np.array_equal(np.stack(outs), host(ns.out))


def test_bad_token_sequence_is_flagged_and_isolated():
    """A token naming a table row past the end: the append skips it and sets
    MLA_DEV_BAD_SEQ, its attention output is NaN; the other tokens are exact."""
    case = S.make_chunk_case(2, [200, 300], [2, 2])
    ns = D.stage(case)
    ref = O.decode_step(case)
    seq = case.token_seq.copy()
    seq[1] = 7                                  # only 2 rows in the table
    ns.token_seq = D.t(seq)
    ws = D.workspace(ns)
    D.append(ns, ws)
    sync()
    assert int(host(ns.status)[0]) == mla.MLA_DEV_BAD_SEQ
    mla.absorb_q(ns.dims, ns.q, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                 ws=ws)
    D.attend(ns, ns.q_abs, 0, ws)
    sync()
    vc = host(ns.v_combine)
    assert np.isnan(vc[1]).all()
    # token 0 sees rows up to its position; token 1's row (skipped) is not among them
    close_bf16(vc[0], ref["v_combine"][0], "token 0")
    close_bf16(vc[2:], ref["v_combine"][2:], "tokens 2, 3")


def test_token_calls_reject_missing_map():
    case = S.make_chunk_case(2, [40], [2])
    ns = D.stage(case)
    ws = D.workspace(ns)
    with pytest.raises(mla.MLAError):
        mla.attn_tokens(ns.dims, ns.q_abs, ns.pool, ns.table, None, ns.lens, ns.max_len,
                        ns.softmax_scale, ns.v_combine, ns.lse, 0, ws)
