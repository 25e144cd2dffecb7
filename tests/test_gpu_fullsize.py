"""GPU parity at the full sizes of configurations 2-5, in the launch configuration
the benchmark uses (automatic split plan), on sampled outputs.

The GPU runs the whole batch; the fp64 oracle recomputes a few sampled sequences
(sequences are independent, so the oracle runs on a sub-case holding just those
sequences, sharing the cache pool).  Tolerances: the bf16-cache bar,
|gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise, and for the attention call the
tight per-query checks of ``tests/parity.py`` (lse to 1e-4, v_combine to 4e-3 of
its largest value), which a missing tile or split at 131072 rows cannot pass.
Where the layer computes the query itself, the attention call is checked again
on the oracle's cache and stored query in the sampled rows.
"""
import copy

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import attn_check, close_bf16 as close

pytestmark = pytest.mark.gpu


def host(x):
    a = x.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def subset(case, idx):
    """The same step restricted to sequences ``idx`` (same pool and weights)."""
    sub = copy.copy(case)
    idx = np.asarray(idx)
    sub.batch = len(idx)
    sub.lens = case.lens[idx]
    sub.table = case.table[idx]
    for f in ("x", "q", "q_abs"):
        v = getattr(case, f)
        if v is not None:
            setattr(sub, f, v[idx])
    return sub


def run_layer(case):
    ns = D.stage(case)
    D.run_step(case, ns)          # split_rows = 0: the automatic plan, as the benchmark
    torch.cuda.synchronize()
    return host(ns.v_combine), host(ns.out), ns


def attn_on_oracle_query(ns, sample, ref, what):
    """decode_attn over the whole batch (automatic plan) on the oracle's cache
    (its own appended rows), with the oracle's stored query in the sampled
    rows; tight checks there."""
    q = ns.q_abs.clone()
    q[torch.as_tensor(sample, device=q.device)] = D.t(ref["q_abs_stored"])
    view = copy.copy(ns)
    view.pool = D.t(ref["pool"])
    ws = D.workspace(ns)
    D.attend(view, q, 0, ws)
    torch.cuda.synchronize()
    attn_check(host(ns.v_combine)[sample], host(ns.lse)[sample], ref["v_combine"], ref["lse"],
               f"{what}, sequences {sample}")


def test_full_config2_single_sequence():
    case = S.make_case(2)
    vc, out, ns = run_layer(case)
    ref = O.decode_step(case)
    close(vc, ref["v_combine"], "v_combine")
    close(out, ref["out"].reshape(case.batch, -1), "out")
    attn_on_oracle_query(ns, [0], ref, "1 x 4096")


def test_full_config3_ragged_paged_batch():
    case = S.make_case(3)
    vc, out, ns = run_layer(case)
    lens = case.lens
    sample = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 7, 40})
    ref = O.decode_step(subset(case, sample))
    close(vc[sample], ref["v_combine"], f"v_combine, sequences {sample}")
    close(out[sample], ref["out"].reshape(len(sample), -1), f"out, sequences {sample}")
    attn_on_oracle_query(ns, sample, ref, "ragged paged batch")


def test_full_config4_long_context_attention():
    case = S.make_case(4)
    ns = D.stage(case)
    ws = D.workspace(ns)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, ns.max_len,
                    ns.softmax_scale, ns.v_combine, ns.lse, 0, ws)
    torch.cuda.synchronize()
    vc, lse = host(ns.v_combine), host(ns.lse)
    del ns, ws
    for b in (0, 3):
        sub = subset(case, [b])
        q64 = O.widen(sub.q_abs, sub.dims.cache_dtype)
        rvc, rlse, _ = O.attention_latent(sub.dims, q64, sub.pool, sub.table, sub.lens,
                                          float(np.float32(case.softmax_scale)))
        attn_check(vc[b:b + 1], lse[b:b + 1], rvc, rlse, f"sequence {b}")


def test_full_config5_layer():
    case = S.make_case(5)
    vc, out, ns = run_layer(case)
    assert int(host(ns.status)[0]) == 0
    sample = [0, 19]
    ref = O.decode_step(subset(case, sample))
    close(vc[sample], ref["v_combine"], f"v_combine, sequences {sample}")
    close(out[sample], ref["out"].reshape(len(sample), -1), f"out, sequences {sample}")
    attn_on_oracle_query(ns, sample, ref, "layer batch")


def test_attn_more_queries_than_the_packed_scan():
    # past 4096 queries the split kernel maps its grid directly (one row per
    # query, empty splits written as empty) instead of packing the non-empty
    # (query, split) pairs; ragged, several splits per query, checked on a sample
    lens = [int(x) for x in np.random.default_rng(23).integers(1, 200, size=4100)]
    case = S.make_case(4, lens=lens, paged=True, seed=23)
    ns = D.stage(case)
    ws = D.workspace(ns, 64)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, ns.max_len,
                    ns.softmax_scale, ns.v_combine, ns.lse, 64, ws)
    torch.cuda.synchronize()
    vc, lse = host(ns.v_combine), host(ns.lse)
    for b in (0, 1, 2047, 4097, 4099):
        sub = subset(case, [b])
        q64 = O.widen(sub.q_abs, sub.dims.cache_dtype)
        rvc, rlse, _ = O.attention_latent(sub.dims, q64, sub.pool, sub.table, sub.lens,
                                          float(np.float32(case.softmax_scale)))
        attn_check(vc[b:b + 1], lse[b:b + 1], rvc, rlse, f"query {b} (len {lens[b]})")
