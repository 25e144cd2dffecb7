"""GPU parity: every call of the HIP library against the fp64 CPU oracle.

Inputs come from the seeded generators in ``mla_synth`` and are fed to both
sides.  Tolerances (stated by the target, applied elementwise):
  * fp32 caches: max |gpu - ref| <= 1e-4, and (non-replacing) <= 1e-3 max|ref|
  * bf16 caches: |gpu - ref| <= 2e-2 + 1e-2 |ref|
  * decode attention on a bf16 cache, beside that bar: per query every lse
    within 1e-4 + 1e-6 |lse| and max |v_combine error| <= 4e-3 max |v_combine|
    (``tests/parity.py``), so that a missing tile or split cannot pass
  * integer work (slots, untouched pool rows, paged == contiguous): bit-exact
"""
import copy
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import attn_check, attn_tight, close_bf16, close_f32

pytestmark = pytest.mark.gpu

def host(x):
    a = x.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# decode attention alone (q_abs drawn by the generator)
# ----------------------------------------------------------------------------
def attn_on_oracle_query(case, ns, res, what, split_rows=0):
    """Run decode attention on the oracle's inputs -- the query it stored and
    its cache after its own append -- and apply the tight checks against the
    oracle's attention.  (The layer's own rows and query carry the 4-bit
    projections' rounding, which on a short sequence moves lse by about the
    tight tolerance; the stated bar covers them.)"""
    q = D.t(res["q_abs_stored"])
    view = copy.copy(ns)
    view.pool = D.t(res["pool"])
    ws = D.workspace(ns, split_rows)
    D.attend(view, q, split_rows, ws)
    sync()
    attn_check(host(ns.v_combine), host(ns.lse), res["v_combine"], res["lse"],
               f"{what}: attention on the oracle's query")

def attn_only(case, ns, split_rows=0):
    ws = D.workspace(ns, split_rows)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, ns.max_len,
                    ns.softmax_scale, ns.v_combine, ns.lse, split_rows, ws)
    sync()
    return host(ns.v_combine), host(ns.lse)


def oracle_attn(case):
    q64 = O.widen(case.q_abs, case.dims.cache_dtype)
    vc, lse, _ = O.attention_latent(case.dims, q64, case.pool, case.table, case.lens,
                                    float(np.float32(case.softmax_scale)))
    return vc, lse


@pytest.mark.parametrize("split_rows", [0, 64, 128])
def test_attn_bf16_ragged_paged(split_rows):
    case = S.make_case(4, lens=[1, 33, 64, 300, 97], paged=True, seed=11)
    ns = D.stage(case)
    vc, lse = attn_only(case, ns, split_rows)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, f"split={split_rows}")


def test_attn_plan_from_lengths_ragged_paged():
    # the length-aware plan on a ragged, paged batch (the batched-decode shape at
    # reduced lengths, query given in latent form): exact against the oracle
    lens = [int(x) for x in np.random.default_rng(21).integers(64, 2500, size=24)]
    case = S.make_case(4, lens=lens, paged=True, seed=21)
    ns = D.stage(case)
    r, s = mla.attn_plan_lens(ns.dims, lens)
    assert r < mla.attn_plan(ns.dims, 24, max(lens), 0)[0] or r == 128
    vc, lse = attn_only(case, ns, r)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, f"plan ({r}, {s})")


def test_attn_more_splits_than_one_weight_chunk():
    # 71 splits of 64 rows for the long sequence: the combine walks its split
    # weights in chunks of 64; the short sequence leaves 69 splits empty.
    case = S.make_case(4, lens=[4500, 130], paged=True, seed=17)
    ns = D.stage(case)
    vc, lse = attn_only(case, ns, 64)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, "attention")


@pytest.mark.parametrize("lens", [[1100, 300], [2300, 64]], ids=["w2", "w4"])
def test_attn_merge_waves_per_head(lens):
    # 128-row splits: 9 splits for the first sequence (two merge waves per
    # head, one batch of 8 partial rows each after the first) and 18 (four
    # waves, the third batch on the first wave)
    case = S.make_case(4, lens=lens, paged=True, seed=29)
    ns = D.stage(case)
    print(f"merge waves per head: lens {lens}", flush=True)
    vc, lse = attn_only(case, ns, 128)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, f"lens {lens}")


def test_attn_merge_rounds_under_the_device_plan():
    # the automatic plan on one long sequence among short ones: the host plan
    # (sized for 64 sequences of the longest length) gives each query 4 splits,
    # so the merge's grid has one wave per head; the device plan cuts 128-row
    # splits from the lengths, 64 of them for the long sequence, whose heads
    # then take four rounds of four-wave groups
    lens = [8192] + [64] * 63
    case = S.make_case(4, lens=lens, paged=True, seed=31)
    ns = D.stage(case)
    r_host, s_host = mla.attn_plan(ns.dims, len(lens), max(lens), 0)
    assert s_host <= 8, (r_host, s_host)
    print(f"merge rounds: host plan {r_host} rows x {s_host}", flush=True)
    vc, lse = attn_only(case, ns, 0)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, "one long sequence among short ones")


def repage(case, block, seed):
    """The same logical rows in a pool of ``block``-row blocks, randomly permuted."""
    import dataclasses
    d = case.dims
    rng = np.random.default_rng(seed)
    rows = [O.gather_rows(case.pool, case.table, b, int(case.lens[b]), d.block_size)
            for b in range(case.batch)]
    nb = [(len(r) + block - 1) // block for r in rows]
    order = rng.permutation(sum(nb)).astype(np.int32)
    pool = np.full((sum(nb), block, d.width), S.BF16_NAN, dtype=np.uint16)
    table = np.full((case.batch, max(nb)), -1, dtype=np.int32)
    k = 0
    for b, r in enumerate(rows):
        ids = order[k:k + nb[b]]
        k += nb[b]
        table[b, :nb[b]] = ids
        flat = np.full((nb[b] * block, d.width), S.BF16_NAN, dtype=np.uint16)
        flat[:len(r)] = r
        pool[ids] = flat.reshape(nb[b], block, d.width)
    out = copy.copy(case)
    out.dims = dataclasses.replace(d, block_size=block)
    out.pool, out.table = pool, table
    return out


@pytest.mark.parametrize("block", [32, 128])
def test_attn_block_sizes(block):
    # tiles are 32 consecutive logical rows whatever the block size, so the
    # result must not change by a single bit when the same rows are re-paged
    case = S.make_case(4, lens=[700, 33, 129, 64], paged=True, seed=18)
    ns = D.stage(case)
    a64, l64 = attn_only(case, ns, 128)
    other = repage(case, block, seed=19)
    ns2 = D.stage(other)
    a, l = attn_only(other, ns2, 128)
    assert np.array_equal(a, a64) and np.array_equal(l, l64), f"block {block} != block 64"
    rvc, rlse = oracle_attn(other)
    attn_check(a, l, rvc, rlse, f"block={block}")


def test_attn_longest_single_split():
    # 32768 rows in one split: the split's tile table (1024 entries) is full
    case = S.make_case(4, batch=1, lens=[32768], seed=20)
    ns = D.stage(case)
    vc, lse = attn_only(case, ns, 32768)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, "attention")


def test_attn_bf16_invariances():
    case = S.make_case(4, lens=[700, 5, 129], paged=True, seed=12)
    ns = D.stage(case)
    a1, l1 = attn_only(case, ns, 64)
    a2, l2 = attn_only(case, ns, 64)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2), "run twice: not bit-identical"
    # paged == contiguous, bit for bit: same logical rows, identity table
    nb = [(int(x) + 63) // 64 for x in case.lens]
    pool_c = np.concatenate([case.pool[case.table[b, :nb[b]]] for b in range(len(nb))])
    table_c = np.full_like(case.table, -1)
    k = 0
    for b in range(len(nb)):
        table_c[b, :nb[b]] = np.arange(k, k + nb[b])
        k += nb[b]
    ns.pool, ns.table = D.t(pool_c), D.t(table_c)
    a3, l3 = attn_only(case, ns, 64)
    assert np.array_equal(a1, a3) and np.array_equal(l1, l3), "paged != contiguous"
    # one split versus many: same values to within the bf16 rounding of p
    a4, l4 = attn_only(case, ns, 0)
    assert np.max(np.abs(a4 - a1)) <= 2e-3 * np.max(np.abs(a1)) + 1e-6
    assert np.max(np.abs(l4 - l1)) <= 1e-4 * np.max(np.abs(l1))


def test_attn_empty_sequences():
    case = S.make_case(4, lens=[64, 1, 64], seed=13)
    ns = D.stage(case)
    ns.lens = D.t(np.array([64, 0, 64], dtype=np.int32))
    vc, lse = attn_only(case, ns, 0)
    assert np.all(vc[1] == 0) and np.all(np.isneginf(lse[1]))
    case.lens = np.array([64, 0, 64], dtype=np.int32)
    rvc, rlse = oracle_attn(case)
    attn_check(vc, lse, rvc, rlse, "with an empty sequence")
    # max_seq_len 0: everything empty
    ws = D.workspace(ns)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, 0, ns.softmax_scale,
                    ns.v_combine, ns.lse, 0, ws)
    sync()
    assert np.all(host(ns.v_combine) == 0) and np.all(np.isneginf(host(ns.lse)))


def test_attn_growing_scores_restart_path():
    # scores rise along the sequence by ~100 (log2 units) so the first tile's
    # reference is exceeded several times; the kernel must still match.
    case = S.make_case(4, lens=[400, 100], seed=14)
    d = case.dims
    q = np.zeros((2, 128, 576), dtype=np.float32)
    q[:, :, 0] = 8.0
    q[:, :, 1:] = np.random.default_rng(5).standard_normal((2, 128, 575)) * 0.1
    case.q_abs = S.to_bf16_bits(q)
    for b in range(2):
        rows = O.gather_rows(case.pool, case.table, b, int(case.lens[b]), 64).copy()
        vals = S.bf16_bits_to_f32(rows)
        vals[:, 0] = np.linspace(0, 60, len(vals))
        nbk = (int(case.lens[b]) + 63) // 64
        flat = case.pool[case.table[b, :nbk]].reshape(-1, 576)
        flat[:len(vals)] = S.to_bf16_bits(vals)
        case.pool[case.table[b, :nbk]] = flat.reshape(nbk, 64, 576)
    ns = D.stage(case)
    for split in (0, 128):
        vc, lse = attn_only(case, ns, split)
        rvc, rlse = oracle_attn(case)
        attn_check(vc, lse, rvc, rlse, f"split={split}")


@pytest.mark.parametrize("head", [5, 37, 127])
def test_attn_restart_needed_by_one_head(head):
    # One row's k_pe times 300 and the rope part of q kept in a single head
    # (not the first of its wave): only that head's maximum leaves the
    # reference's range, so the restart vote must count every lane of the
    # wave, not its first.
    case = S.make_case(4, lens=[300, 1000], seed=21)
    pool = S.bf16_bits_to_f32(case.pool)
    for b, r in ((0, 299), (1, 517)):
        pool[case.table[b][r // 64], r % 64, 512:] *= 300.0
    case.pool = S.to_bf16_bits(pool)
    q = S.bf16_bits_to_f32(case.q_abs)
    keep = q[:, head, 512:].copy()
    q[:, :, 512:] = 0.0
    q[:, head, 512:] = np.abs(keep) * np.sign(
        S.bf16_bits_to_f32(case.pool)[case.table[0][299 // 64], 299 % 64, 512:])
    case.q_abs = S.to_bf16_bits(q)
    ns = D.stage(case)
    rvc, rlse = oracle_attn(case)
    assert rlse[0, head] > rlse[0].max(initial=0, where=np.arange(128) != head) + 100
    for split in (0, 64, 2048):
        vc, lse = attn_only(case, ns, split)
        attn_check(vc, lse, rvc, rlse, f"head {head} split={split}")


@pytest.mark.parametrize("split", [0, 64])
def test_attn_first_tile_without_finite_scores(split):
    """Rows 0..31 of sequence 0 score -inf for every head (a -inf in a rope
    column that every head's query weights by +1; V is the latent part, so
    those rows only get probability 0).  A split whose first tile has no
    finite score must still end and match the oracle.  The latent part of
    the query is scaled by 16 so that later tiles' scores reach past the
    restart threshold and vote restarts from that state."""
    case = S.make_case(4, lens=[300, 100], seed=24)
    d = case.dims
    q = S.bf16_bits_to_f32(case.q_abs)
    q[:, :, :d.kv_lora] *= 16.0
    q[:, :, d.kv_lora] = 1.0
    case.q_abs = S.to_bf16_bits(q)
    nbk = (int(case.lens[0]) + 63) // 64
    flat = case.pool[case.table[0, :nbk]].reshape(-1, d.width)
    flat[:32, d.kv_lora] = 0xFF80                # bf16 -inf
    case.pool[case.table[0, :nbk]] = flat.reshape(nbk, 64, d.width)
    ns = D.stage(case)
    vc, lse = attn_only(case, ns, split)
    rvc, rlse = oracle_attn(case)
    assert np.isfinite(rvc).all() and np.isfinite(vc).all()
    attn_check(vc, lse, rvc, rlse, f"split={split}")


def test_attn_nan_first_tile_ends_with_nan():
    """NaN rows fill the first tile of sequence 0: its outputs are NaN (as in
    the oracle) and the call ends; sequence 1 is exact."""
    case = S.make_case(4, lens=[300, 100], seed=25)
    d = case.dims
    nbk = (int(case.lens[0]) + 63) // 64
    flat = case.pool[case.table[0, :nbk]].reshape(-1, d.width)
    flat[:32, :] = S.BF16_NAN
    case.pool[case.table[0, :nbk]] = flat.reshape(nbk, 64, d.width)
    ns = D.stage(case)
    for split in (0, 64):
        vc, lse = attn_only(case, ns, split)
        assert np.isnan(vc[0]).all() and np.isnan(lse[0]).all()
        rvc, rlse = oracle_attn(case)
        attn_check(vc[1:], lse[1:], rvc[1:], rlse[1:], f"other sequence, split={split}")


def test_attn_split_partials_beyond_fp16_range():
    # Latent values scaled by 2^17 (exact in bf16) and the latent part of q by
    # 2^-17: the scores are unchanged and v_combine scales by 2^17, past the
    # fp16 range the split partials are stored in, so the per-head exponent
    # must carry the scale through the combine.
    case = S.make_case(4, lens=[300, 200], seed=16)
    pool = S.bf16_bits_to_f32(case.pool)
    pool[..., :512] *= 2.0 ** 17
    case.pool = S.to_bf16_bits(pool)
    q = S.bf16_bits_to_f32(case.q_abs)
    q[..., :512] *= 2.0 ** -17
    case.q_abs = S.to_bf16_bits(q)
    ns = D.stage(case)
    rvc, rlse = oracle_attn(case)
    for split in (0, 64):
        vc, lse = attn_only(case, ns, split)
        assert np.isfinite(vc).all()
        close_bf16(vc * 2.0 ** -17, rvc * 2.0 ** -17, f"v_combine / 2^17 split={split}")
        attn_tight(vc, lse, rvc, rlse, f"split={split}")


def test_attn_split_partials_far_below_fp16_normals():
    # Latent values scaled by 2^-20 and the latent part of q by 2^20 (exact in
    # bf16): the scores are unchanged and v_combine scales by 2^-20, below the
    # smallest binary16 normal (2^-14) the split partials are stored in, so the
    # per-head exponent must lift them into range (fp16 subnormals would keep
    # 4 or fewer significant bits and miss the tight check).
    case = S.make_case(4, lens=[300, 200], seed=16)
    pool = S.bf16_bits_to_f32(case.pool)
    pool[..., :512] *= 2.0 ** -20
    case.pool = S.to_bf16_bits(pool)
    q = S.bf16_bits_to_f32(case.q_abs)
    q[..., :512] *= 2.0 ** 20
    case.q_abs = S.to_bf16_bits(q)
    ns = D.stage(case)
    rvc, rlse = oracle_attn(case)
    for split in (0, 64):
        vc, lse = attn_only(case, ns, split)
        close_bf16(vc * 2.0 ** 20, rvc * 2.0 ** 20, f"v_combine * 2^20 split={split}")
        attn_tight(vc, lse, rvc, rlse, f"split={split}")


def test_attn_f32_kernel_config1_shapes():
    case = S.make_case(1, sharp=True)
    rng = np.random.default_rng(15)
    case.lens = np.array([127], dtype=np.int32)      # row 127 is the (unwritten) append target
    case.q_abs = rng.standard_normal((1, 16, 80)).astype(np.float32)
    case.appended = False
    case.softmax_scale = 0.27046755772
    ns = D.stage(case)
    for split in (0, 64):
        vc, lse = attn_only(case, ns, split)
        rvc, rlse = oracle_attn(case)
        close_f32(vc, rvc, f"v_combine split={split}")
        close_f32(lse, rlse, f"lse split={split}")


# ----------------------------------------------------------------------------
# append, absorb, out_proj alone
# ----------------------------------------------------------------------------
def oracle_for(case):
    return O.decode_step(case)


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(lens=[200, 64, 1], batch=3, paged=True)),
                                    (5, dict(lens=[64] * 40, batch=40))])
def test_cache_append(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    ws = D.workspace(ns)
    mla.cache_append(ns.dims, ns.x, ns.kv_a, ns.kv_a_norm, ns.inv_freq, ns.rope_mscale,
                     ns.positions, ns.pool, ns.table, ns.status, ws)
    sync()
    got = host(ns.pool)
    res = oracle_for(case)
    d = case.dims
    assert int(host(ns.status)[0]) == 0
    written = np.zeros(got.shape[:2], dtype=bool)
    for b, pos in enumerate(case.positions):
        pb, r = O.slot(case.table, b, int(pos), d.block_size)
        written[pb, r] = True
        g = O.widen(got[pb, r], d.cache_dtype)
        ref = res["appended_rows"][b]
        if d.cache_dtype == O.F32:
            assert np.max(np.abs(g - ref)) <= 1e-5 * max(1.0, np.max(np.abs(ref)))
        elif case.kv_a is None or O.weight_dtype(case.kv_a) != O.Q4G64:
            # within one bf16 step of the unrounded row
            assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
        else:
            # 4-bit kv_a on fp16 MFMA: operand rounding leaves ~4e-4 rms(row) on
            # top of the bf16 step; 2e-3 rms(row) is about five of those sigmas
            rms = np.sqrt(np.mean(ref ** 2))
            assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-3 * rms)
            close_bf16(g, ref, "appended row")
    # every other row bit-identical (NaN fill included)
    assert np.array_equal(got[~written].view(np.uint8), case.pool[~written].view(np.uint8))


def test_cache_append_bad_positions_flagged():
    case = S.make_case(2, lens=[64, 64], batch=2)
    ns = D.stage(case)
    ns.positions = D.t(np.array([64 * case.table.shape[1], -1], dtype=np.int32))
    ws = D.workspace(ns)
    before = host(ns.pool).copy()
    mla.cache_append(ns.dims, ns.x, ns.kv_a, ns.kv_a_norm, ns.inv_freq, ns.rope_mscale,
                     ns.positions, ns.pool, ns.table, ns.status, ws)
    sync()
    assert int(host(ns.status)[0]) == mla.MLA_DEV_POS_RANGE
    assert np.array_equal(host(ns.pool), before)
    # a table entry out of range
    table = case.table.copy()
    table[0, 0] = 10 ** 6
    ns.table = D.t(table)
    ns.positions = D.t(np.array([3, 3], dtype=np.int32))
    ns.status.zero_()
    mla.cache_append(ns.dims, ns.x, ns.kv_a, ns.kv_a_norm, ns.inv_freq, ns.rope_mscale,
                     ns.positions, ns.pool, ns.table, ns.status, ws)
    sync()
    assert int(host(ns.status)[0]) == mla.MLA_DEV_BAD_BLOCK


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(lens=[300, 1000], batch=2)),
                                    (5, dict(lens=[70, 200], batch=2)),
                                    (5, dict(lens=[64] * 40, batch=40)),
                                    (5, dict(lens=[64] * 96, batch=96))])
def test_absorb_q(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    ws = D.workspace(ns)
    q_in = ns.q if ns.q is not None else ns.x
    mla.absorb_q(ns.dims, q_in, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                 ns.q_a, ns.q_a_norm, ns.q_b, ws)
    sync()
    res = oracle_for(case)
    got = O.widen(host(ns.q_abs), case.dims.cache_dtype)
    if case.dims.cache_dtype == O.F32:
        close_f32(got, res["q_abs64"], "q_abs")
    else:
        close_bf16(got, res["q_abs64"], "q_abs")
        # stored bf16 values sit within one step of the exact product
        ok = np.abs(got - res["q_abs64"]) <= 2.0 ** -7 * np.abs(res["q_abs64"]) + 1e-3
        assert ok.mean() > 0.999


def test_chain_hidden_state_beyond_fp16_range():
    # One token's hidden state holds values far past binary16's range (1.5e5,
    # -8e4) and another's lies far below its normals (x 2^-20).  The 4-bit
    # projections pack x per token by a power of two (and the q latent and
    # the absorbed q_nope rows likewise), so nothing overflows or underflows:
    # the appended rows, q_abs and the layer match the oracle at the bar.
    case = S.make_case(5, batch=3, lens=[300, 1100, 64])
    x = case.x.copy()
    x[0, 17], x[0, 4000] = 1.5e5, -8.0e4
    x[1] *= 2.0 ** -20
    case.x = x
    ns = D.stage(case)
    D.run_step(case, ns)
    sync()
    res = O.decode_step(case)
    assert int(host(ns.status)[0]) == 0
    # per token, relative to the token's own scale as well (the 2^-20 token's
    # rows are far below the absolute part of the bar): fp16 subnormals would
    # leave ~3% errors there, the scaled pack leaves the bf16 rounding
    bs = case.dims.block_size
    got_pool, ref_pool = O.widen(host(ns.pool), O.BF16), O.widen(res["pool"], O.BF16)
    got_q = O.widen(host(ns.q_abs), O.BF16)
    for b, (pos, blk) in enumerate(zip(case.positions, case.table)):
        r = got_pool[blk[pos // bs], pos % bs]
        ref = ref_pool[blk[pos // bs], pos % bs]
        close_bf16(r, ref, f"appended row of sequence {b}")
        assert np.max(np.abs(r - ref)) <= 1e-2 * np.max(np.abs(ref)), f"row {b} relative"
        dq = np.max(np.abs(got_q[b] - res["q_abs64"][b]))
        assert dq <= 1e-2 * np.max(np.abs(res["q_abs64"][b])), f"q_abs of token {b} relative"
    close_bf16(got_q, res["q_abs64"], "q_abs")
    close_bf16(host(ns.v_combine), res["v_combine"], "v_combine")
    close_bf16(host(ns.out), res["out"].reshape(case.batch, -1), "out")


def test_absorb_q_latent_beyond_fp16_range():
    # q_a_norm's gamma times 2^20 (exact in bf16): the normalised q latent and
    # q itself reach ~1e6, past binary16's range, on the way to q_b and the
    # absorb MFMAs.  q_abs scales by 2^20 exactly, so the bar applies to
    # q_abs / 2^20 as it does at the unscaled size.
    case = S.make_case(5, batch=2, lens=[300, 1100])
    case.q_a_norm = S.to_bf16_bits(S.bf16_bits_to_f32(case.q_a_norm) * 2.0 ** 20)
    ns = D.stage(case)
    ws = D.workspace(ns)
    mla.absorb_q(ns.dims, ns.x, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                 ns.q_a, ns.q_a_norm, ns.q_b, ws)
    sync()
    res = oracle_for(case)
    got = O.widen(host(ns.q_abs), case.dims.cache_dtype)
    assert np.isfinite(got).all()
    assert np.max(np.abs(res["q_abs64"])) > 65504.0
    close_bf16(got * 2.0 ** -20, res["q_abs64"] * 2.0 ** -20, "q_abs / 2^20")


def q_chain_case(heads, kv_lora, q_lora, batch, cache_dtype, seed):
    """A 4-bit q chain with q_nope 128 and q_pe 64 at a latent width and q LoRA
    rank other than the full-size ones (q_b and the absorb then run as one
    launch over any rank of 1 to 12 units of 128 and any latent of 32 to 512)."""
    rng = np.random.default_rng(seed)
    H, N, R, V, C = heads, 128, 64, 128, kv_lora
    d = S.Dims(num_heads=H, qk_nope=N, qk_rope=R, v_head=V, kv_lora=C, hidden=256,
               q_lora=q_lora, cache_dtype=cache_dtype)
    L = rng.integers(40, 400, size=batch).astype(np.int32)
    pool, table = S.build_pool(rng, d, L, std=1.0, paged=True)
    return S.Case("q-chain", d, S.Yarn(), batch, L, pool, table, None,
                  x=rng.standard_normal((batch, d.hidden), dtype=np.float32),
                  kv_a=S.draw_q4(rng, C + R, d.hidden),
                  kv_a_norm=S.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(C)),
                  q_a=S.draw_q4(rng, q_lora, d.hidden),
                  q_a_norm=S.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(q_lora)),
                  q_b=S.draw_q4(rng, H * (N + R), q_lora),
                  kv_b=S.draw_q4(rng, H * (N + V), C),
                  o_proj=S.draw_q4(rng, d.hidden, H * V))


# (heads, latent, q LoRA rank, batch, cache dtype, tiled weights): one unit (the
# second K half empty), an odd count (halves of 2 and 1), 5 units, two token
# tiles with a ragged second one, a latent that leaves half the absorb's
# waves without columns
@pytest.mark.parametrize("H,C,ql,B,dt,tiled", [(16, 256, 128, 37, S.F32, False),
                                               (16, 512, 384, 37, S.BF16, True),
                                               (8, 256, 640, 5, S.BF16, False),
                                               (8, 128, 1536, 33, S.F32, True)])
def test_absorb_q_chain_other_shapes(H, C, ql, B, dt, tiled):
    case = q_chain_case(H, C, ql, B, dt, seed=H + C + ql + B)
    print(f"q chain: H {H} C {C} q_lora {ql} batch {B} tiled {tiled}", flush=True)
    ns = D.stage(case, tiled=tiled)
    ws = D.workspace(ns)
    mla.absorb_q(ns.dims, ns.x, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                 ns.q_a, ns.q_a_norm, ns.q_b, ws)
    sync()
    res = O.decode_step(case)
    got = O.widen(host(ns.q_abs), dt)
    assert np.isfinite(got).all()
    # the 4-bit chain multiplies fp16 operands whatever the cache dtype, so
    # the bf16 bar is the one that applies to an fp32 q_abs as well
    close_bf16(got, res["q_abs64"], "q_abs")


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(lens=[50, 10], batch=2)),
                                    (5, dict(lens=[70, 200], batch=2)),
                                    (5, dict(lens=[64] * 40, batch=40))])
def test_out_proj(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    rng = np.random.default_rng(16)
    vc = rng.standard_normal((case.batch, case.dims.num_heads, case.dims.kv_lora)).astype(np.float32)
    ns.v_combine = D.t(vc)
    ws = D.workspace(ns)
    mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, ns.out, ns.o_proj, ws)
    sync()
    d = case.dims
    kvb = O.weight_f64(case.kv_b, O.weight_dtype(case.kv_b), d.num_heads * (d.qk_nope + d.v_head),
                       d.kv_lora)
    o64 = (O.weight_f64(case.o_proj, O.weight_dtype(case.o_proj), d.hidden,
                        d.num_heads * d.v_head) if case.o_proj is not None else None)
    ref = O.out_proj(d, vc.astype(np.float64), kvb, o64).reshape(case.batch, -1)
    got = host(ns.out)
    if d.cache_dtype == O.F32:
        close_f32(got, ref, "out")
    else:
        close_bf16(got, ref, "out")
        # 4-bit weights run on fp16 MFMA: each operand rounded to an 11-bit
        # significand gives ~4e-4 rms relative error per GEMM stage, two stages
        # here, so the largest error over the outputs stays well under 2e-3 max|ref|.
        lim = 2e-3 if O.weight_dtype(case.kv_b) == O.Q4G64 else 1e-4
        assert np.max(np.abs(got - ref)) <= lim * np.max(np.abs(ref))


# ----------------------------------------------------------------------------
# Q8_0 kv_b (absorb and expansion read the blocks in place)
# ----------------------------------------------------------------------------
Q8_CASES = [(1, {}), (2, dict(lens=[300, 1000], batch=2)), (5, dict(lens=[70, 200], batch=2))]


@pytest.mark.parametrize("cfg,kw", Q8_CASES)
def test_absorb_q_q8_0_kv_b(cfg, kw):
    case = S.with_q8_0_kv_b(S.make_case(cfg, **kw))
    ns = D.stage(case)
    assert ns.kv_b.dtype == mla.MLA_Q8_0
    ws = D.workspace(ns)
    q_in = ns.q if ns.q is not None else ns.x
    mla.absorb_q(ns.dims, q_in, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                 ns.q_a, ns.q_a_norm, ns.q_b, ws)
    sync()
    res = oracle_for(case)
    got = O.widen(host(ns.q_abs), case.dims.cache_dtype)
    if case.dims.cache_dtype == O.F32:
        close_f32(got, res["q_abs64"], "q_abs")
    else:
        close_bf16(got, res["q_abs64"], "q_abs")


@pytest.mark.parametrize("cfg,kw", Q8_CASES)
def test_out_proj_q8_0_kv_b(cfg, kw):
    case = S.with_q8_0_kv_b(S.make_case(cfg, **kw))
    ns = D.stage(case)
    rng = np.random.default_rng(17)
    vc = rng.standard_normal((case.batch, case.dims.num_heads, case.dims.kv_lora)).astype(np.float32)
    ns.v_combine = D.t(vc)
    ws = D.workspace(ns)
    mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, ns.out, ns.o_proj, ws)
    sync()
    d = case.dims
    kvb = O.weight_f64(case.kv_b, O.Q8_0, d.num_heads * (d.qk_nope + d.v_head), d.kv_lora)
    o64 = (O.weight_f64(case.o_proj, O.weight_dtype(case.o_proj), d.hidden,
                        d.num_heads * d.v_head) if case.o_proj is not None else None)
    ref = O.out_proj(d, vc.astype(np.float64), kvb, o64).reshape(case.batch, -1)
    got = host(ns.out)
    if d.cache_dtype == O.F32:
        close_f32(got, ref, "out")
    else:
        close_bf16(got, ref, "out")
        # W_UV runs on fp16 MFMA operands (v_combine rounded to binary16, d*q
        # rounded to binary16) with fp32 sums: ~4e-4 rms relative per stage
        assert np.max(np.abs(got - ref)) <= 2e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("cfg,kw", [(2, dict(lens=[1000, 37], batch=2)),
                                    (3, dict(batch=3, lens=[1024, 1500, 2049])),
                                    (5, dict(batch=2, lens=[300, 1100]))])
def test_chain_q8_0_kv_b(cfg, kw):
    case = S.with_q8_0_kv_b(S.make_case(cfg, **kw))
    ns = D.stage(case)
    D.run_step(case, ns)
    sync()
    res = O.decode_step(case)
    close_bf16(host(ns.v_combine), res["v_combine"], "v_combine")
    close_bf16(host(ns.out), res["out"].reshape(case.batch, -1), "out")
    attn_on_oracle_query(case, ns, res, "Q8_0 chain")


# ----------------------------------------------------------------------------
# the whole step, reduced sizes
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,kw", [
    (1, {}),
    (1, dict(sharp=True)),
    (2, dict(lens=[1000, 37], batch=2)),
    (3, dict(batch=3, lens=[1024, 1500, 2049])),
    (5, dict(batch=2, lens=[300, 1100])),
])
def test_chain(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    D.run_step(case, ns)
    sync()
    res = O.decode_step(case)
    d = case.dims
    vc, out = host(ns.v_combine), host(ns.out)
    if d.cache_dtype == O.F32:
        close_f32(vc, res["v_combine"], "v_combine")
        close_f32(out, res["out"].reshape(case.batch, -1), "out")
    else:
        close_bf16(vc, res["v_combine"], "v_combine")
        close_bf16(out, res["out"].reshape(case.batch, -1), "out")
    # against the unabsorbed definition (q_abs not rounded), on a few heads
    res_u = O.decode_step(case, model_q_abs_storage=False)
    heads = list(range(0, d.num_heads, max(1, d.num_heads // 4)))
    o1, _ = O.attention_unabsorbed(d, res_u["q"], res_u["kv_b64"], res_u["pool"], case.table,
                                   case.lens, res_u["softmax_scale"], res_u["inv_freq"],
                                   res_u["rope_mscale"], case.positions, heads=heads)
    if case.o_proj is None:
        got = out.reshape(case.batch, d.num_heads, d.v_head)[:, heads]
        if d.cache_dtype == O.F32:
            close_f32(got, o1, "out vs unabsorbed")
        else:
            close_bf16(got, o1, "out vs unabsorbed")
    if d.cache_dtype == O.F32:
        return
    if case.o_proj is not None:
        # the 4-bit layer against the unabsorbed definition: the per-head W_UV
        # outputs (o_proj not applied) on the sampled heads, and o_proj applied
        # to the unabsorbed attention of every head against the layer's output
        ws = D.workspace(ns)
        per_head = torch.empty((case.batch, d.num_heads * d.v_head), dtype=torch.float32,
                               device="cuda")
        mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, per_head, None, ws)
        sync()
        got = host(per_head).reshape(case.batch, d.num_heads, d.v_head)
        close_bf16(got[:, heads], o1, "per-head W_UV output vs unabsorbed")
        o_all, _ = O.attention_unabsorbed(d, res_u["q"], res_u["kv_b64"], res_u["pool"],
                                          case.table, case.lens, res_u["softmax_scale"],
                                          res_u["inv_freq"], res_u["rope_mscale"], case.positions)
        o64 = O.weight_f64(case.o_proj, O.weight_dtype(case.o_proj), d.hidden,
                           d.num_heads * d.v_head)
        y1 = O.matvec(o64, o_all.reshape(case.batch, -1))
        close_bf16(out, y1, "layer output vs o_proj of the unabsorbed attention")
    # the attention call alone, tight, on the GPU's cache with the oracle's query
    attn_on_oracle_query(case, ns, res, "chain")


@pytest.mark.parametrize("cfg,lens", [(4, [100, 2000]), (1, [100, 600])])
def test_bad_table_entry_gives_nan_through_the_merge(cfg, lens):
    """A block-table entry out of range inside a sequence's length makes that
    sequence's outputs NaN, also when its only non-empty split is the bad one
    and the merge sees the other splits empty; the other sequence is exact."""
    case = S.make_case(cfg, lens=lens, paged=False)
    ref = O.decode_step(case)
    ns = D.stage(case)
    bad = case.table.copy()
    bad[0, 0] = case.pool.shape[0] + 5          # rows 0..63 of sequence 0
    ns.table = D.t(bad)
    q_abs = ns.q_abs_given
    if q_abs is None:                           # fp32 case: q through the absorb
        ws0 = D.workspace(ns)
        D.append(ns, ws0)
        mla.absorb_q(ns.dims, ns.q, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions,
                     ns.q_abs, ws=ws0)
        q_abs = ns.q_abs
    split = 64 if cfg == 1 else 256
    ws = D.workspace(ns, split)
    mla.decode_attn(ns.dims, q_abs, ns.pool, ns.table, ns.lens, ns.max_len, ns.softmax_scale,
                    ns.v_combine, ns.lse, split, ws)
    sync()
    assert mla.attn_plan(ns.dims, 2, ns.max_len, split)[1] > 1
    vc, lse = host(ns.v_combine), host(ns.lse)
    assert np.isnan(vc[0]).all() and np.isnan(lse[0]).all()
    if case.dims.cache_dtype == O.F32:
        close_f32(vc[1], ref["v_combine"][1], "other sequence")
    else:
        attn_check(vc[1:], lse[1:], ref["v_combine"][1:], ref["lse"][1:], "other sequence")
