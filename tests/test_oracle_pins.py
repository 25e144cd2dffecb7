"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties one part of ``oracle/mla_oracle.py`` to a closed form, a hand
derivation stored under ``tests/golden/``, a library routine (torch SDPA,
scipy logsumexp), an invariant, or a pure-Python brute force on tiny inputs.
None of these tests needs a GPU.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

from oracle import mla_oracle as O
import mla_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# storage: bf16 rounding, 4-bit dequant
# ----------------------------------------------------------------------------
def test_bf16_rounding_golden():
    g = golden("bf16_rounding.json")
    got = O.round_bf16(np.array(g["values"]))
    assert got.tolist() == g["bits"]


def test_bf16_rounding_matches_float32_path_on_float32_inputs():
    # On float32 inputs there is no double rounding, so the oracle's direct
    # rounding and the generator's independent float32 bit trick must agree.
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([0.0, -0.0, 3.0e38, -3.0e38], dtype=np.float32)])
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), S.to_bf16_bits(x))


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xC020, 0x0001, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.5, 2.0 ** -133, 3.3895313892515355e38]
    assert O.widen(bits, O.BF16).tolist() == want


def test_q4_dequant_golden():
    g = golden("q4_row.json")
    w = O.dequant_q4(np.array(g["packed"], dtype=np.uint32),
                     np.array([g["scale_bits"]], dtype=np.uint16),
                     np.array([g["bias_bits"]], dtype=np.uint16), 1, 64)
    assert w[0, :16].tolist() == g["expected_first16"]
    assert w[0, 16:32].tolist() == g["expected_first16"]


def test_q4_quantise_dequantise_error_bound():
    # brute force: pick the nearest nibble for each value given (scale, bias);
    # dequantising must land within scale/2 of any value inside the grid's range.
    rng = np.random.default_rng(3)
    rows, cols = 3, 128
    lo = rng.uniform(-1.0, -0.5, size=(rows, cols // 64))
    hi = rng.uniform(0.5, 1.0, size=(rows, cols // 64))
    scale_b = S.to_bf16_bits((hi - lo) / 15.0)
    bias_b = S.to_bf16_bits(lo)
    sc = S.bf16_bits_to_f32(scale_b).astype(np.float64)
    bi = S.bf16_bits_to_f32(bias_b).astype(np.float64)
    vals = np.empty((rows, cols))
    packed = np.zeros((rows, cols // 8), dtype=np.uint32)
    for r in range(rows):
        for k in range(cols):
            g = k // 64
            v = rng.uniform(bi[r, g], bi[r, g] + 15 * sc[r, g])
            vals[r, k] = v
            best = min(range(16), key=lambda q: abs(sc[r, g] * q + bi[r, g] - v))
            packed[r, k // 8] |= np.uint32(best) << np.uint32(4 * (k % 8))
    w = O.dequant_q4(packed, scale_b, bias_b, rows, cols)
    tol = np.repeat(sc, 64, axis=1) / 2 * (1 + 1e-12)
    assert np.all(np.abs(w - vals) <= tol)


def _q8_0_block(scale_half_bits: int, q) -> bytes:
    """One Q8_0 block spelled out byte by byte: little-endian binary16 scale, 32 signed bytes."""
    assert len(q) == 32
    return struct.pack("<H", scale_half_bits) + struct.pack("<32b", *q)


def test_q8_0_dequant_single_block_closed_form():
    # d = 0.5 (binary16 0x3800); q spans the whole int8 range, so a byte read as
    # unsigned, a swapped scale byte order or a dropped scale all fail.
    q = [0, 1, -1, 2, -2, 127, -128, 64, -64, 3, -3, 100, -100, 5, -5, 7,
         -7, 9, -9, 11, -11, 13, -13, 15, -15, 17, -17, 19, -19, 21, -21, 126]
    raw = np.frombuffer(_q8_0_block(0x3800, q), dtype=np.uint8)
    w = O.dequant_q8_0(raw, 1, 32)
    assert w.shape == (1, 32)
    assert w[0].tolist() == [0.5 * v for v in q]
    assert O.weight_f64(raw, O.Q8_0, 1, 32).tolist() == w.tolist()
    assert O.weight_dtype(raw) == O.Q8_0


def test_q8_0_block_order_and_scales():
    # 2 rows x 64 columns = 4 blocks, row-major, each with its own scale:
    # 1.0 (0x3c00), -2.0 (0xc000), 2^-14 (0x0400, smallest normal) and the
    # subnormal 2^-24 (0x0001); q = k + 1 - 16 * (block index) within a block.
    scales = [(0x3C00, 1.0), (0xC000, -2.0), (0x0400, 2.0 ** -14), (0x0001, 2.0 ** -24)]
    raw = b""
    expect = np.zeros((2, 64))
    for blk, (bits, d) in enumerate(scales):
        q = [(k + 1 - 16 * blk) for k in range(32)]
        raw += _q8_0_block(bits, q)
        r, c0 = divmod(blk, 2)
        expect[r, 32 * c0:32 * c0 + 32] = [d * v for v in q]
    w = O.dequant_q8_0(np.frombuffer(raw, dtype=np.uint8), 2, 64)
    assert np.array_equal(w, expect)


def test_q8_0_round_trip_of_grid_values():
    # values on a block's grid d * q (|q| <= 127) come back exactly
    rng = np.random.default_rng(11)
    rows, cols = 3, 96
    d = np.float16(rng.uniform(0.01, 0.1, size=(rows, cols // 32)))
    q = rng.integers(-127, 128, size=(rows, cols))
    raw = bytearray()
    for r in range(rows):
        for b in range(cols // 32):
            raw += _q8_0_block(int(d[r, b].view(np.uint16)), q[r, 32 * b:32 * b + 32].tolist())
    w = O.dequant_q8_0(np.frombuffer(bytes(raw), dtype=np.uint8), rows, cols)
    assert np.array_equal(w, np.repeat(d.astype(np.float64), 32, axis=1) * q)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def test_rope_consecutive_pairing_golden():
    g = golden("rope_quarter_turn.json")
    got = O.rope_consecutive(np.array(g["x"]), g["pos"], np.array(g["inv_freq"]))
    assert np.allclose(got, g["expected"], atol=1e-15)
    assert not np.allclose(got, g["neox_pairing_would_give"], atol=1e-3)


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    inv = O.yarn_inv_freq(64, 1e4, 40, 4096, 32, 1)
    assert np.array_equal(O.rope_consecutive(x, 0.0, inv), x)


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 16))
    inv = O.yarn_inv_freq(16, 1e4, 40, 4096, 32, 1)
    y = O.rope_consecutive(x, 127.0, inv)
    assert np.allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                       rtol=1e-13)
    # R(a) R(b) = R(a + b)
    assert np.allclose(O.rope_consecutive(O.rope_consecutive(x, 40.0, inv), 87.0, inv), y,
                       atol=1e-12)


def test_rope_relative_position_property():
    # <R(m) q, R(n) k> = <R(m - n) q, k>: the score depends only on the offset.
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    inv = O.yarn_inv_freq(64, 1e4, 40, 4096, 32, 1)
    lhs = O.rope_consecutive(q, 1000.0, inv) @ O.rope_consecutive(k, 937.0, inv)
    rhs = O.rope_consecutive(q, 63.0, inv) @ k
    assert abs(lhs - rhs) < 1e-11


def test_rope_brute_force_scalar_loop():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(8)
    inv = [0.9, 0.31, 0.05, 0.002]
    pos, ms = 5.0, 1.25
    want = []
    for i in range(4):
        a = pos * inv[i]
        want += [ms * (x[2 * i] * math.cos(a) - x[2 * i + 1] * math.sin(a)),
                 ms * (x[2 * i] * math.sin(a) + x[2 * i + 1] * math.cos(a))]
    assert np.allclose(O.rope_consecutive(x, pos, np.array(inv), ms), want, atol=1e-15)


# ----------------------------------------------------------------------------
# YaRN
# ----------------------------------------------------------------------------
def test_yarn_golden_deepseek_v3():
    g = golden("yarn_deepseek_v3.json")
    args = (g["theta"], g["original_max_pos"], g["beta_fast"], g["beta_slow"])
    assert list(O.yarn_correction_range(64, *args)) == g["R64_low_high"]
    assert list(O.yarn_correction_range(16, *args)) == g["R16_low_high"]
    inv = O.yarn_inv_freq(64, g["theta"], g["factor"], g["original_max_pos"], g["beta_fast"],
                          g["beta_slow"])
    for i, v in g["R64_inv_freq_at"].items():
        assert inv[int(i)] == pytest.approx(v, rel=1e-12)
    assert O.yarn_get_mscale(40.0, 1.0) == pytest.approx(g["mscale_factor40"], rel=1e-15)
    rm, sc = O.yarn_scalars(40.0, 1.0, 1.0, 192)
    assert rm == g["rope_mscale"]
    assert sc == pytest.approx(g["softmax_scale_qk192"], rel=1e-14)
    assert O.yarn_scalars(40.0, 1.0, 1.0, 48)[1] == pytest.approx(g["softmax_scale_qk48"], rel=1e-14)


def test_yarn_factor_one_is_plain_rope():
    for R in (16, 64):
        inv = O.yarn_inv_freq(R, 1e4, 1.0, 4096, 32, 1)
        assert np.allclose(inv, 1e4 ** (-np.arange(0, R, 2) / R), rtol=1e-14)
    assert O.yarn_get_mscale(1.0, 1.0) == 1.0
    assert O.yarn_get_mscale(0.5, 3.0) == 1.0


def test_yarn_correction_dims_match_rotation_counts():
    # A pair turns orig * theta^(-2i/R) / (2 pi) times over the original context.
    # low is the last pair still turning >= beta_fast times; high the first
    # pair turning <= beta_slow times.
    for R in (16, 64, 128):
        theta, orig, bf, bs = 1e4, 4096.0, 32.0, 1.0
        turns = [orig * theta ** (-2.0 * i / R) / (2 * math.pi) for i in range(R)]
        low, high = O.yarn_correction_range(R, theta, orig, bf, bs)
        assert turns[low] >= bf > turns[low + 1]
        assert turns[high - 1] > bs >= turns[high]


def test_yarn_ramp_endpoints_and_monotone():
    R, factor = 64, 40.0
    inv = O.yarn_inv_freq(R, 1e4, factor, 4096, 32, 1)
    base = 1e4 ** (-np.arange(0, R, 2) / R)
    low, high = O.yarn_correction_range(R, 1e4, 4096, 32, 1)
    assert np.allclose(inv[:low + 1], base[:low + 1], rtol=1e-15)
    assert np.allclose(inv[high:], base[high:] / factor, rtol=1e-15)
    mid = inv[low + 1:high] / base[low + 1:high]
    assert np.all(mid < 1.0) and np.all(mid > 1.0 / factor) and np.all(np.diff(mid) < 0)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------
def test_rmsnorm_golden():
    g = golden("rmsnorm_3_4.json")
    x = np.array(g["x"])
    assert np.allclose(O.rmsnorm(x, np.ones(2), g["eps"]), g["gamma_ones_expected"], rtol=1e-14)
    assert np.allclose(O.rmsnorm(x, np.array(g["gamma"]), g["eps"]), g["gamma_expected"],
                       rtol=1e-14)


def test_rmsnorm_closed_form_mean_square():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 512)) * 0.3
    eps = 1e-6
    y = O.rmsnorm(x, np.ones(512), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13)


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _tiny_latent_case(H=3, C=8, R=4, L=(5, 1, 9), block=4, dtype=O.F32, seed=0, paged=True):
    rng = np.random.default_rng(seed)
    d = S.Dims(num_heads=H, qk_nope=2, qk_rope=R, v_head=2, kv_lora=C, block_size=block,
               cache_dtype=dtype)
    pool, table = S.build_pool(rng, d, np.array(L), paged=paged, appended=False)
    q_abs = rng.standard_normal((len(L), H, C + R))
    return d, pool, table, np.array(L), q_abs


def test_two_row_softmax_closed_form():
    # H=1, C=2, R=2, scale 1.  q_abs = [1, 0, 0, 0] picks row[0] as the score.
    # Scores ln 3 and 0 give weights 3/4 and 1/4; lse = ln 4.
    d = S.Dims(num_heads=1, qk_nope=1, qk_rope=2, v_head=1, kv_lora=2, block_size=2,
               cache_dtype=O.F32)
    pool = np.array([[[math.log(3.0), 5.0, 0.0, 0.0], [0.0, -7.0, 0.0, 0.0]]], dtype=np.float32)
    table = np.array([[0]], dtype=np.int32)
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    vc, lse, p = O.attention_latent(d, q, pool, table, [2], 1.0)
    l3 = float(np.float32(math.log(3.0)))
    assert p[0][0].tolist() == pytest.approx([0.75, 0.25], abs=1e-7)
    assert vc[0, 0].tolist() == pytest.approx([0.75 * l3, 0.75 * 5.0 - 0.25 * 7.0], abs=1e-7)
    assert lse[0, 0] == pytest.approx(math.log(4.0), abs=1e-7)


def test_softmax_rows_sum_to_one_and_lse_matches_scipy():
    from scipy.special import logsumexp
    d, pool, table, L, q = _tiny_latent_case()
    vc, lse, ps = O.attention_latent(d, q, pool, table, L, 0.37)
    for b, p in enumerate(ps):
        assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
        rows = O.widen(O.gather_rows(pool, table, b, int(L[b]), d.block_size), O.F32)
        s = 0.37 * q[b] @ rows.T
        assert np.allclose(lse[b], logsumexp(s, axis=1), rtol=1e-13)


def test_single_row_returns_that_row():
    d, pool, table, L, q = _tiny_latent_case(L=(1, 1), dtype=O.BF16)
    vc, lse, _ = O.attention_latent(d, q, pool, table, L, 0.5)
    for b in range(2):
        row = O.widen(O.gather_rows(pool, table, b, 1, d.block_size), O.BF16)[0]
        for h in range(d.num_heads):
            assert np.array_equal(vc[b, h], row[:d.kv_lora])


def test_zero_query_gives_row_mean():
    d, pool, table, L, q = _tiny_latent_case()
    vc, _, _ = O.attention_latent(d, np.zeros_like(q), pool, table, L, 1.0)
    for b in range(len(L)):
        rows = O.widen(O.gather_rows(pool, table, b, int(L[b]), d.block_size), O.F32)
        assert np.allclose(vc[b], rows[:, :d.kv_lora].mean(axis=0)[None, :], atol=1e-14)


def test_empty_sequence_defined_as_zero_and_minus_inf():
    d, pool, table, L, q = _tiny_latent_case(L=(3, 2))
    vc, lse, _ = O.attention_latent(d, q, pool, table, [3, 0], 1.0)
    assert np.all(vc[1] == 0.0) and np.all(np.isneginf(lse[1]))


def test_row_permutation_invariance():
    d, pool, table, L, q = _tiny_latent_case(L=(9,), paged=False)
    vc, lse, _ = O.attention_latent(d, q, pool, table, L, 0.8)
    rows = O.gather_rows(pool, table, 0, 9, d.block_size)
    perm = np.random.default_rng(9).permutation(9)
    pool2 = np.full_like(pool, np.nan)
    pool2.reshape(-1, pool.shape[-1])[:9] = rows[perm]
    vc2, lse2, _ = O.attention_latent(d, q, pool2, table, L, 0.8)
    assert np.allclose(vc, vc2, rtol=1e-13, atol=1e-15) and np.allclose(lse, lse2, rtol=1e-14)


def test_paged_equals_contiguous_exactly():
    d, pool, table, L, q = _tiny_latent_case(L=(13, 6, 1), block=4, paged=True)
    vc, lse, _ = O.attention_latent(d, q, pool, table, L, 0.6)
    # rebuild the same logical rows in an identity-mapped pool
    pool_c = np.concatenate([pool[table[b][:(int(L[b]) + 3) // 4]] for b in range(len(L))])
    starts = np.cumsum([0] + [(int(x) + 3) // 4 for x in L])
    table_c = np.full_like(table, -1)
    for b in range(len(L)):
        nb = starts[b + 1] - starts[b]
        table_c[b, :nb] = np.arange(starts[b], starts[b + 1])
    vc2, lse2, _ = O.attention_latent(d, q, pool_c, table_c, L, 0.6)
    assert np.array_equal(vc, vc2) and np.array_equal(lse, lse2)


def test_slot_formula_brute_force_walk():
    # walk the blocks of each sequence in order and count rows
    rng = np.random.default_rng(11)
    block, B = 4, 3
    lens = [7, 12, 1]
    nb = [(x + block - 1) // block for x in lens]
    perm = rng.permutation(sum(nb))
    table = np.full((B, max(nb)), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        table[b, :nb[b]] = perm[k:k + nb[b]]
        k += nb[b]
    for b in range(B):
        walk = []
        for j in range(nb[b]):
            for r in range(block):
                walk.append((int(table[b][j]), r))
        for pos in range(lens[b]):
            assert O.slot(table, b, pos, block) == walk[pos]


def test_absorbed_equals_unabsorbed_config1():
    case = S.make_case(1)
    res = O.decode_step(case, model_q_abs_storage=False)
    d = case.dims
    o1, lse1 = O.attention_unabsorbed(d, res["q"], res["kv_b64"], res["pool"], case.table,
                                      case.lens, res["softmax_scale"], res["inv_freq"],
                                      res["rope_mscale"], case.positions)
    o2 = O.out_proj(d, res["v_combine"], res["kv_b64"])
    assert np.allclose(o2, o1, rtol=1e-12, atol=1e-15)
    assert np.allclose(res["lse"], lse1, rtol=1e-12)


def test_absorbed_equals_unabsorbed_deepseek_shape_subsample():
    case = S.make_case(2, lens=[257, 64], batch=2)
    res = O.decode_step(case, model_q_abs_storage=False)
    heads = [0, 17, 127]
    o1, lse1 = O.attention_unabsorbed(case.dims, res["q"], res["kv_b64"], res["pool"],
                                      case.table, case.lens, res["softmax_scale"],
                                      res["inv_freq"], res["rope_mscale"], case.positions,
                                      heads=heads)
    o2 = O.out_proj(case.dims, res["v_combine"], res["kv_b64"])[:, heads]
    assert np.allclose(o2, o1, rtol=1e-11, atol=1e-14)
    assert np.allclose(res["lse"][:, heads], lse1, rtol=1e-12)


def test_unabsorbed_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    case = S.make_case(1, sharp=True)
    res = O.decode_step(case, model_q_abs_storage=False)
    d = case.dims
    H, N, V, C = d.num_heads, d.qk_nope, d.v_head, d.kv_lora
    o1, _ = O.attention_unabsorbed(d, res["q"], res["kv_b64"], res["pool"], case.table,
                                   case.lens, res["softmax_scale"], res["inv_freq"],
                                   res["rope_mscale"], case.positions)
    # decompress independently with torch and run the library's attention
    rows = torch.from_numpy(O.widen(O.gather_rows(res["pool"], case.table, 0, 128, 64), O.F32))
    kvb = torch.from_numpy(res["kv_b64"]).reshape(H, N + V, C)
    k_nope = torch.einsum("tc,hnc->htn", rows[:, :C], kvb[:, :N])
    k = torch.cat([k_nope, rows[None, :, C:].expand(H, -1, -1)], dim=2)
    v = torch.einsum("tc,hvc->htv", rows[:, :C], kvb[:, N:])
    q = torch.from_numpy(res["q"][0]).clone()
    q[:, N:] = torch.from_numpy(O.rope_consecutive(res["q"][0, :, N:], 127.0, res["inv_freq"],
                                                   res["rope_mscale"]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], k, v, scale=res["softmax_scale"])[:, 0, :]
    assert np.allclose(o1[0], ref.numpy(), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# whole step against a pure-Python brute force on tiny shapes
# ----------------------------------------------------------------------------
def _f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def test_whole_step_brute_force_tiny():
    H, N, R, V, C, hidden, block = 2, 2, 2, 3, 3, 4, 2
    W = C + R
    rng = np.random.default_rng(21)
    d = S.Dims(num_heads=H, qk_nope=N, qk_rope=R, v_head=V, kv_lora=C, hidden=hidden,
               block_size=block, cache_dtype=O.F32, rms_eps=1e-6)
    L = 3
    pos = L - 1
    prior = rng.standard_normal((L - 1, W)).astype(np.float32)
    pool = np.full((2, block, W), np.nan, dtype=np.float32)
    table = np.array([[1, 0]], dtype=np.int32)        # logical block 0 -> 1, 1 -> 0
    pool[1, 0], pool[1, 1] = prior[0], prior[1]
    x = rng.standard_normal(hidden).astype(np.float32)
    Wk = (rng.standard_normal((W, hidden)) * 0.5).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    q = rng.standard_normal((H, N + R)).astype(np.float32)
    kvb = (rng.standard_normal((H * (N + V), C)) * 0.5).astype(np.float32)
    Wo = (rng.standard_normal((5, H * V)) * 0.5).astype(np.float32)
    inv = [0.7]
    rm, scale = 1.1, 0.45

    # ---- brute force ----
    kv_pre = [sum(float(Wk[o][k]) * float(x[k]) for k in range(hidden)) for o in range(W)]
    ms = sum(v * v for v in kv_pre[:C]) / C
    c_new = [kv_pre[i] / math.sqrt(ms + d.rms_eps) * float(gamma[i]) for i in range(C)]
    a = pos * inv[0]
    k_new = [rm * (kv_pre[C] * math.cos(a) - kv_pre[C + 1] * math.sin(a)),
             rm * (kv_pre[C] * math.sin(a) + kv_pre[C + 1] * math.cos(a))]
    rows = [[float(v) for v in prior[0]], [float(v) for v in prior[1]],
            [_f32(v) for v in c_new + k_new]]
    outs = []
    for h in range(H):
        base = h * (N + V)
        qn = [float(v) for v in q[h][:N]]
        qr = [rm * (float(q[h][N]) * math.cos(a) - float(q[h][N + 1]) * math.sin(a)),
              rm * (float(q[h][N]) * math.sin(a) + float(q[h][N + 1]) * math.cos(a))]
        scores, vals = [], []
        for t in range(L):
            kn = [sum(float(kvb[base + n][c]) * rows[t][c] for c in range(C)) for n in range(N)]
            kk = kn + rows[t][C:]
            scores.append(scale * sum(qi * ki for qi, ki in zip(qn + qr, kk)))
            vals.append([sum(float(kvb[base + N + v][c]) * rows[t][c] for c in range(C))
                         for v in range(V)])
        mx = max(scores)
        e = [math.exp(s - mx) for s in scores]
        z = sum(e)
        outs += [sum(e[t] / z * vals[t][v] for t in range(L)) for v in range(V)]
    y = [sum(float(Wo[o][i]) * outs[i] for i in range(H * V)) for o in range(5)]

    # ---- oracle, composed from its step functions ----
    invf = np.array(inv)
    new_pool, _ = O.cache_append(d, x[None], Wk, O.F32, gamma, O.F32, invf, rm, [pos], pool,
                                 table)
    assert np.array_equal(new_pool[1], pool[1])                       # prior rows untouched
    assert np.allclose(new_pool[0, 0], rows[2], rtol=0, atol=0)        # slot (block 0, row 0)
    assert np.all(np.isnan(new_pool[0, 1]))
    kvb64 = O.widen(kvb, O.F32)
    q_abs = O.absorb_q(d, q[None].astype(np.float64), kvb64, invf, rm, [pos])
    vc, _, _ = O.attention_latent(d, q_abs, new_pool, table, [L], scale)
    y_or = O.out_proj(d, vc, kvb64, O.widen(Wo, O.F32))
    assert np.allclose(y_or[0], y, rtol=1e-12, atol=1e-14)
    o1, _ = O.attention_unabsorbed(d, q[None].astype(np.float64), kvb64, new_pool, table, [L],
                                   scale, invf, rm, [pos])
    assert np.allclose(o1.reshape(-1), outs, rtol=1e-12, atol=1e-14)


def test_q_chain_brute_force_tiny():
    H, N, R, hidden, ql = 1, 2, 2, 64, 64
    rng = np.random.default_rng(23)
    d = S.Dims(num_heads=H, qk_nope=N, qk_rope=R, v_head=1, kv_lora=4, hidden=hidden, q_lora=ql)
    qa = S.draw_q4(rng, ql, hidden)
    qb = S.draw_q4(rng, H * (N + R), ql)
    g = S.to_bf16_bits(1 + 0.1 * rng.standard_normal(ql))
    x = rng.standard_normal(hidden).astype(np.float32)

    def deq(w, r, k):
        word = int(w.packed[r][k // 8])
        nib = (word >> (4 * (k % 8))) & 15
        s = float(S.bf16_bits_to_f32(w.scales[r][k // 64:k // 64 + 1])[0])
        b = float(S.bf16_bits_to_f32(w.biases[r][k // 64:k // 64 + 1])[0])
        return s * nib + b

    lat = [sum(deq(qa, o, k) * float(x[k]) for k in range(hidden)) for o in range(ql)]
    ms = sum(v * v for v in lat) / ql
    gam = S.bf16_bits_to_f32(g).astype(np.float64)
    latn = [lat[i] / math.sqrt(ms + 1e-6) * gam[i] for i in range(ql)]
    want = [sum(deq(qb, o, k) * latn[k] for k in range(ql)) for o in range(H * (N + R))]
    got = O.q_chain(d, x[None], qa, g, qb)
    assert np.allclose(got.reshape(-1), want, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# several tokens per sequence (chunked prefill / multi-token decode)
# ----------------------------------------------------------------------------
def _token_subcase(case, idx, pool):
    """Tokens ``idx`` of a multi-token case as a case of their own, on ``pool``."""
    import copy
    sub = copy.copy(case)
    idx = np.asarray(idx)
    sub.batch = len(idx)
    sub.lens = case.lens[idx]
    sub.token_seq = case.token_seq[idx]
    sub.pool = pool
    for f in ("x", "q", "q_abs"):
        v = getattr(case, f)
        if v is not None:
            setattr(sub, f, np.asarray(v)[idx])
    return sub


@pytest.mark.parametrize("cfg,prior,chunk", [(1, [5, 70], [4, 3]), (2, [64, 3], [2, 5])])
def test_chunk_equals_token_by_token_decode(cfg, prior, chunk):
    """A step over several new tokens per sequence gives, token by token, what
    single-token decode steps give when run in position order: the causal
    reading (token at position p sees rows 0..p, all rows appended first)."""
    case = S.make_chunk_case(cfg, prior, chunk)
    res = O.decode_step(case)
    pool = case.pool
    for t in range(case.batch):
        r = O.decode_step(_token_subcase(case, [t], pool))
        pool = r["pool"]
        for key in ("v_combine", "lse", "out"):
            np.testing.assert_allclose(r[key][0], res[key][t], rtol=1e-12, atol=1e-14,
                                       err_msg=f"{key} token {t}")
    np.testing.assert_array_equal(O.widen(pool, case.dims.cache_dtype),
                                  O.widen(res["pool"], case.dims.cache_dtype))


def test_chunk_token_sees_only_its_prefix():
    """Each token's softmax spans exactly its position + 1 rows and sums to 1."""
    case = S.make_chunk_case(1, [6], [3])
    res = O.decode_step(case)
    assert [p.shape[1] for p in res["p"]] == [7, 8, 9]
    for p in res["p"]:
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)
