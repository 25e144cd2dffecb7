"""CPU test that the oracle's pins can see mistakes (no GPU).

Each case below plants one plausible mistake in the oracle, in memory (a
mutated copy of one function, patched into ``oracle.mla_oracle`` for the
test's duration), and runs the pins of ``tests/test_oracle_pins.py``: at least
one pin must fail with an assertion.  The mutations are the kinds of slips the
pins exist to catch: a rotation sign or pairing, a dropped term or factor, a
swapped operand, an off-by-one row or column, a floor for a ceiling, a
rounding mode, a nibble order.  All keep the shapes, so a pin fails on values,
not on a crash.
"""
import inspect
import math

import numpy as np
import pytest

from oracle import mla_oracle as O

import test_oracle_pins as P

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _pins():
    out = []
    for name, fn in sorted(vars(P).items()):
        if name.startswith("test_") and callable(fn) and not inspect.signature(fn).parameters:
            out.append((name, fn))
    for args in ((1, [5, 70], [4, 3]), (2, [64, 3], [2, 5])):
        out.append(("test_chunk_equals_token_by_token_decode",
                    lambda a=args: P.test_chunk_equals_token_by_token_decode(*a)))
    return out


# ---- mutated copies -------------------------------------------------------
def _rope(sign=1.0, pairing="consecutive", use_mscale=True, pos_shift=0.0):
    def rope(x, pos, inv_freq, mscale=1.0):
        x = np.asarray(x, dtype=np.float64)
        ang = (np.asarray(pos, dtype=np.float64)[..., None] + pos_shift) * np.asarray(inv_freq)
        c, s = np.cos(ang), sign * np.sin(ang)
        ms = mscale if use_mscale else 1.0
        h = x.shape[-1] // 2
        if pairing == "consecutive":
            ia, ib = np.s_[..., 0::2], np.s_[..., 1::2]
        else:  # the two halves paired instead of neighbours
            ia, ib = np.s_[..., :h], np.s_[..., h:]
        a, b = x[ia], x[ib]
        out = np.empty_like(x)
        out[ia] = ms * (a * c - b * s)
        out[ib] = ms * (a * s + b * c)
        return out
    return rope


def _rmsnorm(kind):
    def rmsnorm(x, gamma, eps):
        x = np.asarray(x, dtype=np.float64)
        g = np.asarray(gamma, dtype=np.float64)
        if kind == "abs":
            ms = np.mean(np.abs(x), axis=-1, keepdims=True)
        elif kind == "sum":
            ms = np.sum(x * x, axis=-1, keepdims=True)
        else:
            ms = np.mean(x * x, axis=-1, keepdims=True)
        y = x / np.sqrt(ms + eps)
        return y if kind == "no_gamma" else y * g
    return rmsnorm


def _dequant_q4(kind):
    def dequant_q4(packed, scales, biases, rows, cols, group=64):
        packed = np.asarray(packed, dtype=np.uint32).reshape(rows, cols // 8)
        order = np.arange(8, dtype=np.uint32)
        if kind == "high_nibble_first":
            order = order[::-1].copy()
        q = ((packed[:, :, None] >> (4 * order)[None, None, :]) & np.uint32(15)).reshape(rows, cols)
        s = np.repeat(O.widen(scales, O.BF16).reshape(rows, -1), group, axis=1)
        b = np.repeat(O.widen(biases, O.BF16).reshape(rows, -1), group, axis=1)
        if kind == "scale_bias_swapped":
            s, b = b, s
        q = q.astype(np.float64)
        return q * s - b if kind == "bias_subtracted" else q * s + b
    return dequant_q4


def _correction_range_swapped(R, theta, orig_max_pos, beta_fast, beta_slow):
    def d(r):
        return R * math.log(orig_max_pos / (r * 2.0 * math.pi)) / (2.0 * math.log(theta))
    return max(math.ceil(d(beta_fast)), 0), min(math.floor(d(beta_slow)), R - 1)


def _inv_freq_ramp_reversed(R, theta, factor, orig_max_pos, beta_fast, beta_slow):
    i = np.arange(R // 2, dtype=np.float64)
    extra = theta ** (-2.0 * i / R)
    low, high = O.yarn_correction_range(R, theta, orig_max_pos, beta_fast, beta_slow)
    if low == high:
        high += 0.001
    ramp = np.clip((i - low) / (high - low), 0.0, 1.0)
    return extra * ramp + extra / factor * (1.0 - ramp)


def _scalars_without_temperature(factor, mscale, mscale_all_dim, qk_head_dim):
    m, m_all = O.yarn_get_mscale(factor, mscale), O.yarn_get_mscale(factor, mscale_all_dim)
    return m / m_all, 1.0 / math.sqrt(qk_head_dim)


def _get_mscale_without_tenth(scale, mscale=1.0):
    return 1.0 if scale <= 1.0 else mscale * math.log(scale) + 1.0


def _attention(kind):
    def attention_latent(dims, q_abs64, pool, table, lens, scale, token_seq=None):
        C, blk = dims.kv_lora, dims.block_size
        B, H = q_abs64.shape[0], q_abs64.shape[1]
        vc, lse, ps = np.zeros((B, H, C)), np.full((B, H), -np.inf), []
        for b in range(B):
            L = int(lens[b]) - (1 if kind == "last_row_dropped" and int(lens[b]) > 1 else 0)
            if L == 0:
                ps.append(np.zeros((H, 0)))
                continue
            seq = b if token_seq is None else int(token_seq[b])
            rows = O.widen(O.gather_rows(pool, table, seq, L, blk), dims.cache_dtype)
            keys = rows[:, :C] if kind == "latent_only_scores" else rows
            q = q_abs64[b][:, :C] if kind == "latent_only_scores" else q_abs64[b]
            s = (1.0 if kind == "no_scale" else scale) * (q @ keys.T)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            vals = rows[:, 1:C + 1] if kind == "value_columns_shifted" else rows[:, :C]
            vc[b] = p @ vals
            lse[b] = (m + np.log(z))[:, 0]
            ps.append(p)
        return vc, lse, ps
    return attention_latent


def _slot_table_ignored(table, b, pos, block):
    return pos // block, pos % block


def _kv_b_split_swapped(kv_b64, H, N, V):
    w = kv_b64.reshape(H, N + V, -1)
    return w[:, V:, :], w[:, :V, :]


def _round_bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _absorb_q_without_rope(dims, q, kv_b64, inv_freq, rope_mscale, positions):
    H, N, V = dims.num_heads, dims.qk_nope, dims.v_head
    q = np.asarray(q, dtype=np.float64)
    W_UK, _ = O.kv_b_split(kv_b64, H, N, V)
    return np.concatenate([np.einsum("bhn,hnc->bhc", q[:, :, :N], W_UK), q[:, :, N:]], axis=2)


def _out_proj_with_w_uk(dims, v_combine64, kv_b64, o_proj64=None):
    H, N, V = dims.num_heads, dims.qk_nope, dims.v_head
    W_UK, _ = O.kv_b_split(kv_b64, H, N, V)
    out = np.einsum("hvc,bhc->bhv", W_UK, np.asarray(v_combine64, dtype=np.float64))
    return out if o_proj64 is None else O.matvec(o_proj64, out.reshape(out.shape[0], -1))


def _q_chain_norm_after_q_b(dims, x, q_a, q_a_norm, q_b):
    H, N, R = dims.num_heads, dims.qk_nope, dims.qk_rope
    Wa = O.weight_f64(q_a, O.Q4G64, dims.q_lora, dims.hidden)
    Wb = O.weight_f64(q_b, O.Q4G64, H * (N + R), dims.q_lora)
    g = O.widen(q_a_norm, O.BF16)
    y = O.matvec(Wb, O.matvec(Wa, x) * g)
    return (y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + dims.rms_eps)).reshape(-1, H, N + R)


def _cache_append_norm_whole_row(dims, x, kv_a, kv_a_dtype, kv_a_norm, norm_dtype, inv_freq,
                                 rope_mscale, positions, pool, table, token_seq=None):
    C, W, blk = dims.kv_lora, dims.width, dims.block_size
    x64 = np.asarray(x, dtype=np.float64).reshape(len(positions), -1)
    kv_pre = O.matvec(O.weight_f64(kv_a, kv_a_dtype, W, dims.hidden), x64) if dims.hidden else x64
    ms = np.mean(kv_pre * kv_pre, axis=-1, keepdims=True)  # over latent and rope parts
    c = kv_pre[:, :C] / np.sqrt(ms + dims.rms_eps) * O.widen(kv_a_norm, norm_dtype)
    k_pe = O.rope_consecutive(kv_pre[:, C:], np.asarray(positions), inv_freq, rope_mscale)
    rows = np.concatenate([c, k_pe], axis=1)
    out = np.array(pool, copy=True)
    stored = O.round_to(rows, dims.cache_dtype)
    for b, pos in enumerate(positions):
        seq = b if token_seq is None else int(token_seq[b])
        pb, r = O.slot(table, seq, int(pos), blk)
        out[pb, r] = stored[b]
    return out, rows


MUTATIONS = {
    "rope: rotation sign": ("rope_consecutive", _rope(sign=-1.0)),
    "rope: halves paired instead of neighbours": ("rope_consecutive", _rope(pairing="halves")),
    "rope: mscale dropped": ("rope_consecutive", _rope(use_mscale=False)),
    "rope: position off by one": ("rope_consecutive", _rope(pos_shift=1.0)),
    "rmsnorm: mean |x| for mean x^2": ("rmsnorm", _rmsnorm("abs")),
    "rmsnorm: sum for mean": ("rmsnorm", _rmsnorm("sum")),
    "rmsnorm: gamma dropped": ("rmsnorm", _rmsnorm("no_gamma")),
    "4-bit: high nibble first": ("dequant_q4", _dequant_q4("high_nibble_first")),
    "4-bit: scale and bias swapped": ("dequant_q4", _dequant_q4("scale_bias_swapped")),
    "4-bit: bias subtracted": ("dequant_q4", _dequant_q4("bias_subtracted")),
    "yarn: floor and ceil swapped": ("yarn_correction_range", _correction_range_swapped),
    "yarn: ramp reversed": ("yarn_inv_freq", _inv_freq_ramp_reversed),
    "yarn: scale without the temperature": ("yarn_scalars", _scalars_without_temperature),
    "yarn: 0.1 factor dropped": ("yarn_get_mscale", _get_mscale_without_tenth),
    "attention: scale dropped": ("attention_latent", _attention("no_scale")),
    "attention: scores from the latent part only": ("attention_latent", _attention("latent_only_scores")),
    "attention: last row dropped": ("attention_latent", _attention("last_row_dropped")),
    "attention: value columns shifted by one": ("attention_latent", _attention("value_columns_shifted")),
    "paging: logical block taken as physical": ("slot", _slot_table_ignored),
    "kv_b: W_UK and W_UV swapped": ("kv_b_split", _kv_b_split_swapped),
    "bf16: truncation for round to nearest even": ("round_bf16", _round_bf16_truncate),
    "absorb: q_pe not rotated": ("absorb_q", _absorb_q_without_rope),
    "out_proj: W_UK for W_UV": ("out_proj", _out_proj_with_w_uk),
    "q chain: norm after q_b": ("q_chain", _q_chain_norm_after_q_b),
    "append: norm over the whole row": ("cache_append", _cache_append_norm_whole_row),
}

PINS = _pins()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_the_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    assert attr in _orig, attr
    monkeypatch.setattr(O, attr, fn)
    for pin_name, pin in PINS:
        try:
            pin()
        except AssertionError:
            return  # a pin sees the mistake
        except pytest.skip.Exception:
            continue
    pytest.fail(f"no pin fails with the oracle mutated: {name}")


def test_pins_pass_on_the_oracle():
    for pin_name, pin in PINS:
        pin()
