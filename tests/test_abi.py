"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, rejects bad arguments before touching the device, and its host YaRN
helper matches the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_latent_kv_11_amd as mla
from oracle import mla_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built; run __graft_entry__.build() first")
    return mla.load_library()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(mla_\w+)\s*\(", src, re.M)))


def test_header_declares_the_expected_calls():
    assert declared_functions() == sorted(mla.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert mla.status_str(code) and "unknown" not in mla.status_str(code)
    assert "unknown" in mla.status_str(-99)


DS = mla.Dims(128, 128, 64, 128, 512, hidden=0, q_lora=0, block_size=64, cache_dtype=mla.MLA_BF16)


def _w(dtype, rows, cols, ptr=0x1000, sc=None, bi=None):
    return mla.CWeight(dtype, rows, cols, ptr, sc, bi)


def call_attn(lib, dims=DS, B=2, q=0x1000, pool=0x2000, table=0x3000, lens=0x4000, max_len=100,
              scale=0.1, split=0, vc=0x5000, lse=None, ws=None, ws_bytes=0, nblocks=4, maxb=2):
    cache = mla.CCache(pool, table, nblocks, maxb)
    return lib.mla_decode_attn(ctypes.byref(dims.c()), B, q, ctypes.byref(cache), lens, max_len,
                               scale, split, vc, lse, ws, ws_bytes, None)


def test_attn_validation_before_launch(lib):
    # every one of these returns before any HIP call (no device here)
    assert call_attn(lib, q=None) == mla.MLA_ERR_NULL
    assert call_attn(lib, vc=None) == mla.MLA_ERR_NULL
    assert call_attn(lib, max_len=-1) == mla.MLA_ERR_DIMS
    assert call_attn(lib, max_len=129) == mla.MLA_ERR_CAPACITY          # 2 blocks x 64 rows
    assert call_attn(lib, split=100) == mla.MLA_ERR_DIMS                 # not a multiple of 64
    assert call_attn(lib, scale=float("inf")) == mla.MLA_ERR_DIMS
    bad = mla.Dims(**{**DS.__dict__, "num_heads": 64})
    assert call_attn(lib, dims=bad) == mla.MLA_ERR_UNSUPPORTED
    odd = mla.Dims(**{**DS.__dict__, "qk_rope": 63})
    assert call_attn(lib, dims=odd) == mla.MLA_ERR_DIMS
    dt = mla.Dims(**{**DS.__dict__, "cache_dtype": 7})
    assert call_attn(lib, dims=dt) == mla.MLA_ERR_DTYPE
    # two splits of 64 rows need a workspace
    assert call_attn(lib, split=64, max_len=128) == mla.MLA_ERR_WORKSPACE
    assert call_attn(lib, split=64, max_len=128, ws=0x9000, ws_bytes=16) == mla.MLA_ERR_WORKSPACE
    # batch 0 is a no-op success
    assert call_attn(lib, B=0) == mla.MLA_OK


def test_plan_and_workspace(lib):
    r, s = mla.attn_plan(DS, 4, 131072, 2048)
    assert (r, s) == (2048, 64)
    r, s = mla.attn_plan(DS, 1, 100, 0)   # automatic: splits of >= 128 rows covering the context
    assert r % 64 == 0 and r >= 128 and r * s >= 100 and r * (s - 1) < 100
    need = mla.workspace_bytes(DS, 4, 131072, 2048)
    # bf16 cache: fp16 split partials, plus an lse and an exponent per (seq, split, head)
    assert need >= 4 * 64 * 128 * 512 * 2 + 2 * (4 * 64 * 128 * 4)
    assert mla.workspace_bytes(DS, 1, 100, 64 * 3) >= 0
    with pytest.raises(mla.MLAError):
        mla.attn_plan(DS, 1, 100, 65)
    # the bf16 kernel's largest split is 32768 rows (1024 tiles); one more block is refused
    assert mla.attn_plan(DS, 1, 32768, 32768) == (32768, 1)
    assert mla.attn_plan(DS, 1, 131072, 32768) == (32768, 4)
    with pytest.raises(mla.MLAError):
        mla.attn_plan(DS, 1, 32768 + 64, 32768 + 64)


def test_plan_from_lengths(lib):
    # uniform batches get the automatic plan: one workgroup per compute unit (256 here)
    assert mla.attn_plan_lens(DS, [16384] * 32) == mla.attn_plan(DS, 32, 16384, 0) == (2048, 8)
    assert mla.attn_plan_lens(DS, [131072] * 4) == (2048, 64)
    assert mla.attn_plan_lens(DS, [4096]) == mla.attn_plan(DS, 1, 4096, 0) == (128, 32)
    # a ragged batch: the smallest split whose non-empty workgroups fit 256 compute units
    lens = np.random.default_rng(3).integers(1024, 8193, size=64)
    r, s = mla.attn_plan_lens(DS, lens)
    wgs = lambda r: int(np.sum((lens + r - 1) // r))
    assert r % 64 == 0 and r >= 128 and s == -(-int(lens.max()) // r)
    assert wgs(r) <= 256 < wgs(r - 64)
    assert r < mla.attn_plan(DS, 64, int(lens.max()), 0)[0]  # shorter than the max-length plan
    # more sequences than compute units: no split fits, so the automatic plan is kept
    assert mla.attn_plan_lens(DS, [1024] * 300) == mla.attn_plan(DS, 300, 1024, 0)
    # one long sequence among short ones: the long one takes most of the workgroups
    lens2 = np.array([131072] + [256] * 31)
    r2, s2 = mla.attn_plan_lens(DS, lens2)
    assert int(np.sum((lens2 + r2 - 1) // r2)) <= 256 and s2 == -(-131072 // r2)
    assert int(np.sum((lens2 + r2 - 65) // (r2 - 64))) > 256
    # empty sequences and an empty batch
    assert mla.attn_plan_lens(DS, [0, 0]) == mla.attn_plan(DS, 2, 0, 0)
    assert mla.attn_plan_lens(DS, []) == mla.attn_plan(DS, 0, 0, 0)
    with pytest.raises(mla.MLAError):
        mla.attn_plan_lens(DS, [5, -1])


def test_weight_validation(lib):
    d = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    cache = mla.CCache(0x200, 0x300, 2, 2)
    kv_a = _w(mla.MLA_F32, 80, 256)
    norm = _w(mla.MLA_F32, 1, 64)

    def app(kv_a=kv_a, norm=norm, ws=0x900, wsb=1 << 20, x=0x400):
        return lib.mla_cache_append(ctypes.byref(d.c()), 1, x, ctypes.byref(kv_a) if kv_a else None,
                                    ctypes.byref(norm), ctypes.byref(rope), 0x500,
                                    ctypes.byref(cache), None, ws, wsb, None)
    assert app(x=None) == mla.MLA_ERR_NULL
    assert app(kv_a=None) == mla.MLA_ERR_NULL                     # hidden > 0 needs kv_a
    assert app(kv_a=_w(mla.MLA_F32, 79, 256)) == mla.MLA_ERR_DIMS  # one row short
    assert app(kv_a=_w(5, 80, 256)) == mla.MLA_ERR_DTYPE
    assert app(norm=_w(mla.MLA_Q4G64, 1, 64)) == mla.MLA_ERR_DTYPE
    assert app(ws=None) == mla.MLA_ERR_WORKSPACE
    assert app(wsb=10) == mla.MLA_ERR_WORKSPACE
    # 4-bit weights need group-aligned columns and scale/bias pointers
    q4 = _w(mla.MLA_Q4G64, 80, 256)
    assert app(kv_a=q4) == mla.MLA_ERR_NULL
    d2 = mla.Dims(16, 32, 16, 32, 64, hidden=96, q_lora=0, cache_dtype=mla.MLA_F32)
    q4b = _w(mla.MLA_Q4G64, 80, 96, sc=0x10, bi=0x20)
    assert lib.mla_cache_append(ctypes.byref(d2.c()), 1, 0x400, ctypes.byref(q4b),
                                ctypes.byref(norm), ctypes.byref(rope), 0x500, ctypes.byref(cache),
                                None, 0x900, 1 << 20, None) == mla.MLA_ERR_DIMS


def test_absorb_and_out_proj_validation(lib):
    d = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    kvb = _w(mla.MLA_F32, 16 * 64, 64)
    assert lib.mla_absorb_q(ctypes.byref(d.c()), 1, 0x10, None, None, None, ctypes.byref(kvb),
                            ctypes.byref(rope), 0x20, None, None, 0, None) == mla.MLA_ERR_NULL
    short = _w(mla.MLA_F32, 16 * 64 - 1, 64)
    assert lib.mla_absorb_q(ctypes.byref(d.c()), 1, 0x10, None, None, None, ctypes.byref(short),
                            ctypes.byref(rope), 0x20, 0x30, None, 0, None) == mla.MLA_ERR_DIMS
    # q_a without q_lora in the dims
    qa = _w(mla.MLA_F32, 8, 256)
    assert lib.mla_absorb_q(ctypes.byref(d.c()), 1, 0x10, ctypes.byref(qa), None, None,
                            ctypes.byref(kvb), ctypes.byref(rope), 0x20, 0x30, None, 0,
                            None) == mla.MLA_ERR_DIMS
    wo = _w(mla.MLA_F32, 256, 16 * 32)
    assert lib.mla_out_proj(ctypes.byref(d.c()), 1, 0x10, ctypes.byref(kvb), ctypes.byref(wo),
                            0x20, None, 0, None) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_out_proj(ctypes.byref(d.c()), 1, None, ctypes.byref(kvb), None, 0x20, None, 0,
                            None) == mla.MLA_ERR_NULL


def test_q8_0_kv_b_validation(lib):
    # the pages' kv_b check: dtype, shape (H*(N+V), C), C tiling 32-value blocks,
    # packed size rows * C/32 * 34 -- heads 4, nope 2, kv_lora 64, v 1 as in
    # the pages' unit test
    ok = dict(dtype=mla.MLA_Q8_0, rows=12, cols=64, size_bytes=12 * 2 * 34, heads=4, nope=2,
              kv_lora=64, v_head=1)
    assert mla.validate_q8_0_kv_b(**ok) == mla.MLA_OK
    assert mla.validate_q8_0_kv_b(**{**ok, "dtype": 12}) == mla.MLA_ERR_DTYPE
    assert mla.validate_q8_0_kv_b(**{**ok, "dtype": mla.MLA_BF16}) == mla.MLA_ERR_DTYPE
    assert mla.validate_q8_0_kv_b(**{**ok, "rows": 11}) == mla.MLA_ERR_DIMS
    assert mla.validate_q8_0_kv_b(**{**ok, "cols": 32}) == mla.MLA_ERR_DIMS
    assert mla.validate_q8_0_kv_b(**{**ok, "size_bytes": 12 * 2 * 34 - 1}) == mla.MLA_ERR_DIMS
    assert mla.validate_q8_0_kv_b(**{**ok, "size_bytes": 12 * 2 * 34 + 1}) == mla.MLA_ERR_DIMS
    # a width that does not tile whole blocks
    assert mla.validate_q8_0_kv_b(**{**ok, "cols": 48, "kv_lora": 48,
                                     "size_bytes": 12 * 34}) == mla.MLA_ERR_DIMS
    assert mla.validate_q8_0_kv_b(**{**ok, "kv_lora": 0, "cols": 0,
                                     "size_bytes": 0}) == mla.MLA_ERR_DIMS
    # DeepSeek-V3 kv_b: 128 heads x (128 + 128) rows x 512
    assert mla.validate_q8_0_kv_b(mla.MLA_Q8_0, 32768, 512, 32768 * 16 * 34, 128, 128, 512,
                                  128) == mla.MLA_OK


def test_q8_0_accepted_for_kv_b_only(lib):
    d = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    kvb8 = _w(mla.MLA_Q8_0, 16 * 64, 64)
    # kv_b as Q8_0 passes the weight checks and stops at the missing workspace
    wo = _w(mla.MLA_F32, 256, 16 * 32)
    assert lib.mla_out_proj(ctypes.byref(d.c()), 1, 0x10, ctypes.byref(kvb8), ctypes.byref(wo),
                            0x20, None, 0, None) == mla.MLA_ERR_WORKSPACE
    # ... but not where its width does not tile 32-value blocks
    d48 = mla.Dims(16, 32, 16, 32, 48, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)
    assert lib.mla_out_proj(ctypes.byref(d48.c()), 1, 0x10,
                            ctypes.byref(_w(mla.MLA_Q8_0, 16 * 64, 48)), ctypes.byref(wo), 0x20,
                            None, 0, None) == mla.MLA_ERR_DIMS
    # o_proj, q_a, q_b and kv_a do not take Q8_0
    wo8 = _w(mla.MLA_Q8_0, 256, 16 * 32)
    kvb = _w(mla.MLA_F32, 16 * 64, 64)
    assert lib.mla_out_proj(ctypes.byref(d.c()), 1, 0x10, ctypes.byref(kvb), ctypes.byref(wo8),
                            0x20, None, 0, None) == mla.MLA_ERR_DTYPE
    dq = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=32, cache_dtype=mla.MLA_F32)
    qa8, qan = _w(mla.MLA_Q8_0, 32, 256), _w(mla.MLA_F32, 1, 32)
    qb = _w(mla.MLA_F32, 16 * 48, 32)
    assert lib.mla_absorb_q(ctypes.byref(dq.c()), 1, 0x10, ctypes.byref(qa8), ctypes.byref(qan),
                            ctypes.byref(qb), ctypes.byref(kvb), ctypes.byref(rope), 0x20, 0x30,
                            None, 0, None) == mla.MLA_ERR_DTYPE
    norm = _w(mla.MLA_F32, 1, 64)
    cache = mla.CCache(0x200, 0x300, 2, 2)
    assert lib.mla_cache_append(ctypes.byref(d.c()), 1, 0x400,
                                ctypes.byref(_w(mla.MLA_Q8_0, 80, 256)), ctypes.byref(norm),
                                ctypes.byref(rope), 0x500, ctypes.byref(cache), None, 0x900,
                                1 << 20, None) == mla.MLA_ERR_DTYPE


@pytest.mark.parametrize("R,head", [(64, 192), (16, 48)])
def test_library_yarn_table_matches_oracle(lib, R, head):
    inv, rm, sc = mla.yarn_tables(R, head)
    ref = O.yarn_inv_freq(R, 1e4, 40.0, 4096.0, 32.0, 1.0)
    assert np.array_equal(np.array(inv, dtype=np.float32), ref.astype(np.float32))
    orm, osc = O.yarn_scalars(40.0, 1.0, 1.0, head)
    assert rm == np.float32(orm) and sc == np.float32(osc)


def test_yarn_validation(lib):
    y = mla.CYarn(1e4, 40, 4096, 32, 1, 1, 1)
    assert lib.mla_yarn_tables(ctypes.byref(y), 63, 192, None, None, None) == mla.MLA_ERR_DIMS
    assert lib.mla_yarn_tables(None, 64, 192, None, None, None) == mla.MLA_ERR_NULL
    y0 = mla.CYarn(1.0, 40, 4096, 32, 1, 1, 1)
    assert lib.mla_yarn_tables(ctypes.byref(y0), 64, 192, None, None, None) == mla.MLA_ERR_DIMS


def test_token_calls_validation_before_launch(lib):
    """The several-tokens-per-sequence calls: a map is required, num_seqs must
    cover at least one sequence when there are tokens; the rest is checked as
    in the one-token calls.  All return before any HIP call."""
    cache = mla.CCache(0x2000, 0x3000, 4, 2)

    def attn(tseq=0x6000, nseq=2, n=3, max_len=100, q=0x1000):
        return lib.mla_attn_tokens(ctypes.byref(DS.c()), n, q, ctypes.byref(cache), tseq, nseq,
                                   0x4000, max_len, 0.1, 0, 0x5000, None, None, 0, None)
    assert attn(tseq=None) == mla.MLA_ERR_NULL
    assert attn(nseq=0) == mla.MLA_ERR_DIMS
    assert attn(q=None) == mla.MLA_ERR_NULL
    assert attn(max_len=129) == mla.MLA_ERR_CAPACITY
    assert attn(n=0, nseq=0) == mla.MLA_OK

    d = mla.Dims(16, 32, 16, 32, 64, hidden=0, q_lora=0, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    norm = _w(mla.MLA_F32, 1, 64)

    def app(tseq=0x600, nseq=2, n=3, x=0x400):
        return lib.mla_cache_append_tokens(ctypes.byref(d.c()), n, x, None, ctypes.byref(norm),
                                           ctypes.byref(rope), 0x500, tseq, nseq,
                                           ctypes.byref(cache), None, None, 0, None)
    assert app(tseq=None) == mla.MLA_ERR_NULL
    assert app(nseq=-1) == mla.MLA_ERR_DIMS
    assert app(x=None) == mla.MLA_ERR_NULL
    assert app(n=0, nseq=0) == mla.MLA_OK


def test_one_hip_runtime_in_the_process():
    """Loading the library (even before torch is imported) leaves a single
    HIP runtime mapped: torch's, which owns the memory and streams passed in."""
    import re
    import subprocess
    import sys
    code = ("import mla_latent_kv_11_amd as m; m.load_library(); import torch, re; "
            "maps = open('/proc/self/maps').read(); "
            "print(len(set(re.findall(r'/\\S*libamdhip64\\S*', maps))))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_layer_validation_before_launch(lib):
    """mla_decode_layer checks the arguments of all four steps before it
    enqueues anything: an error in the last step (out_proj) is reported as
    that step reports it, with no launch (there is no device here)."""
    d = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=0, block_size=64, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    kva, norm = _w(mla.MLA_F32, 80, 256), _w(mla.MLA_F32, 1, 64)
    kvb, wo = _w(mla.MLA_F32, 16 * 64, 64), _w(mla.MLA_F32, 256, 16 * 32)
    cache = mla.CCache(0x2000, 0x3000, 4, 2)
    null = ctypes.POINTER(mla.CWeight)()

    def layer(o_proj=wo, kv_b=kvb, q_in=0x700, ws=0x9000, ws_bytes=None, B=2, x=0x600):
        L = mla.CLayer(ctypes.pointer(kva), ctypes.pointer(norm), null, null, null,
                       ctypes.pointer(kv_b) if kv_b is not None else null,
                       ctypes.pointer(o_proj) if o_proj is not None else null,
                       ctypes.pointer(rope))
        need = lib.mla_layer_workspace_bytes(ctypes.byref(d.c()), B, 100, 0)
        return lib.mla_decode_layer(ctypes.byref(d.c()), B, x, q_in, ctypes.byref(L), 0x800,
                                    ctypes.byref(cache), 0x4000, 100, 0.1, 0, 0xa000, 0x5000,
                                    None, 0xb000, None, ws, need if ws_bytes is None else ws_bytes,
                                    None)
    assert lib.mla_decode_layer(ctypes.byref(d.c()), 2, 0x600, 0x700, None, 0x800,
                                ctypes.byref(cache), 0x4000, 100, 0.1, 0, 0xa000, 0x5000, None,
                                0xb000, None, 0x9000, 1 << 20, None) == mla.MLA_ERR_NULL
    assert layer(kv_b=None) == mla.MLA_ERR_NULL
    assert layer(q_in=None) == mla.MLA_ERR_NULL          # no q_a: the query is given
    assert layer(x=None) == mla.MLA_ERR_NULL
    assert layer(o_proj=_w(mla.MLA_F32, 256, 16 * 32 + 1)) == mla.MLA_ERR_DIMS
    assert layer(ws_bytes=64) == mla.MLA_ERR_WORKSPACE
    assert layer(ws=None) == mla.MLA_ERR_WORKSPACE
    assert layer(B=0) == mla.MLA_OK
    # the layer's workspace holds every call's regions side by side
    for B, L in ((1, 128), (32, 16384)):
        assert (lib.mla_layer_workspace_bytes(ctypes.byref(d.c()), B, L, 0)
                >= lib.mla_workspace_bytes(ctypes.byref(d.c()), B, L, 0))


def test_tiled_4bit_validation(lib):
    # mla_repack_q4g64 checks before any launch
    src = _w(mla.MLA_Q4G64, 64, 256, sc=0x10, bi=0x20)

    def repack(w=src, data=0x100, sc=0x200, bi=0x300):
        return lib.mla_repack_q4g64(ctypes.byref(w) if w else None, data, sc, bi, None)
    assert repack(w=None) == mla.MLA_ERR_NULL
    assert repack(data=None) == mla.MLA_ERR_NULL
    assert repack(bi=None) == mla.MLA_ERR_NULL
    assert repack(w=_w(mla.MLA_Q4G64, 64, 256)) == mla.MLA_ERR_NULL      # no scales
    assert repack(w=_w(mla.MLA_BF16, 64, 256, sc=0x10, bi=0x20)) == mla.MLA_ERR_DTYPE
    assert repack(w=_w(mla.MLA_Q4G64_T, 64, 256, sc=0x10, bi=0x20)) == mla.MLA_ERR_DTYPE
    assert repack(w=_w(mla.MLA_Q4G64, 48, 256, sc=0x10, bi=0x20)) == mla.MLA_ERR_DIMS   # rows
    assert repack(w=_w(mla.MLA_Q4G64, 64, 192, sc=0x10, bi=0x20)) == mla.MLA_ERR_DIMS   # cols
    # a tiled weight is taken where the 4-bit one is, with its own shape rules
    d = mla.Dims(16, 32, 16, 32, 64, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)
    rope = mla.CRope(0x100, 1.0)
    cache = mla.CCache(0x200, 0x300, 2, 2)
    norm = _w(mla.MLA_F32, 1, 64)

    def app(dims, kv_a):
        return lib.mla_cache_append(ctypes.byref(dims.c()), 1, 0x400, ctypes.byref(kv_a),
                                    ctypes.byref(norm), ctypes.byref(rope), 0x500,
                                    ctypes.byref(cache), None, 0x900, 1 << 20, None)
    d3 = mla.Dims(16, 32, 32, 32, 64, hidden=256, q_lora=0, cache_dtype=mla.MLA_F32)  # W = 96
    assert app(d3, _w(mla.MLA_Q4G64_T, 96, 256)) == mla.MLA_ERR_NULL       # no scales
    assert app(d, _w(mla.MLA_Q4G64_T, 80, 256, sc=0x10, bi=0x20)) == mla.MLA_ERR_DIMS  # 80 rows
    d4 = mla.Dims(16, 32, 32, 32, 64, hidden=192, q_lora=0, cache_dtype=mla.MLA_F32)
    assert app(d4, _w(mla.MLA_Q4G64_T, 96, 192, sc=0x10, bi=0x20)) == mla.MLA_ERR_DIMS  # 192 cols
    assert app(d, _w(mla.MLA_Q4G64_T, 1, 64, sc=0x10, bi=0x20)) == mla.MLA_ERR_DIMS
