"""Python binding of the MLA latent-KV decode library (``include/mla.h``).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libmla.so``.  PyTorch supplies device memory and the current
stream; the functions take torch tensors (any dtype with the right byte
layout: bf16 may be ``torch.bfloat16`` or 16-bit integer bit patterns) and pass
their device pointers through the C ABI.

Loading fails loudly when the library has not been built (there is no
fallback).  Build it with ``python -m mla_latent_kv_11_amd.build`` or
``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

# ---- constants mirrored from mla.h ----
MLA_OK = 0
MLA_ERR_NULL, MLA_ERR_DIMS, MLA_ERR_DTYPE, MLA_ERR_UNSUPPORTED = -1, -2, -3, -4
MLA_ERR_CAPACITY, MLA_ERR_WORKSPACE, MLA_ERR_HIP = -5, -6, -7
MLA_F32, MLA_BF16, MLA_Q4G64, MLA_Q8_0, MLA_Q4G64_T = 0, 1, 2, 3, 4
MLA_DEV_POS_RANGE, MLA_DEV_BAD_BLOCK, MLA_DEV_BAD_SEQ = 1, 2, 4

EXPORTED = ("mla_yarn_tables", "mla_cache_append", "mla_absorb_q", "mla_decode_attn",
            "mla_out_proj", "mla_cache_append_tokens", "mla_attn_tokens",
            "mla_validate_q8_0_kv_b", "mla_workspace_bytes", "mla_attn_plan",
            "mla_attn_plan_lens", "mla_status_str", "mla_decode_attn_noalloc",
            "mla_decode_layer", "mla_layer_workspace_bytes", "mla_repack_q4g64")
MLA_NOALLOC_SCRATCH_BYTES = 48 << 20


class MLAError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class CDims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("qk_nope", ctypes.c_int32),
                ("qk_rope", ctypes.c_int32), ("v_head", ctypes.c_int32),
                ("kv_lora", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("q_lora", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float)]


class CWeight(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p)]


class CRope(ctypes.Structure):
    _fields_ = [("inv_freq", ctypes.c_void_p), ("mscale", ctypes.c_float)]


class CCache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32)]


class CLayer(ctypes.Structure):
    _fields_ = [("kv_a", ctypes.POINTER(CWeight)), ("kv_a_norm", ctypes.POINTER(CWeight)),
                ("q_a", ctypes.POINTER(CWeight)), ("q_a_norm", ctypes.POINTER(CWeight)),
                ("q_b", ctypes.POINTER(CWeight)), ("kv_b", ctypes.POINTER(CWeight)),
                ("o_proj", ctypes.POINTER(CWeight)), ("rope", ctypes.POINTER(CRope))]


class CYarn(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("factor", ctypes.c_double),
                ("original_max_pos", ctypes.c_double), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("mscale", ctypes.c_double),
                ("mscale_all_dim", ctypes.c_double)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so once and declare the exported signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"MLA HIP library not built ({path} missing); "
                           "run `python -m mla_latent_kv_11_amd.build`")
    # torch brings its own HIP runtime (same soname as the system one).  Load
    # it first so that the library binds to that runtime: loaded the other way
    # round, the process holds two HIP runtimes, and kernels launched by one on
    # the other's streams and memory fail.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PD, PW = ctypes.POINTER(CDims), ctypes.POINTER(CWeight)
    PR, PC = ctypes.POINTER(CRope), ctypes.POINTER(CCache)
    PF = ctypes.POINTER(ctypes.c_float)
    sig = {
        "mla_yarn_tables": ([ctypes.POINTER(CYarn), I32, I32, PF, PF, PF], ctypes.c_int),
        "mla_cache_append": ([PD, I32, P, PW, PW, PR, P, PC, P, P, SZ, P], ctypes.c_int),
        "mla_absorb_q": ([PD, I32, P, PW, PW, PW, PW, PR, P, P, P, SZ, P], ctypes.c_int),
        "mla_decode_attn": ([PD, I32, P, PC, P, I32, ctypes.c_float, I32, P, P, P, SZ, P],
                            ctypes.c_int),
        "mla_out_proj": ([PD, I32, P, PW, PW, P, P, SZ, P], ctypes.c_int),
        "mla_decode_attn_noalloc": ([PD, I32, P, PC, P, I32, ctypes.c_float, I32, P, P, P],
                                    ctypes.c_int),
        "mla_cache_append_tokens": ([PD, I32, P, PW, PW, PR, P, P, I32, PC, P, P, SZ, P],
                                    ctypes.c_int),
        "mla_attn_tokens": ([PD, I32, P, PC, P, I32, P, I32, ctypes.c_float, I32, P, P, P, SZ,
                             P], ctypes.c_int),
        "mla_validate_q8_0_kv_b": ([I32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, I32, I32,
                                    I32, I32], ctypes.c_int),
        "mla_workspace_bytes": ([PD, I32, I32, I32], SZ),
        "mla_attn_plan": ([PD, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)],
                          ctypes.c_int),
        "mla_attn_plan_lens": ([PD, I32, P, ctypes.POINTER(I32), ctypes.POINTER(I32)],
                               ctypes.c_int),
        "mla_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "mla_decode_layer": ([PD, I32, P, P, ctypes.POINTER(CLayer), P, PC, P, I32,
                              ctypes.c_float, I32, P, P, P, P, P, P, SZ, P], ctypes.c_int),
        "mla_layer_workspace_bytes": ([PD, I32, I32, I32], SZ),
        "mla_repack_q4g64": ([PW, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().mla_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != MLA_OK:
        raise MLAError(what, status)


# ----------------------------------------------------------------------------
# argument objects
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Dims:
    num_heads: int
    qk_nope: int
    qk_rope: int
    v_head: int
    kv_lora: int
    hidden: int = 0
    q_lora: int = 0
    block_size: int = 64
    cache_dtype: int = MLA_BF16
    rms_eps: float = 1e-6

    @property
    def width(self) -> int:
        return self.kv_lora + self.qk_rope

    def c(self) -> CDims:
        return CDims(self.num_heads, self.qk_nope, self.qk_rope, self.v_head, self.kv_lora,
                     self.hidden, self.q_lora, self.block_size, self.cache_dtype,
                     float(self.rms_eps))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


@dataclasses.dataclass
class Weight:
    """A weight matrix [rows, cols] on the device (see mla_weight in mla.h)."""
    dtype: int
    rows: int
    cols: int
    data: object
    scales: object = None
    biases: object = None

    def c(self) -> CWeight:
        return CWeight(self.dtype, self.rows, self.cols, _ptr(self.data), _ptr(self.scales),
                       _ptr(self.biases))


def repack_q4g64(w: Weight, stream=None) -> Weight:
    """The MLA_Q4G64 weight ``w`` repacked as MLA_Q4G64_T (mla_repack_q4g64):
    the same values in the layout the 4-bit MFMA products read in whole lines.
    The new buffers are torch tensors on ``w``'s device."""
    import torch
    if w.dtype != MLA_Q4G64:
        raise MLAError("mla_repack_q4g64", MLA_ERR_DTYPE)
    dev = w.data.device
    data = torch.empty(w.rows * w.cols // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(w.rows * w.cols // 64, dtype=torch.int16, device=dev)
    biases = torch.empty_like(scales)
    _check(load_library().mla_repack_q4g64(ctypes.byref(w.c()), _ptr(data), _ptr(scales),
                                           _ptr(biases), _stream(stream)), "mla_repack_q4g64")
    return Weight(MLA_Q4G64_T, w.rows, w.cols, data, scales, biases)


def _c_or_null(obj, ctype):
    return ctypes.byref(obj.c()) if obj is not None else ctypes.cast(None, ctypes.POINTER(ctype))


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _cache(pool, table) -> CCache:
    return CCache(_ptr(pool), _ptr(table), int(pool.shape[0]), int(table.shape[1]))


# ----------------------------------------------------------------------------
# the calls
# ----------------------------------------------------------------------------
def yarn_tables(rope_dim: int, qk_head_dim: int, theta=10000.0, factor=40.0,
                original_max_pos=4096.0, beta_fast=32.0, beta_slow=1.0, mscale=1.0,
                mscale_all_dim=1.0):
    """(inv_freq list [R/2], rope_mscale, softmax_scale) from the library's host helper."""
    lib = load_library()
    y = CYarn(theta, factor, original_max_pos, beta_fast, beta_slow, mscale, mscale_all_dim)
    inv = (ctypes.c_float * (rope_dim // 2))()
    rm, sc = ctypes.c_float(), ctypes.c_float()
    _check(lib.mla_yarn_tables(ctypes.byref(y), rope_dim, qk_head_dim, inv, ctypes.byref(rm),
                               ctypes.byref(sc)), "mla_yarn_tables")
    return list(inv), rm.value, sc.value


def workspace_bytes(dims: Dims, batch: int, max_seq_len: int, split_rows: int = 0) -> int:
    return int(load_library().mla_workspace_bytes(ctypes.byref(dims.c()), batch, max_seq_len,
                                                  split_rows))


def validate_q8_0_kv_b(dtype: int, rows: int, cols: int, size_bytes: int, heads: int, nope: int,
                       kv_lora: int, v_head: int) -> int:
    """Status of the host-side Q8_0 kv_b check (MLA_OK when the tensor is usable)."""
    return int(load_library().mla_validate_q8_0_kv_b(dtype, rows, cols, size_bytes, heads, nope,
                                                     kv_lora, v_head))


def attn_plan(dims: Dims, batch: int, max_seq_len: int, split_rows: int = 0):
    """(rows per split, splits per sequence) that mla_decode_attn would use."""
    r, s = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().mla_attn_plan(ctypes.byref(dims.c()), batch, max_seq_len, split_rows,
                                        ctypes.byref(r), ctypes.byref(s)), "mla_attn_plan")
    return r.value, s.value


def attn_plan_lens(dims: Dims, lens) -> tuple:
    """(rows per split, splits per sequence) sized from host-side lengths: the
    smallest split whose non-empty workgroups fit one per compute unit."""
    import numpy as _np
    arr = _np.ascontiguousarray(_np.asarray(lens, dtype=_np.int32))
    r, s = ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().mla_attn_plan_lens(ctypes.byref(dims.c()), int(arr.shape[0]),
                                             arr.ctypes.data_as(ctypes.c_void_p),
                                             ctypes.byref(r), ctypes.byref(s)),
           "mla_attn_plan_lens")
    return r.value, s.value


def cache_append(dims: Dims, x, kv_a: Optional[Weight], kv_a_norm: Weight, inv_freq,
                 rope_mscale: float, positions, pool, table, dev_status=None, ws=None,
                 stream=None) -> None:
    lib = load_library()
    rope = CRope(_ptr(inv_freq), float(rope_mscale))
    cache = _cache(pool, table)
    B = int(positions.shape[0])
    st = lib.mla_cache_append(ctypes.byref(dims.c()), B, _ptr(x), _c_or_null(kv_a, CWeight),
                              ctypes.byref(kv_a_norm.c()), ctypes.byref(rope), _ptr(positions),
                              ctypes.byref(cache), _ptr(dev_status), _ptr(ws),
                              ws.numel() * ws.element_size() if ws is not None else 0,
                              _stream(stream))
    _check(st, "mla_cache_append")


def absorb_q(dims: Dims, q_in, kv_b: Weight, inv_freq, rope_mscale: float, positions, q_abs,
             q_a: Optional[Weight] = None, q_a_norm: Optional[Weight] = None,
             q_b: Optional[Weight] = None, ws=None, stream=None) -> None:
    lib = load_library()
    rope = CRope(_ptr(inv_freq), float(rope_mscale))
    B = int(positions.shape[0])
    st = lib.mla_absorb_q(ctypes.byref(dims.c()), B, _ptr(q_in), _c_or_null(q_a, CWeight),
                          _c_or_null(q_a_norm, CWeight), _c_or_null(q_b, CWeight),
                          ctypes.byref(kv_b.c()), ctypes.byref(rope), _ptr(positions),
                          _ptr(q_abs), _ptr(ws),
                          ws.numel() * ws.element_size() if ws is not None else 0,
                          _stream(stream))
    _check(st, "mla_absorb_q")


def decode_attn(dims: Dims, q_abs, pool, table, seq_lens, max_seq_len: int,
                softmax_scale: float, v_combine, lse=None, split_rows: int = 0, ws=None,
                stream=None) -> None:
    lib = load_library()
    cache = _cache(pool, table)
    B = int(seq_lens.shape[0])
    st = lib.mla_decode_attn(ctypes.byref(dims.c()), B, _ptr(q_abs), ctypes.byref(cache),
                             _ptr(seq_lens), int(max_seq_len), float(softmax_scale),
                             int(split_rows), _ptr(v_combine), _ptr(lse), _ptr(ws),
                             ws.numel() * ws.element_size() if ws is not None else 0,
                             _stream(stream))
    _check(st, "mla_decode_attn")


def decode_attn_noalloc(dims: Dims, q_abs, pool, table, seq_lens, max_seq_len: int,
                        softmax_scale: float, v_combine, lse=None, split_rows: int = 0,
                        stream=None) -> None:
    """decode_attn with the split partials in the library's static device
    scratch (no workspace; calls overlapping on one device race)."""
    lib = load_library()
    cache = _cache(pool, table)
    B = int(seq_lens.shape[0])
    st = lib.mla_decode_attn_noalloc(ctypes.byref(dims.c()), B, _ptr(q_abs), ctypes.byref(cache),
                                     _ptr(seq_lens), int(max_seq_len), float(softmax_scale),
                                     int(split_rows), _ptr(v_combine), _ptr(lse),
                                     _stream(stream))
    _check(st, "mla_decode_attn_noalloc")


def cache_append_tokens(dims: Dims, x, kv_a: Optional[Weight], kv_a_norm: Weight, inv_freq,
                        rope_mscale: float, positions, token_seq, pool, table, dev_status=None,
                        ws=None, stream=None) -> None:
    """``cache_append`` for tokens that may share sequences: token t writes
    position ``positions[t]`` of table row ``token_seq[t]``."""
    lib = load_library()
    rope = CRope(_ptr(inv_freq), float(rope_mscale))
    cache = _cache(pool, table)
    n = int(positions.shape[0])
    st = lib.mla_cache_append_tokens(ctypes.byref(dims.c()), n, _ptr(x),
                                     _c_or_null(kv_a, CWeight), ctypes.byref(kv_a_norm.c()),
                                     ctypes.byref(rope), _ptr(positions), _ptr(token_seq),
                                     int(table.shape[0]), ctypes.byref(cache), _ptr(dev_status),
                                     _ptr(ws),
                                     ws.numel() * ws.element_size() if ws is not None else 0,
                                     _stream(stream))
    _check(st, "mla_cache_append_tokens")


def attn_tokens(dims: Dims, q_abs, pool, table, token_seq, seq_lens, max_seq_len: int,
                softmax_scale: float, v_combine, lse=None, split_rows: int = 0, ws=None,
                stream=None) -> None:
    """``decode_attn`` for queries that may share sequences: query t attends
    the first ``seq_lens[t]`` rows of table row ``token_seq[t]``."""
    lib = load_library()
    cache = _cache(pool, table)
    n = int(seq_lens.shape[0])
    st = lib.mla_attn_tokens(ctypes.byref(dims.c()), n, _ptr(q_abs), ctypes.byref(cache),
                             _ptr(token_seq), int(table.shape[0]), _ptr(seq_lens),
                             int(max_seq_len), float(softmax_scale), int(split_rows),
                             _ptr(v_combine), _ptr(lse), _ptr(ws),
                             ws.numel() * ws.element_size() if ws is not None else 0,
                             _stream(stream))
    _check(st, "mla_attn_tokens")


def out_proj(dims: Dims, v_combine, kv_b: Weight, out, o_proj: Optional[Weight] = None,
             ws=None, stream=None) -> None:
    lib = load_library()
    B = int(v_combine.shape[0])
    st = lib.mla_out_proj(ctypes.byref(dims.c()), B, _ptr(v_combine), ctypes.byref(kv_b.c()),
                          _c_or_null(o_proj, CWeight), _ptr(out), _ptr(ws),
                          ws.numel() * ws.element_size() if ws is not None else 0,
                          _stream(stream))
    _check(st, "mla_out_proj")


def layer_workspace_bytes(dims: Dims, batch: int, max_seq_len: int, split_rows: int = 0) -> int:
    return int(load_library().mla_layer_workspace_bytes(ctypes.byref(dims.c()), batch,
                                                        max_seq_len, split_rows))


def decode_layer(dims: Dims, x, positions, pool, table, seq_lens, max_seq_len: int,
                 softmax_scale: float, q_abs, v_combine, out, *, kv_a: Optional[Weight],
                 kv_a_norm: Weight, kv_b: Weight, inv_freq, rope_mscale: float,
                 q_a: Optional[Weight] = None, q_a_norm: Optional[Weight] = None,
                 q_b: Optional[Weight] = None, o_proj: Optional[Weight] = None, q_in=None,
                 lse=None, split_rows: int = 0, dev_status=None, ws=None, stream=None) -> None:
    """The whole decode step in one call (mla_decode_layer): the results of
    cache_append, absorb_q, decode_attn and out_proj in that order."""
    lib = load_library()
    rope = CRope(_ptr(inv_freq), float(rope_mscale))
    cw = {k: (w.c() if w is not None else None)
          for k, w in (("kv_a", kv_a), ("kv_a_norm", kv_a_norm), ("q_a", q_a),
                       ("q_a_norm", q_a_norm), ("q_b", q_b), ("kv_b", kv_b), ("o_proj", o_proj))}
    null = ctypes.POINTER(CWeight)()
    layer = CLayer(*[ctypes.pointer(cw[k]) if cw[k] is not None else null
                     for k in ("kv_a", "kv_a_norm", "q_a", "q_a_norm", "q_b", "kv_b", "o_proj")],
                   ctypes.pointer(rope))
    cache = _cache(pool, table)
    B = int(positions.shape[0])
    st = lib.mla_decode_layer(ctypes.byref(dims.c()), B, _ptr(x), _ptr(q_in), ctypes.byref(layer),
                              _ptr(positions), ctypes.byref(cache), _ptr(seq_lens),
                              int(max_seq_len), float(softmax_scale), int(split_rows),
                              _ptr(q_abs), _ptr(v_combine), _ptr(lse), _ptr(out),
                              _ptr(dev_status), _ptr(ws),
                              ws.numel() * ws.element_size() if ws is not None else 0,
                              _stream(stream))
    _check(st, "mla_decode_layer")
