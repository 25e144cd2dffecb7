"""Stage a synthetic case on the GPU as torch tensors and library weight descriptors.

Pure data movement (numpy -> torch device memory); no arithmetic of the method.
"""
from __future__ import annotations

import copy
import dataclasses
import types

import numpy as np
import torch

import mla_latent_kv_11_amd as mla
from . import Case, Q4Weight, F32, BF16


def t(arr, device="cuda") -> torch.Tensor:
    """numpy -> device tensor with the same bytes (uint16 -> int16, uint32 -> int32)."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def weight(w, rows: int, cols: int, device="cuda") -> mla.Weight:
    if isinstance(w, Q4Weight):
        return mla.Weight(mla.MLA_Q4G64, rows, cols, t(w.packed, device), t(w.scales, device),
                          t(w.biases, device))
    a = np.asarray(w)
    if a.dtype == np.uint8:  # Q8_0 blocks
        return mla.Weight(mla.MLA_Q8_0, rows, cols, t(a.reshape(-1), device))
    dt = mla.MLA_BF16 if a.dtype == np.uint16 else mla.MLA_F32
    return mla.Weight(dt, rows, cols, t(a.reshape(rows, cols), device))


def dims_of(case: Case) -> mla.Dims:
    d = case.dims
    return mla.Dims(d.num_heads, d.qk_nope, d.qk_rope, d.v_head, d.kv_lora, d.hidden, d.q_lora,
                    d.block_size, d.cache_dtype, d.rms_eps)


def tile_weights(ns) -> None:
    """Swap every 4-bit weight of ``ns`` whose shape allows it (rows a multiple
    of 32, cols of 128) for its MLA_Q4G64_T repack."""
    for name in ("kv_a", "q_a", "q_b", "kv_b", "o_proj"):
        w = getattr(ns, name)
        if w is not None and w.dtype == mla.MLA_Q4G64 and w.rows % 32 == 0 and w.cols % 128 == 0:
            setattr(ns, name, mla.repack_q4g64(w))


def stage(case: Case, device="cuda", tiled: bool = False) -> types.SimpleNamespace:
    """Everything a decode step of ``case`` needs, resident in device memory
    (``tiled``: the 4-bit weights repacked by the library, see tile_weights)."""
    d = case.dims
    H, N, R, V, C = d.num_heads, d.qk_nope, d.qk_rope, d.v_head, d.kv_lora
    ns = types.SimpleNamespace()
    ns.dims = dims_of(case)
    ns.pool = t(case.pool, device)
    ns.table = t(case.table, device)
    ns.lens = t(case.lens.astype(np.int32), device)
    ns.positions = t(case.positions, device)
    ns.token_seq = t(case.token_seq, device) if case.token_seq is not None else None
    ns.max_len = int(case.lens.max()) if len(case.lens) else 0
    ns.x = t(case.x, device) if case.x is not None else None
    ns.kv_a = weight(case.kv_a, d.width, d.hidden, device) if case.kv_a is not None else None
    ns.kv_a_norm = weight(case.kv_a_norm, 1, C, device) if case.kv_a_norm is not None else None
    ns.q = t(case.q, device) if case.q is not None else None
    ns.q_a = weight(case.q_a, d.q_lora, d.hidden, device) if case.q_a is not None else None
    ns.q_a_norm = weight(case.q_a_norm, 1, d.q_lora, device) if case.q_a_norm is not None else None
    ns.q_b = weight(case.q_b, H * (N + R), d.q_lora, device) if case.q_b is not None else None
    ns.kv_b = weight(case.kv_b, H * (N + V), C, device) if case.kv_b is not None else None
    ns.o_proj = (weight(case.o_proj, d.hidden, H * V, device)
                 if case.o_proj is not None else None)
    ns.q_abs_given = t(case.q_abs, device) if case.q_abs is not None else None
    cdt = torch.float32 if d.cache_dtype == F32 else torch.int16
    B = case.batch
    ns.q_abs = torch.empty((B, H, d.width), dtype=cdt, device=device)
    ns.v_combine = torch.empty((B, H, C), dtype=torch.float32, device=device)
    ns.lse = torch.empty((B, H), dtype=torch.float32, device=device)
    out_cols = d.hidden if case.o_proj is not None else H * V
    ns.out = torch.empty((B, out_cols), dtype=torch.float32, device=device)
    ns.status = torch.zeros(1, dtype=torch.int32, device=device)
    y = case.yarn
    inv, rm, sc = mla.yarn_tables(R, N + R, y.theta, y.factor, y.original_max_pos, y.beta_fast,
                                  y.beta_slow, y.mscale, y.mscale_all_dim)
    ns.inv_freq = torch.tensor(inv, dtype=torch.float32, device=device)
    ns.rope_mscale = rm
    ns.softmax_scale = float(case.softmax_scale) if case.softmax_scale is not None else sc
    if tiled:
        tile_weights(ns)
    return ns


WEIGHT_NAMES = ("kv_a", "kv_a_norm", "q_a", "q_a_norm", "q_b", "kv_b", "o_proj")


def weight_copies(ns, n: int) -> list:
    """``ns`` and n - 1 copies of it whose weights live in buffers of their
    own (the same values; every other buffer shared): steps that use them in
    turn read their weights from memory as the layers of a model do, where a
    single set reused every step would stay in the device caches."""
    out = [ns]
    for _ in range(n - 1):
        c = copy.copy(ns)
        for name in WEIGHT_NAMES:
            w = getattr(ns, name)
            if w is not None:
                setattr(c, name, dataclasses.replace(
                    w, data=w.data.clone(),
                    scales=w.scales.clone() if w.scales is not None else None,
                    biases=w.biases.clone() if w.biases is not None else None))
        out.append(c)
    return out


def workspace(ns, split_rows: int = 0, device="cuda") -> torch.Tensor:
    n = mla.workspace_bytes(ns.dims, int(ns.lens.shape[0]), ns.max_len, split_rows)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def append(ns, ws, stream=None) -> None:
    """The append call of the staged case (per-token sequence map when it has one)."""
    if ns.token_seq is None:
        mla.cache_append(ns.dims, ns.x, ns.kv_a, ns.kv_a_norm, ns.inv_freq, ns.rope_mscale,
                         ns.positions, ns.pool, ns.table, ns.status, ws, stream)
    else:
        mla.cache_append_tokens(ns.dims, ns.x, ns.kv_a, ns.kv_a_norm, ns.inv_freq,
                                ns.rope_mscale, ns.positions, ns.token_seq, ns.pool, ns.table,
                                ns.status, ws, stream)


def attend(ns, q_abs, split_rows, ws, stream=None) -> None:
    """The attention call of the staged case (per-token sequence map when it has one)."""
    if ns.token_seq is None:
        mla.decode_attn(ns.dims, q_abs, ns.pool, ns.table, ns.lens, ns.max_len, ns.softmax_scale,
                        ns.v_combine, ns.lse, split_rows, ws, stream)
    else:
        mla.attn_tokens(ns.dims, q_abs, ns.pool, ns.table, ns.token_seq, ns.lens, ns.max_len,
                        ns.softmax_scale, ns.v_combine, ns.lse, split_rows, ws, stream)


def run_step(case: Case, ns, split_rows: int = 0, ws=None, stream=None) -> None:
    """append -> absorb -> attention -> out_proj on the staged case (library calls only)."""
    ws = workspace(ns, split_rows) if ws is None else ws
    if case.appended:
        append(ns, ws, stream)
    if ns.q_abs_given is not None:
        q_abs = ns.q_abs_given
    else:
        q_in = ns.q if ns.q is not None else ns.x
        mla.absorb_q(ns.dims, q_in, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                     ns.q_a, ns.q_a_norm, ns.q_b, ws, stream)
        q_abs = ns.q_abs
    attend(ns, q_abs, split_rows, ws, stream)
    if ns.kv_b is not None:
        mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, ns.out, ns.o_proj, ws, stream)


def layer_workspace(ns, split_rows: int = 0, device="cuda") -> torch.Tensor:
    n = mla.layer_workspace_bytes(ns.dims, int(ns.lens.shape[0]), ns.max_len, split_rows)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def run_layer(case: Case, ns, split_rows: int = 0, ws=None, stream=None) -> None:
    """The staged case's step as one decode_layer call (a case with an append
    and a query to absorb: configurations 1, 2, 3 and 5)."""
    ws = layer_workspace(ns, split_rows) if ws is None else ws
    mla.decode_layer(ns.dims, ns.x, ns.positions, ns.pool, ns.table, ns.lens, ns.max_len,
                     ns.softmax_scale, ns.q_abs, ns.v_combine, ns.out, kv_a=ns.kv_a,
                     kv_a_norm=ns.kv_a_norm, kv_b=ns.kv_b, inv_freq=ns.inv_freq,
                     rope_mscale=ns.rope_mscale, q_a=ns.q_a, q_a_norm=ns.q_a_norm, q_b=ns.q_b,
                     o_proj=ns.o_proj, q_in=ns.q, lse=ns.lse, split_rows=split_rows,
                     dev_status=ns.status, ws=ws, stream=stream)


class GraphStep:
    """One decode step as the library calls it, replayable as one HIP graph:

      pre   cache_append on the calling stream and, at the same time, absorb_q
            on a side stream (independent: both only read x; each has its own
            workspace) -- or both on the calling stream (two_streams=False)
      attn  decode_attn
      post  out_proj

    ``run(eager=True)`` launches the calls; ``capture()`` records the whole
    step into one graph and ``run()`` replays it on the current stream.
    Library calls only; the graph allocates nothing.
    """

    def __init__(self, case: Case, ns, split_rows: int = 0, two_streams: bool = True):
        self.case, self.ns, self.split_rows = case, ns, split_rows
        self.two_streams = two_streams
        self.ws_a = workspace(ns, split_rows)
        self.ws_b = workspace(ns, split_rows)
        self.side = torch.cuda.Stream()
        self.q_abs = ns.q_abs_given if ns.q_abs_given is not None else ns.q_abs
        self.graph = None

    def pre(self):
        ns, case = self.ns, self.case
        cur = torch.cuda.current_stream()
        side = self.two_streams and ns.q_abs_given is None
        if ns.q_abs_given is None:
            if side:
                self.side.wait_stream(cur)
            with torch.cuda.stream(self.side if side else cur):
                q_in = ns.q if ns.q is not None else ns.x
                mla.absorb_q(ns.dims, q_in, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions,
                             ns.q_abs, ns.q_a, ns.q_a_norm, ns.q_b, self.ws_b)
        if case.appended:
            append(ns, self.ws_a)
        if side:
            cur.wait_stream(self.side)

    def attn(self):
        attend(self.ns, self.q_abs, self.split_rows, self.ws_a)

    def post(self):
        ns = self.ns
        if ns.kv_b is not None:
            mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, ns.out, ns.o_proj, self.ws_a)

    def capture(self):
        """Record the whole step (run it eagerly at least once before)."""
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.pre()
            self.attn()
            self.post()
        torch.cuda.synchronize()

    def run(self, eager=False):
        if eager:
            self.pre()
            self.attn()
            self.post()
        else:
            self.graph.replay()


class LayerStep:
    """Decode steps as decode_layer calls (on the 4-bit layer: 7 kernels on one
    stream each), ``per_graph`` of them per run: one HIP graph holds that many
    steps, as a multi-layer model's graph holds one step per layer, so the
    gap between graph launches is paid once per run.  ``sets`` (from
    weight_copies; default [ns]) are used in turn, one per step.  Library
    calls only."""

    def __init__(self, case: Case, ns, split_rows: int = 0, per_graph: int = 1, sets=None):
        self.case, self.ns, self.split_rows = case, ns, split_rows
        self.per_graph = per_graph
        self.sets = list(sets) if sets else [ns]
        self.ws = layer_workspace(ns, split_rows)
        self.graph = None
        self.i = 0

    def call(self):
        run_layer(self.case, self.sets[self.i % len(self.sets)], self.split_rows, self.ws)
        self.i += 1

    def capture(self):
        """Record per_graph calls (run the call eagerly at least once before)."""
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        self.i = 0
        with torch.cuda.graph(self.graph):
            for _ in range(self.per_graph):
                self.call()
        torch.cuda.synchronize()

    def run(self, eager=False):
        """per_graph steps."""
        if eager:
            for _ in range(self.per_graph):
                self.call()
        else:
            self.graph.replay()
