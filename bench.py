#!/usr/bin/env python3
"""Benchmark of single-token MLA decode (one layer) on one MI355X.

A step is one pass of the whole decode path over one batch: kv_a projection +
latent RMSNorm + YaRN RoPE + paged append, the q chain + absorb, decode
attention over the paged latent cache, the W_UV expansion and o_proj.  The
step is one mla_decode_layer call (7 kernels on one stream), replayed from HIP
graphs that hold up to 10 steps each, as a multi-layer model's graph holds one
step per layer (``--eager``: the call launched every step); the same step as the
four separate calls (append and absorb on two streams, one graph) is timed
beside it.  The attention call is then timed where the step runs it (HIP events
around decode_attn inside eager steps of the four calls, between
append/absorb and out_proj), and also back to back (a replayed graph of 20
calls; ``--eager``: one by one).  The
workload is the full per-layer configuration: batch 32, 16384 cached rows per
sequence (append at 16383), DeepSeek-V3 shapes (128 heads, latent 512, rope
64), hidden 7168, q_lora 1536, 4-bit affine (group 64) projections (repacked
once, before timing, into the library's tiled layout; ``--row-major-weights``:
as given), bf16 cache.  Inputs are synthetic (seeded) and resident in HBM
before timing.

Prints one JSON line.  ``roofline`` describes the attention call (its split
kernel plus the split-K combine kernel), timed with HIP events on the stream
it is launched on, hot (back-to-back calls) and cold (``ms_per_launch_cold``:
a 1 GiB write evicts the last-level cache before each call); ``cpu_baseline``
is the fp64 oracle timed on a bounded sample of the same workload on the host
cores.  ``attn_only`` repeats the attention measurement on the other
full-size workloads (one 4096-row sequence; 64 ragged paged sequences of
1024-8192 rows; 4 sequences of 131072 rows), each with the oracle's attention
timed on the same inputs.
"""
from __future__ import annotations

import argparse
import copy
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attn: HBM GB/s + MFMA util + tokens/s, 128 heads, L=4096..131072"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROW_BYTES = 576 * 2            # one bf16 cache row [c_kv ; k_pe]
ROW_FLOPS = 2 * 128 * 576 + 2 * 128 * 512   # scores + latent combine per row, 128 heads
COUNTERS = os.path.join(ROOT, "profiles", "attn_mfma_b32_L16384_counters.md")
KERNEL_SRC = os.path.join(ROOT, "mla_latent_kv_11_amd", "csrc", "attn_mfma.hip")


def attn_alg(B, rows, H=128, W=576, C=512):
    """Algorithmic bytes and flops of one attention call: every cache row once,
    q_abs (bf16) in, v_combine (fp32) out."""
    byts = rows * ROW_BYTES + B * H * W * 2 + B * H * C * 4
    return byts, rows * ROW_FLOPS


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """Counter-measured HBM bytes per attention call, if taken on this kernel source.

    The figures live in a JSON block of the counter summary under profiles/."""
    try:
        with open(COUNTERS) as f:
            text = f.read()
        c = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    if c.get("kernel_sha256_16") != kernel_hash():
        return None
    return c.get("hbm_bytes_per_call")


def cold_call_ms(torch, call, stream, runs=20, scratch_bytes=1 << 30):
    """Median time of single calls, each after a 1 GiB write (not timed) that
    evicts the 256 MB last-level cache, so that every input comes from HBM."""
    scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device="cuda")
    ev = []
    for r in range(runs):
        scratch.fill_(r & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    del scratch
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in ev)


def oracle_attn_seconds(case):
    """The oracle's latent attention (fp64 numpy) on the same inputs, one pass;
    its query is the oracle's own absorbed query, computed outside the timing."""
    from oracle import mla_oracle as O
    q64 = O.attention_query(case)
    sc = float(O.tables_for(case)[2])
    t0 = time.perf_counter()
    O.attention_latent(case.dims, q64, case.pool, case.table, case.lens, sc)
    return time.perf_counter() - t0


def time_attn_only(cfg, torch, D, S, mla, iters=50, warm=50, oracle=True, lens_plan=False):
    """Attention call alone on a full-size configuration (q_abs given or absorbed
    once): hot (back-to-back calls) and cold (cache evicted before each call),
    and the oracle's attention on the same inputs.  ``lens_plan``: also the
    split plan sized from the host-side lengths (mla_attn_plan_lens)."""
    case = S.make_case(cfg)
    ns = D.stage(case)
    ws = D.workspace(ns)
    r_lens = mla.attn_plan_lens(ns.dims, case.lens)[0] if lens_plan else 0
    if r_lens:
        ws_l = D.workspace(ns, r_lens)
        ws = ws if ws.numel() >= ws_l.numel() else ws_l
    if ns.q_abs_given is not None:
        q_abs = ns.q_abs_given
    else:
        mla.absorb_q(ns.dims, ns.q, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions, ns.q_abs,
                     ws=ws)
        q_abs = ns.q_abs
    stream = torch.cuda.current_stream()
    rows = int(case.lens.sum())
    byts, flops = attn_alg(case.batch, rows)

    def measure(split_rows):
        def call():
            mla.decode_attn(ns.dims, q_abs, ns.pool, ns.table, ns.lens, ns.max_len,
                            ns.softmax_scale, ns.v_combine, ns.lse, split_rows, ws)
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        settle(call, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        ms_cold = cold_call_ms(torch, call, stream)
        t = ms * 1e-3
        return {
            "split_rows": mla.attn_plan(ns.dims, case.batch, ns.max_len, split_rows)[0],
            "ms": round(ms, 4), "ms_cold": round(ms_cold, 4),
            "gbps": round(byts / t / 1e9, 1), "tflops": round(flops / t / 1e12, 1),
            "f_hbm": round(byts / t / 1e9 / HBM_PEAK_GBS, 3),
            "f_mfma": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 3),
            "f_roof": round(max(byts / (HBM_PEAK_GBS * 1e9),
                                flops / (BF16_PEAK_TFLOPS * 1e12)) / t, 3),
            "tokens_per_s": round(case.batch / t, 1),
            "f_roof_cold": round(max(byts / (HBM_PEAK_GBS * 1e9),
                                     flops / (BF16_PEAK_TFLOPS * 1e12)) / (ms_cold * 1e-3), 3),
        }
    out = {"batch": case.batch, "rows": rows, **measure(0)}
    if r_lens:
        out["plan_from_lengths"] = measure(r_lens)
    del ns, ws
    if oracle:
        sec = oracle_attn_seconds(case)
        out["oracle"] = {"seconds": round(sec, 3), "rows_per_s": round(rows / sec, 1),
                         "gbps_equiv": round(byts / sec / 1e9, 3),
                         "tokens_per_s": round(case.batch / sec, 3),
                         "gpu_speedup": round(sec / (out["ms"] * 1e-3), 1),
                         "cores": oracle_threads()}
    return out


def settle(run, torch, min_ms=150.0):
    """Untimed steps until at least ``min_ms`` of wall time has passed, whatever
    the warm-up count: the GPU needs some tens of ms of sustained load before
    its clocks settle.  Returns (milliseconds, steps)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(10):
            run()
        n += 10
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms:
            return el, n


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:
        return os.cpu_count() or 1


def time_kv_b_formats(case, torch, D, S, mla, iters=20):
    """absorb_q and out_proj of the same layer with kv_b as 4-bit affine and as
    Q8_0 (both read in place by the MFMA kernels); HIP events around ``iters``
    back-to-back calls of each."""
    import numpy as np
    out = {}
    stream = torch.cuda.current_stream()
    for name, c in (("q4g64", case), ("q8_0", S.with_q8_0_kv_b(case))):
        ns = D.stage(c)
        ws = D.workspace(ns)

        def absorb():
            mla.absorb_q(ns.dims, ns.q if ns.q is not None else ns.x, ns.kv_b, ns.inv_freq, ns.rope_mscale, ns.positions,
                         ns.q_abs, ns.q_a, ns.q_a_norm, ns.q_b, ws)

        def expand():
            mla.out_proj(ns.dims, ns.v_combine, ns.kv_b, ns.out, ns.o_proj, ws)
        r = {}
        for fname, f in (("absorb_q_ms", absorb), ("out_proj_ms", expand)):
            for _ in range(5):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            r[fname] = round(e0.elapsed_time(e1) / iters, 4)
        kv = c.kv_b
        r["kv_b_bytes"] = int(kv.packed.nbytes + kv.scales.nbytes + kv.biases.nbytes
                              if hasattr(kv, "packed") else np.asarray(kv).nbytes)
        out[name] = r
        del ns, ws
    return out


def time_tokens(torch, D, S, mla, iters=10):
    """The whole layer (4-bit projections) over several new tokens per sequence,
    through the token calls: multi-token decode (32 sequences x 4 tokens on
    16380 prior rows) and a prefill chunk (4 sequences x 512 tokens on 8192
    prior rows).  Step: HIP events around ``iters`` replays of the captured
    step; attention: events around the attention call inside ``iters`` eager
    steps.  Algorithmic attention bytes count each sequence's rows once."""
    import numpy as np
    out = {}
    stream = torch.cuda.current_stream()
    for name, prior, chunk in (("decode_b32_t4_L16384", [16380] * 32, 4),
                               ("prefill_b4_t512_L8192", [8192] * 4, 512)):
        case = S.make_chunk_case(5, prior, chunk)
        ns = D.stage(case, tiled=True)
        step = D.GraphStep(case, ns)
        for _ in range(3):
            step.run(eager=True)
        step.capture()
        for _ in range(3):
            step.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            step.run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / iters
        ta = []
        for _ in range(iters):
            step.pre()
            e0.record(stream)
            step.attn()
            e1.record(stream)
            step.post()
            torch.cuda.synchronize()
            ta.append(e0.elapsed_time(e1))
        ms_attn = float(np.mean(ta))
        n = case.batch
        rows_unique = int(np.sum(np.asarray(prior) + chunk))
        byts = rows_unique * ROW_BYTES + n * 128 * 576 * 2 + n * 128 * 512 * 4
        flops = int(case.lens.astype(np.int64).sum()) * ROW_FLOPS
        t = ms_attn * 1e-3
        out[name] = {
            "seqs": len(prior), "tokens": n, "ms_per_step": round(ms_step, 4),
            "tokens_per_s": round(n / (ms_step * 1e-3), 1), "attn_ms": round(ms_attn, 4),
            "attn_tflops": round(flops / t / 1e12, 1),
            "attn_f_mfma": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 3),
            "attn_gbps_unique_rows": round(byts / t / 1e9, 1),
            "attn_f_roof": round(max(byts / (HBM_PEAK_GBS * 1e9),
                                     flops / (BF16_PEAK_TFLOPS * 1e12)) / t, 3),
        }
        del step, ns
    return out


def cpu_baseline(case, seqs, min_seconds=10.0, max_reps=8):
    """The oracle's whole step on ``seqs`` sequences of the same workload,
    repeated until about ``min_seconds`` of host work."""
    import numpy as np
    from oracle import mla_oracle as O
    sub = S_sub(case, seqs)
    cores = oracle_threads()
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        res = O.decode_step(sub)
        total += time.perf_counter() - t0
        reps += 1
    assert np.isfinite(res["out"]).all()
    return {"value": round(seqs * reps / total, 4), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{seqs} of 32 sequences (16384 rows each), whole layer step in fp64 numpy, "
                      f"{reps} repetitions, {total:.1f} s"}


def copy_calibration(torch, gib=1):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters to bytes: each copy reads and writes exactly ``gib`` GiB."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def S_sub(case, seqs):
    import copy
    sub = copy.copy(case)
    sub.batch = seqs
    sub.lens = case.lens[:seqs]
    sub.table = case.table[:seqs]
    nb = int(((case.lens[:seqs].astype(int) + 63) // 64).sum())
    used = sorted(set(case.table[:seqs].reshape(-1).tolist()) - {-1})
    assert len(used) == nb
    sub.x = case.x[:seqs]
    return sub


class Turns:
    """Several steps run in turn, one per run (each captures its own graph)."""

    per_graph = 1

    def __init__(self, steps):
        self.steps, self.k = steps, 0

    def capture(self):
        for s in self.steps:
            s.capture()

    def run(self, eager=False):
        self.steps[self.k % len(self.steps)].run(eager=eager)
        self.k += 1


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clocks settle under some tens of ms of sustained load: besides the
    # warm-up steps, at least 150 ms of untimed steps run before the timing
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extra", action="store_true", help="skip the per-configuration attention lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--eager", action="store_true",
                    help="launch every call eagerly on one stream (no graphs, no second stream)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--attn-only", action="store_true",
                    help="only the attention call on the other full-size workloads (one JSON "
                         "object of them; not the benchmark line)")
    ap.add_argument("--row-major-weights", action="store_true",
                    help="time the step on the 4-bit weights as given (no tiled repack)")
    ap.add_argument("--weight-sets", type=int, default=4,
                    help="copies of the layer's weights used in turn, one per step (4 x 105 MB "
                         "exceed the 256 MB last-level cache, so each step reads its weights "
                         "from HBM, as in a model whose layers each bring their own)")
    ap.add_argument("--attn-cfg", type=int, choices=(2, 3, 4), default=None,
                    help="with --attn-only: just this workload (2: 1 x 4096, 3: 64 ragged "
                         "paged sequences, 4: 4 x 131072), e.g. for counter passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import mla_latent_kv_11_amd as mla
    import mla_synth as S
    from mla_synth import device as D
    globals()["S"] = S

    mla.load_library()
    if args.attn_only:
        extra = {}
        for cfg, name in ((2, "b1_L4096"), (3, "b64_L1024-8192_paged"), (4, "b4_L131072")):
            if args.attn_cfg not in (None, cfg):
                continue
            extra[name] = time_attn_only(cfg, torch, D, S, mla, oracle=not args.no_cpu,
                                         lens_plan=(cfg == 3 and args.attn_cfg is None))
        print(json.dumps({"attn_only": extra}), flush=True)
        return
    case = S.make_case(5)
    # The 4-bit weights are repacked once, before timing, into the tiled
    # format the MFMA products read in whole lines (mla_repack_q4g64), as a
    # server would at load time; the row-major step is timed beside it.
    ns_rm = D.stage(case)
    ns = ns_rm
    if not args.row_major_weights:
        ns = copy.copy(ns_rm)
        D.tile_weights(ns)
    B = case.batch
    rows = int(case.lens.sum())
    # One step = one mla_decode_layer call (the fused front, attention with its
    # merge, W_UV and o_proj: 7 kernels on one stream), replayed from HIP graphs
    # of step_graph steps (--eager: the call launched every step).
    def timed_steps(step):
        g = getattr(step, "per_graph", 1)  # steps per run
        for _ in range(max(1, args.warmup // g)):
            step.run(eager=True)
        torch.cuda.synchronize()
        if not args.eager:
            step.capture()
            for _ in range(max(1, args.warmup // g)):
                step.run()
        torch.cuda.synchronize()
        settle_ms_, runs = settle(lambda: step.run(eager=args.eager), torch)
        t0 = time.perf_counter()
        for i in range(args.steps // g):
            step.run(eager=args.eager)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, (settle_ms_, runs * g)

    # Steps per graph: the largest of 10, 5, 4, 2, 1 that divides --steps.
    step_graph = next(g for g in (10, 5, 4, 2, 1) if args.steps % g == 0)
    # Consecutive steps use the copies of the weights in turn: one set reused
    # by every step would stay in the 256 MB last-level cache, since the cache
    # rows' copies are non-temporal, and the projections would then be timed
    # on cached weights, as no model with several layers runs them.
    n_sets = max(1, args.weight_sets)
    sets = D.weight_copies(ns, n_sets)
    ms_step, (settle_ms, settle_steps) = timed_steps(
        D.LayerStep(case, ns, per_graph=step_graph, sets=sets))
    assert int(ns.status.cpu()[0]) == 0
    ms_step_rm = None
    if ns is not ns_rm:
        sets_rm = D.weight_copies(ns_rm, n_sets)
        ms_step_rm, _ = timed_steps(D.LayerStep(case, ns_rm, per_graph=step_graph, sets=sets_rm))
        del sets_rm
    # The same step as the four calls: cache_append and absorb_q on two streams
    # (independent), then decode_attn, then out_proj, replayed as one HIP graph
    # per step (--eager: launched one by one on one stream); the weight sets in
    # turn, one graph each.
    four = [D.GraphStep(case, w, two_streams=not args.eager) for w in sets]
    step = four[0]
    ms_step_calls, _ = timed_steps(Turns(four))
    assert int(ns.status.cpu()[0]) == 0

    # The attention call timed where the step runs it: eager steps (the same
    # kernels the graph replays), HIP events on its stream right before and
    # after decode_attn, between the step's append/absorb and its out_proj.
    stream = torch.cuda.current_stream()
    n_in = max(args.steps, 50)
    in_step = []
    for _ in range(n_in):
        step.pre()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step.attn()
        e1.record(stream)
        step.post()
        in_step.append((e0, e1))
    torch.cuda.synchronize()
    attn_ms = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in in_step)

    # The same call back to back: a graph of 20 calls on the step's inputs,
    # replayed between two HIP events (events cannot be read from nodes inside
    # a replayed graph); --eager: the calls launched one by one.
    per_graph, reps = 20, max(args.steps // 20, 5)
    n_attn = per_graph * reps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.eager:
        attn_run = lambda: [step.attn() for _ in range(per_graph)]
    else:
        g_attn = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g_attn):
            for _ in range(per_graph):
                step.attn()
        attn_run = g_attn.replay
    attn_run()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        attn_run()
    e1.record(stream)
    torch.cuda.synchronize()
    attn_b2b_ms = e0.elapsed_time(e1) / n_attn

    byts, flops = attn_alg(B, rows)
    t_attn = attn_ms * 1e-3
    achieved = byts / t_attn / 1e9
    r_split, n_split = mla.attn_plan(ns.dims, B, ns.max_len, 0)
    line = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "MLA decode layer, batch 32, L=16384 (append at 16383), 128 heads, "
                        "kv_lora 512 + rope 64, hidden 7168, q_lora 1536, 4-bit g64 projections, "
                        "bf16 paged cache (64-row blocks)",
            "launch": "one mla_decode_layer call per step, eager" if args.eager else
                      f"HIP graphs of {step_graph} steps, each step one mla_decode_layer call "
                      "(7 kernels, one stream)",
            "weights": "4-bit g64 as given (row-major)" if ns is ns_rm else
                       "4-bit g64 repacked once before timing into the tiled layout "
                       "(mla_repack_q4g64, MLA_Q4G64_T; same values, same results)",
            "weight_sets": f"{n_sets} copies of the layer's weights (105 MB each) used in turn, "
                           "one per step, so that each step reads its weights from HBM",
            "ms_per_step_row_major_weights": None if ms_step_rm is None else round(ms_step_rm, 4),
            "ms_per_step_four_calls": round(ms_step_calls, 4),
            "four_calls_launch": "eager, one stream" if args.eager else
                                 "cache_append | absorb_q on two streams, decode_attn, "
                                 "out_proj; one HIP graph per step",
            "global_batch": B, "seq_len": int(ns.max_len), "parallelism": "none (1 GPU)",
            "split_rows": r_split, "splits_per_seq": n_split,
            "precision": "attention: bf16 MFMA operands, fp32 accumulate, fp32 softmax; "
                         "4-bit projections: fp16 MFMA operands, fp32 accumulate",
            "settle": f"{settle_steps} untimed steps ({settle_ms:.0f} ms) after the warm-up",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 3),
            "traffic": stored_traffic(),
            "kernel": "mla_decode_attn (attn_mfma_kernel + attn_combine_f16_kernel)",
            "ms_per_launch": round(attn_ms, 4),
            "timing": f"mean of {n_in} decode_attn calls inside eager steps, HIP events on "
                      "their stream around each call",
            "ms_per_launch_back_to_back": round(attn_b2b_ms, 4),
            "timing_back_to_back": f"{n_attn} back-to-back decode_attn calls ("
                      + ("eager" if args.eager else f"graphs of {per_graph}, replayed")
                      + ") between two HIP events",
            "alg_bytes": byts,
            "mfma_tflops": round(flops / t_attn / 1e12, 1),
            "mfma_frac": round(flops / t_attn / 1e12 / BF16_PEAK_TFLOPS, 3),
        },
    }
    # the same call on this workload with the last-level cache evicted before each call
    line["roofline"]["ms_per_launch_cold"] = round(cold_call_ms(torch, step.attn, stream), 4)
    if not args.no_extra:
        extra = {}
        for cfg, name in ((2, "b1_L4096"), (3, "b64_L1024-8192_paged"), (4, "b4_L131072")):
            extra[name] = time_attn_only(cfg, torch, D, S, mla, oracle=not args.no_cpu,
                                         lens_plan=(cfg == 3))
        line["attn_only"] = extra
        line["kv_b_formats"] = time_kv_b_formats(case, torch, D, S, mla)
        line["several_tokens"] = time_tokens(torch, D, S, mla)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seqs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
