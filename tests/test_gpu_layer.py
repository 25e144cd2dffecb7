"""GPU tests of mla_decode_layer, the whole decode step in one call.

The call is defined as cache_append, absorb_q, decode_attn and out_proj in
that order with the same arguments.  Its fused launches (one fp16 pack of x,
kv_a and q_a in one launch, the append and the q-latent RMSNorm in one launch,
the merge also writing W_UV's packed input) do the same arithmetic as the
separate calls, so every result -- the cache pool included -- must equal the
four calls' bit for bit.  The layer is also held to the stated bars against
the fp64 oracle, and a captured graph of the call replays to the eager
results.  On the 4-bit layer the graph holds seven kernels (q_b and the
absorb are one launch, and so are the attention merge and W_UV).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import attn_check, close_bf16, close_f32

pytestmark = pytest.mark.gpu

OUTPUTS = ("q_abs", "v_combine", "lse", "out", "pool", "status")


def host(x):
    a = x.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def raw(x):
    """The tensor's bytes (NaN padding compares equal to itself)."""
    return np.ascontiguousarray(x.detach().cpu().numpy()).view(np.uint8)


def sync():
    torch.cuda.synchronize()


CASES = [
    (1, {}),
    (2, dict(lens=[1000, 37], batch=2)),
    (3, dict(batch=3, lens=[1024, 1500, 2049])),
    (5, dict(batch=2, lens=[300, 1100])),
    (5, dict(batch=33, lens=[int(v) for v in np.random.default_rng(41).integers(1, 3000, 33)])),
    # one long query among two: the device plan cuts it into far more than 8
    # splits, so the layer's merge forms the merge kernel's 4 per-wave sums in
    # turn, over several batches each and past the first 64 splits
    (5, dict(batch=2, lens=[8192, 64])),
]
IDS = ["1", "2", "3", "5-b2", "5-b33", "5-long"]


@pytest.mark.parametrize("cfg,kw", CASES, ids=IDS)
def test_layer_equals_the_four_calls(cfg, kw):
    case = S.make_case(cfg, **kw)
    print(f"layer vs calls: config {cfg} {kw}", flush=True)
    a = D.stage(case)
    D.run_step(case, a)
    b = D.stage(case)
    D.run_layer(case, b)
    sync()
    for name in OUTPUTS:
        ga, gb = raw(getattr(a, name)), raw(getattr(b, name))
        if not np.array_equal(ga, gb):
            n = int(np.sum(ga != gb))
            pytest.fail(f"{name}: {n} of {ga.size} bytes differ from the four calls")


@pytest.mark.parametrize("cfg,kw", CASES[:4], ids=IDS[:4])
def test_layer_against_the_oracle(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    D.run_layer(case, ns)
    sync()
    res = O.decode_step(case)
    d = case.dims
    vc, lse, out = host(ns.v_combine), host(ns.lse), host(ns.out)
    if d.cache_dtype == O.F32:
        close_f32(vc, res["v_combine"], "v_combine")
        close_f32(out, res["out"].reshape(case.batch, -1), "out")
    else:
        close_bf16(vc, res["v_combine"], "v_combine")
        close_bf16(lse, res["lse"], "lse")
        close_bf16(out, res["out"].reshape(case.batch, -1), "out")
        # tight checks of the attention part on the oracle's cache and query
        q = ns.q_abs.clone()
        q.copy_(D.t(res["q_abs_stored"]))
        view = D.stage(case)
        view.pool = D.t(res["pool"])
        ws = D.workspace(view)
        D.attend(view, q, 0, ws)
        sync()
        attn_check(host(view.v_combine), host(view.lse), res["v_combine"], res["lse"],
                   f"config {cfg} layer attention")
    assert int(host(ns.status)[0]) == 0


def capture_layer(case, ns, ws):
    g = torch.cuda.CUDAGraph(keep_graph=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            D.run_layer(case, ns, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    sync()
    g.instantiate()
    return g


def test_layer_graph_replays_to_the_eager_results():
    case = S.make_case(5, batch=4, lens=[700, 64, 2000, 1333])
    ns = D.stage(case)
    ws = D.layer_workspace(ns)
    D.run_layer(case, ns, ws=ws)
    sync()
    ref = {k: raw(getattr(ns, k)) for k in OUTPUTS}
    g = capture_layer(case, ns, ws)
    for rep in range(3):
        # eager work between the replays: outputs cleared, the pool untouched
        for k in ("q_abs", "v_combine", "lse", "out"):
            getattr(ns, k).zero_()
        sync()
        g.replay()
        sync()
        for k in OUTPUTS:
            assert np.array_equal(raw(getattr(ns, k)), ref[k]), f"replay {rep}: {k} differs"


def kernel_nodes(g) -> int:
    """Kernel nodes of a captured graph (hipGraphGetNodes / hipGraphNodeGetType
    of the process's HIP runtime, the one torch loaded)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    graph = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    kernels = 0
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        kernels += t.value == 0  # hipGraphNodeTypeKernel
    return kernels


def test_layer_is_seven_kernels_on_the_4bit_layer():
    case = S.make_case(5, batch=2, lens=[300, 1100])
    ns = D.stage(case)
    ws = D.layer_workspace(ns)
    D.run_layer(case, ns, ws=ws)
    sync()
    g = capture_layer(case, ns, ws)
    assert kernel_nodes(g) == 7
