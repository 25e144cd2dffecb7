"""GPU tests of the tiled 4-bit weight format (MLA_Q4G64_T).

mla_repack_q4g64 moves the bytes of a row-major 4-bit weight into 2 KB blocks
per (32-row tile, 128 input columns) in the order the MFMA products load them.
The repack is checked byte for byte against the layout the header states,
written out here with numpy; and since only the reads change, every output of
the four calls and of the layer call with tiled weights must equal, bit for
bit, the outputs with the row-major weights -- on the MFMA paths and on the
VALU path that reads single elements (a q_nope depth of 64 sends the absorb
there).  The row-major results are held to the oracle by the parity tests; the
small case here is also checked against the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import close_bf16

pytestmark = pytest.mark.gpu

OUTPUTS = ("q_abs", "v_combine", "lse", "out", "pool", "status")


def raw(x):
    return np.ascontiguousarray(x.detach().cpu().numpy()).view(np.uint8)


def expected_tiled(w: S.Q4Weight):
    """The MLA_Q4G64_T bytes of ``w`` as the header describes them: block
    (t, u) = 2048 bytes at (t * cols/128 + u) * 2048; inside it part p (1 KB)
    holds, for lane L = l + 32 h, the 16 bytes of row 32 t + l at byte
    64 u + 32 h + 16 p of that row; scale and bias of lane L at
    (t * cols/128 + u) * 64 + L are those of group 2 u + h of the row."""
    rows, cols = w.rows, w.cols
    T, Un = rows // 32, cols // 128
    b = np.ascontiguousarray(w.packed).view(np.uint8).reshape(T, 32, Un, 2, 2, 16)  # t l u h p j
    data = b.transpose(0, 2, 4, 3, 1, 5).reshape(-1)                                # t u p h l j
    def groups(g):
        return np.ascontiguousarray(g).reshape(T, 32, Un, 2).transpose(0, 2, 3, 1).reshape(-1)
    return data, groups(w.scales), groups(w.biases)


@pytest.mark.parametrize("rows,cols", [(32, 128), (96, 384), (576, 1024)])
def test_repack_layout(rows, cols):
    print(f"repack {rows} x {cols}", flush=True)
    w = S.draw_q4(np.random.default_rng(rows + cols), rows, cols)
    tw = mla.repack_q4g64(D.weight(w, rows, cols))
    torch.cuda.synchronize()
    assert tw.dtype == mla.MLA_Q4G64_T
    data, sc, bi = expected_tiled(w)
    assert np.array_equal(raw(tw.data), data)
    assert np.array_equal(raw(tw.scales).view(np.uint16), sc)
    assert np.array_equal(raw(tw.biases).view(np.uint16), bi)


def small_q4_case(batch=3, seed=77):
    """A 4-bit layer with q_nope 64 (the absorb's VALU path): 128 heads, latent
    512, rope 64 (the bf16 attention kernel's shape), v_head 64, hidden 256,
    q_lora 128, bf16 cache."""
    rng = np.random.default_rng(seed)
    d = S.Dims(num_heads=128, qk_nope=64, qk_rope=64, v_head=64, kv_lora=512, hidden=256,
               q_lora=128, cache_dtype=S.BF16)
    H, N, R, V, C = 128, 64, 64, 64, 512
    L = rng.integers(40, 400, size=batch).astype(np.int32)
    pool, table = S.build_pool(rng, d, L, std=1.0, paged=True)
    return S.Case("small-q4", d, S.Yarn(), batch, L, pool, table, None,
                  x=rng.standard_normal((batch, d.hidden), dtype=np.float32),
                  kv_a=S.draw_q4(rng, C + R, d.hidden),
                  kv_a_norm=S.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(C)),
                  q_a=S.draw_q4(rng, d.q_lora, d.hidden),
                  q_a_norm=S.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(d.q_lora)),
                  q_b=S.draw_q4(rng, H * (N + R), d.q_lora),
                  kv_b=S.draw_q4(rng, H * (N + V), C),
                  o_proj=S.draw_q4(rng, d.hidden, H * V))


def compare(a, b, what):
    for name in OUTPUTS:
        ga, gb = raw(getattr(a, name)), raw(getattr(b, name))
        if not np.array_equal(ga, gb):
            pytest.fail(f"{what}: {name}: {int(np.sum(ga != gb))} of {ga.size} bytes differ "
                        "between the tiled and the row-major weights")


CASES = [
    (5, dict(batch=2, lens=[300, 1100])),
    (5, dict(batch=33, lens=[int(v) for v in np.random.default_rng(43).integers(1, 2000, 33)])),
    (5, dict(batch=40, lens=[64] * 40)),
]


@pytest.mark.parametrize("cfg,kw", CASES, ids=["b2", "b33", "b40"])
@pytest.mark.parametrize("run", ["calls", "layer"])
def test_tiled_weights_give_the_row_major_bits(cfg, kw, run):
    case = S.make_case(cfg, **kw)
    print(f"tiled vs row-major: {run} config {cfg} batch {case.batch}", flush=True)
    step = D.run_step if run == "calls" else D.run_layer
    a = D.stage(case)
    step(case, a)
    b = D.stage(case, tiled=True)
    for name in ("kv_a", "q_a", "q_b", "kv_b", "o_proj"):
        assert getattr(b, name).dtype == mla.MLA_Q4G64_T, name
    step(case, b)
    torch.cuda.synchronize()
    compare(a, b, f"{run}, batch {case.batch}")


@pytest.mark.parametrize("run", ["calls", "layer"])
def test_tiled_weights_on_the_element_paths(run):
    case = small_q4_case()
    print(f"tiled vs row-major, small 4-bit layer: {run}", flush=True)
    step = D.run_step if run == "calls" else D.run_layer
    a = D.stage(case)
    step(case, a)
    b = D.stage(case, tiled=True)
    assert b.kv_b.dtype == mla.MLA_Q4G64_T
    step(case, b)
    torch.cuda.synchronize()
    compare(a, b, f"small 4-bit layer, {run}")
    res = O.decode_step(case)
    close_bf16(raw(b.v_combine).view(np.float32).reshape(res["v_combine"].shape),
               res["v_combine"], "v_combine")
    close_bf16(raw(b.out).view(np.float32).reshape(case.batch, -1),
               res["out"].reshape(case.batch, -1), "out")
