"""GPU test of mla_decode_attn_noalloc, the attention entry point that keeps its
split partials in the library's static device scratch instead of a caller
workspace.  Through the C ABI it must give, bit for bit, what mla_decode_attn
gives with a workspace, on two calls in a row (the second smaller, reusing the
scratch the first left behind), and both must meet the oracle's tight checks;
a plan whose partials exceed the scratch is refused before any launch.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_11_amd as mla
import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

from parity import attn_check

pytestmark = pytest.mark.gpu


def host(x):
    return x.detach().cpu().numpy()


def both(case, split_rows):
    ns = D.stage(case)
    ws = D.workspace(ns, split_rows)
    vc_ws, lse_ws = torch.empty_like(ns.v_combine), torch.empty_like(ns.lse)
    mla.decode_attn(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, ns.max_len,
                    ns.softmax_scale, vc_ws, lse_ws, split_rows, ws)
    mla.decode_attn_noalloc(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, ns.max_len,
                            ns.softmax_scale, ns.v_combine, ns.lse, split_rows)
    torch.cuda.synchronize()
    return host(vc_ws), host(lse_ws), host(ns.v_combine), host(ns.lse)


def oracle(case):
    q64 = O.widen(case.q_abs, case.dims.cache_dtype)
    vc, lse, _ = O.attention_latent(case.dims, q64, case.pool, case.table, case.lens,
                                    float(np.float32(case.softmax_scale)))
    return vc, lse


@pytest.mark.parametrize("split_rows", [0, 128])
def test_noalloc_matches_workspace_call_twice(split_rows):
    first = S.make_case(4, lens=[3000, 1500, 700, 5000, 64], paged=True, seed=31)
    second = S.make_case(4, lens=[300, 129], paged=True, seed=32)
    for i, case in enumerate((first, second)):
        print(f"[noalloc] call {i + 1}: lens {case.lens.tolist()} split_rows {split_rows}",
              flush=True)
        r, s = mla.attn_plan(D.dims_of(case), case.batch, int(case.lens.max()), split_rows)
        assert s > 1, "the case must use split partials"
        vc_ws, lse_ws, vc, lse = both(case, split_rows)
        assert np.array_equal(vc, vc_ws) and np.array_equal(lse, lse_ws), f"call {i + 1}"
        rvc, rlse = oracle(case)
        attn_check(vc, lse, rvc, rlse, f"no-alloc call {i + 1}")


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    # one 32768-row sequence in 64-row splits: 512 partials of 129 KB > 48 MiB
    case = S.make_case(4, lens=[64], seed=33)
    ns = D.stage(case)
    need = mla.workspace_bytes(ns.dims, 1, 32768, 64)
    assert need > mla.MLA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MLAError) as e:
        mla.decode_attn_noalloc(ns.dims, ns.q_abs_given, ns.pool, ns.table, ns.lens, 32768,
                                ns.softmax_scale, ns.v_combine, ns.lse, 64)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
