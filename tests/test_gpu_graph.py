"""The decode step captured as one HIP graph.

The benchmark replays the whole step as one graph (append and absorb on two
streams, then attention and out_proj).  Every replay must reproduce the eager
step bit for bit; between replays the outputs are overwritten by the
program's own eager work and the device is synchronised, so a stale result
cannot pass.  The eager step itself is checked against the fp64 oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_synth as S
from mla_synth import device as D
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

OUTPUTS = ("q_abs", "v_combine", "lse", "out")


def host(x):
    a = x.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def scramble(ns):
    ns.q_abs.fill_(0x7fc1)          # bf16 NaN bits
    ns.v_combine.fill_(float("nan"))
    ns.lse.fill_(float("nan"))
    ns.out.fill_(float("nan"))


@pytest.mark.parametrize("cfg,kw", [(5, dict(batch=4, lens=[300, 1100, 64, 700])),
                                    (3, dict(batch=3, lens=[1024, 77, 2049]))])
def test_graph_replays_match_the_eager_step(cfg, kw):
    case = S.make_case(cfg, **kw)
    ns = D.stage(case)
    step = D.GraphStep(case, ns)
    step.run(eager=True)
    torch.cuda.synchronize()
    ref = {k: host(getattr(ns, k)).copy() for k in OUTPUTS}
    pool = host(ns.pool).copy()

    res = O.decode_step(case)
    got, want = ref["v_combine"].astype(np.float64), res["v_combine"]
    assert np.all(np.abs(got - want) <= 2e-2 + 1e-2 * np.abs(want))
    got, want = ref["out"].astype(np.float64), res["out"].reshape(case.batch, -1)
    assert np.all(np.abs(got - want) <= 2e-2 + 1e-2 * np.abs(want))

    step.capture()
    for replay in range(4):
        scramble(ns)
        torch.cuda.synchronize()
        step.run()
        torch.cuda.synchronize()
        for k in OUTPUTS:
            assert np.array_equal(host(getattr(ns, k)).view(np.uint8), ref[k].view(np.uint8)), \
                f"replay {replay}: {k} differs from the eager step"
        assert np.array_equal(host(ns.pool).view(np.uint8), pool.view(np.uint8)), \
            f"replay {replay}: cache pool differs"
        # eager work of the program between replays
        torch.cuda.synchronize()
        _ = (ns.v_combine * 2).sum().item()
