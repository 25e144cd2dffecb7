"""Comparison helpers shared by the parity tests (not a test module).

Two kinds of check are applied to GPU results against the fp64 oracle:

* the stated bars: fp32 caches max |gpu - ref| <= 1e-4; bf16 caches
  |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise;
* for decode attention, non-replacing checks that a missing part of the work
  cannot pass.  At 131072 rows the stated bar leaves lse about 0.15 of slack,
  while dropping one 32-row tile moves lse by only ~32 / 131072 = 2.4e-4, so
  per query every head's lse must agree to 1e-4 + 1e-6 |lse| and the largest
  v_combine error must stay under 4e-3 of the query's largest |v_combine|.
  The kernel's own error budget sits inside both: its lse is fp32 over exact
  bf16 products (no rounding of p enters the denominator), and the only
  rounding in v_combine is p to bf16 as an MFMA operand (at most 2^-9 relative
  per term) plus the fp16 split partial (2^-11): at most 2.44e-3 of |v| where
  one row dominates a short query, ~1.1e-3 rms where many rows average out.  ``tests/test_parity_checker.py`` shows on the CPU that these checks
  reject the oracle's own result with one tile or one split removed at 131072
  rows and accept a model of the kernel's rounding.
"""
import numpy as np

ATOL_BF16, RTOL_BF16 = 2e-2, 1e-2
LSE_ATOL, LSE_RTOL = 1e-4, 1e-6
VC_REL = 4e-3


def close_bf16(got, ref, what):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, what
    with np.errstate(invalid="ignore"):
        ok = (got == ref) | (np.abs(got - ref) <= ATOL_BF16 + RTOL_BF16 * np.abs(ref))
    bad = ~ok  # equal infinities (the lse of an empty query) match; NaN never does
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, "
                           f"max abs err {np.nanmax(np.abs(got - ref)):.3e}")


def close_f32(got, ref, what):
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    err = np.max(np.abs(got - ref))
    assert err <= 1e-4, f"{what}: max abs err {err:.3e} > 1e-4"
    assert err <= 1e-3 * np.max(np.abs(ref)) + 1e-12, f"{what}: err {err:.3e} vs scale"


def attn_tight(vc, lse, rvc, rlse, what):
    """Per-query checks on decode attention outputs [Q, H, C] and [Q, H].

    An empty query (oracle lse = -inf) must give v_combine = 0 and lse = -inf;
    otherwise every lse within LSE_ATOL + LSE_RTOL |lse| and the largest
    v_combine error within VC_REL of the query's largest |v_combine|."""
    vc, lse = np.asarray(vc, dtype=np.float64), np.asarray(lse, dtype=np.float64)
    rvc, rlse = np.asarray(rvc, dtype=np.float64), np.asarray(rlse, dtype=np.float64)
    assert vc.shape == rvc.shape and lse.shape == rlse.shape, what
    for q in range(rlse.shape[0]):
        empty = np.isneginf(rlse[q])
        if empty.all():
            assert np.isneginf(lse[q]).all() and np.all(vc[q] == 0), f"{what}: query {q} empty"
            continue
        assert not empty.any(), f"{what}: query {q} partly empty in the oracle"
        dl = np.abs(lse[q] - rlse[q])
        lim = LSE_ATOL + LSE_RTOL * np.abs(rlse[q])
        assert np.all(dl <= lim), (f"{what}: query {q} lse off by up to {np.nanmax(dl):.3e} "
                                   f"({int(np.sum(~(dl <= lim)))} heads past {LSE_ATOL:g})")
        dv = np.nanmax(np.abs(vc[q] - rvc[q])) if np.isfinite(vc[q]).all() else np.inf
        scale = np.max(np.abs(rvc[q]))
        assert dv <= VC_REL * scale + 1e-30, (f"{what}: query {q} v_combine off by {dv:.3e}, "
                                              f"{dv / scale:.2e} of max|ref|")


def attn_check(vc, lse, rvc, rlse, what):
    """The stated bf16 bar and the tight per-query checks together."""
    close_bf16(vc, rvc, f"{what} v_combine")
    close_bf16(lse, rlse, f"{what} lse")
    attn_tight(vc, lse, rvc, rlse, what)
