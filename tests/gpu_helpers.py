"""Shared helpers for the GPU parity tests (host <-> device copies, error
measures, tolerances).  Imported only by tests marked ``gpu``."""
import numpy as np
import torch

# Tolerances for floating-point results.
TOL_F32_ABS = 1e-4          # fp32 weights: max-abs error
TOL_F16_REL = 2e-2          # fp16 weights, fp32 accumulate: normwise relative error (the contract)
# A tighter bound every fp16 output also meets.  Within one step, fp32
# accumulation over d terms of fp16 weights is off the float64 result by
# about sqrt(d) * 2^-24 of the dot products' scale (measured: ~2e-7).  Over
# several steps each side rounds its own K/V to fp16, and an entry whose fp32
# and float64 values straddle a rounding boundary differs by one fp16 unit
# (2^-11 relative); through attention and W^O that moves later outputs by
# up to ~2e-5 of max|out| (measured at d = 9216).  A dropped bias (b2 ~
# N(0, 0.02^2) against |out| ~ 4: ~1e-2) or one missing fc2 row (~1e-2) is
# far above the bound.
TOL_F16_TIGHT = 1e-4


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def normwise(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    den = np.abs(want).max()
    return float(np.abs(got - want).max() / (den if den > 0 else 1.0))


def maxabs(got, want):
    return float(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)).max())


def check_close(got, want, wdt: str, what: str = "", tight: float = TOL_F16_TIGHT):
    """fp32 path: max-abs <= 1e-4; fp16 weights: normwise relative <= 2e-2
    (the contract) and <= ``tight``, i.e. every element within
    tight * max|want| of the oracle."""
    if wdt == "f32":
        e = maxabs(got, want)
        assert e <= TOL_F32_ABS, f"{what}: max-abs {e:.3e}"
    else:
        e = normwise(got, want)
        assert e <= TOL_F16_REL, f"{what}: normwise {e:.3e}"
        assert e <= tight, f"{what}: normwise {e:.3e} above the tight bound {tight:.0e}"
    return e


def f16_kv_ok(got, want, rel=1e-5):
    """Both sides round their own fp32 / fp64 value to fp16: entries may differ
    by one fp16 unit in the last place, or, near zero where that unit is
    smaller than the accumulation error, by rel * max|want|."""
    g = np.asarray(got, np.float16).astype(np.float64)
    w = np.asarray(want, np.float16)
    ulp = np.spacing(np.abs(w)).astype(np.float64)
    tol = ulp + rel * (np.abs(w).max() if w.size else 0.0)
    bad = np.abs(g - w.astype(np.float64)) > tol
    return not bool(bad.any()), int(bad.sum())


def upload(W: dict) -> dict:
    return {k: dev(v) for k, v in W.items()}


def assert_selection_close(got_idx, want_idx, scores, k, tol, what=""):
    """The two selections may differ only in entries whose (oracle) score is
    within tol of the k-th largest score: a swap across the boundary that
    rounding of the scores can cause, and nothing else."""
    s = np.asarray(scores, np.float64)
    got, want = set(np.asarray(got_idx).tolist()), set(np.asarray(want_idx).tolist())
    assert len(got) == len(want) == k, f"{what}: sizes {len(got)} {len(want)} (k={k})"
    if got == want:
        return 0
    kth = np.sort(s)[::-1][k - 1]
    off = [j for j in got ^ want if not abs(s[j] - kth) <= tol]
    assert not off, f"{what}: entries {off[:8]} differ beyond the rounding margin"
    return len(got ^ want)


def selection_margin(scores, k):
    """Gap between the k-th and (k+1)-th largest score (inf when k == 0 or n)."""
    s = np.sort(np.asarray(scores, np.float64))[::-1]
    if k <= 0 or k >= s.size:
        return np.inf
    return float(s[k - 1] - s[k])
