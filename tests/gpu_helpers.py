"""Shared helpers for the GPU parity tests (host <-> device copies, error
measures, tolerances).  Imported only by tests marked ``gpu``."""
import numpy as np
import torch

# Tolerances for floating-point results.
TOL_F32_ABS = 1e-4          # fp32 weights: max-abs error
TOL_F16_REL = 2e-2          # fp16 weights, fp32 accumulate: normwise relative error


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


def check_close(got, want, wdt: str, what: str = ""):
    """fp32 path: max-abs <= 1e-4; fp16 weights: normwise relative <= 2e-2."""
    if wdt == "f32":
        e = maxabs(got, want)
        assert e <= TOL_F32_ABS, f"{what}: max-abs {e:.3e}"
    else:
        e = normwise(got, want)
        assert e <= TOL_F16_REL, f"{what}: normwise {e:.3e}"
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


def selection_margin(scores, k):
    """Gap between the k-th and (k+1)-th largest score (inf when k == 0 or n)."""
    s = np.sort(np.asarray(scores, np.float64))[::-1]
    if k <= 0 or k >= s.size:
        return np.inf
    return float(s[k - 1] - s[k])
