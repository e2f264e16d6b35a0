"""Tolerance rule for bf16 outputs and gradients.  TEST INFRASTRUCTURE ONLY.

The bar (relative Frobenius error <= 5e-3, max elementwise error <= 1e-2 of
the output RMS) is the one stated for this layer.  Reading R10:
the elementwise bound is taken as

    |got - ref| <= max_tol * RMS(ref) + 0.5 * ulp_bf16(max(|ref|, |got|))

because a correctly rounded bf16 output already sits up to half a bf16 ulp
from the exact value; at the largest outputs (|y| > 4 RMS) that half ulp alone
exceeds 1e-2 RMS.  Integer and byte results are compared for equality instead.
"""

from __future__ import annotations

import numpy as np


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (0 where x == 0)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)               # a = f * 2**e, f in [0.5, 1)
    u = np.ldexp(1.0, e - 8)         # 8 significant bits in bf16
    return np.where(a > 0, u, 0.0)


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def max_excess(got, ref, max_tol: float = 1e-2) -> float:
    """Largest |got-ref| minus the elementwise allowance, in units of RMS(ref).

    <= 0 means every element is within the bound.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    allow = max_tol * rms + 0.5 * ulp_bf16(np.maximum(np.abs(ref), np.abs(got)))
    excess = np.abs(got - ref) - allow
    return float(excess.max() / rms) if rms > 0 else float(excess.max())


def check_close(got, ref, rel_tol: float = 5e-3, max_tol: float = 1e-2):
    """(ok, info) for the bf16 tolerance rule above."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        return False, {"error": f"shape {got.shape} != {ref.shape}"}
    if not np.all(np.isfinite(got)):
        return False, {"error": "non-finite output"}
    rf = rel_fro(got, ref)
    mx = max_excess(got, ref, max_tol)
    return (rf <= rel_tol and mx <= 0.0), {"rel_fro": rf, "max_excess_rms": mx}
