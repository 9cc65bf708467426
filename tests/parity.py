"""Element-by-element comparison of fp32 GPU results with fp64 oracle results.

Tolerance: |gpu - ref| <= atol + rtol * |ref| for finite ref (atol 1e-5,
rtol 2e-6 for the reductions; rtol 5e-4 for the conv chain).  A non-finite
ref demands the same class from the GPU: -inf == -inf, +inf == +inf, NaN ==
NaN.
"""
from __future__ import annotations

import numpy as np

ATOL = 1e-5
RTOL = 2e-6
RTOL_CHAIN = 5e-4


def compare(gpu, ref, atol=ATOL, rtol=RTOL, what=""):
    gpu = np.asarray(gpu, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    fin = np.isfinite(ref)
    bad_class = np.zeros(ref.shape, dtype=bool)
    nan = np.isnan(ref)
    bad_class[nan] = ~np.isnan(gpu[nan])
    inf = np.isinf(ref)
    bad_class[inf] = gpu[inf] != ref[inf]
    err = np.zeros(ref.shape)
    err[fin] = np.abs(gpu[fin] - ref[fin])
    tol = atol + rtol * np.abs(np.where(fin, ref, 0.0))
    bad_val = fin & ~(err <= tol)          # NaN gpu on a finite ref fails here
    nbad = int(bad_class.sum() + bad_val.sum())
    rel = np.zeros(ref.shape)
    rel[fin] = err[fin] / np.maximum(np.abs(ref[fin]), 1e-30)
    summary = {
        "n": int(ref.size),
        "max_abs": float(err[fin].max()) if fin.any() else 0.0,
        "max_rel": float(rel[fin].max()) if fin.any() else 0.0,
        "violations": nbad,
    }
    if nbad:
        idx = np.flatnonzero(bad_class | bad_val)[:8]
        detail = ", ".join(f"[{i}] gpu={gpu[i]!r} ref={ref[i]!r}" for i in idx)
        raise AssertionError(f"{what}: {nbad} of {ref.size} outside tolerance; {detail}; "
                             f"{summary}")
    return summary
