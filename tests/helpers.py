"""Glue between the seeded input generators and the CPU oracle (tests only)."""
import numpy as np
import torch

import oracle


def f64(t):
    return None if t is None else t.to(torch.float64).numpy()


def oracle_of(P, chains=None, n_threads=0):
    """Run the fp64 recurrence on a Problem's exact input values."""
    return oracle.recurrence(f64(P.q), f64(P.k), f64(P.v), f64(P.beta), log_alpha=f64(P.log_alpha),
                             a=f64(P.a), b=f64(P.b), S0=f64(P.S0),
                             cu_seqlens=None if P.cu_seqlens is None else P.cu_seqlens.numpy(),
                             chains=chains, n_threads=n_threads)


def rel_err(x, ref):
    """max|x - ref| / max|ref| over all finite reference entries."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.isfinite(ref)
    denom = np.max(np.abs(ref[m])) if m.any() else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(x[m]))) if m.any() else 0.0
    return float(np.max(np.abs(x[m] - ref[m])) / denom)
