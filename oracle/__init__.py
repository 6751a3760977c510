"""CPU oracle for the gated delta-rule forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  Nothing here is imported by, or imports,
the GPU library; inputs arrive as plain numpy arrays.

* ``recurrence``        -- the definition: fp64 token-by-token recurrence (C, OpenMP),
                           built from ``gdr_ref.c``.
* ``recurrence_bwd``    -- its gradients: reverse-mode differentiation of the same
                           recurrence, written out by hand (``gdr_ref_bwd.c``).
* ``spectral_norm_rank1`` -- closed form of ||I - eta k j^T||_2 for unit k, j
                           ("How to make GDN2 more stable", eq. 4).
* ``chunk_mirror``      -- the chunk-form algebra of the pages in fp64 numpy, used to
                           pin the chunk rewrite against the definition.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        # GDR_ORACLE_LIB names another build of the same sources (the sanitizer build
        # of the CPU test suite); by default the one oracle/build.py makes
        path = os.environ.get("GDR_ORACLE_LIB") or os.path.join(_HERE, "libgdr_ref.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdr_ref_fwd.restype = I
        lib.gdr_ref_fwd.argtypes = [P, P, P, P, P, P, I, I, P, P, P, P, P, I, I, I, I, I, I, P, I, I]
        lib.gdr_ref_bwd.restype = I
        lib.gdr_ref_bwd.argtypes = [P] * 6 + [I] + [P] * 12 + [P, I, I, I, I, I, I, P, I, I]
        lib.gdr_ref_max_threads.restype = I
        lib.gdr_ref_max_threads.argtypes = []
        _LIB = lib
    return _LIB


def max_threads() -> int:
    return int(_lib().gdr_ref_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def recurrence(q, k, v, beta, log_alpha=None, a=None, b=None, S0=None, cu_seqlens=None,
               chains=None, n_threads: int = 0, want_state: bool = True, clip: bool = False):
    """Run the fp64 recurrence.

    clip: spectral clipping of the gate, alpha_t <- min(alpha_t, 1/||I - b_t a_t^T||_2)
    per token ("How to make GDN2 more stable", eq. 7; also without a gate, where
    alpha_t = 1/rho_t).

    q, k, a, b: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H];
    log_alpha: None (no gate), [B, T, H] (head gate) or [B, T, H, dk] (channel gate);
    S0: None or [N, H, dv, dk]; cu_seqlens: None or int [N+1] (then B == 1).
    chains: None (all) or a list of (sequence, head) pairs to compute; the other
    entries of O and S_final are left as NaN.
    Returns (O [B, T, H, dv], S_final [N, H, dv, dk] or None), float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    a, b, log_alpha, S0 = _f64(a), _f64(b), _f64(log_alpha), _f64(S0)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == q.shape[:3] and beta.shape == q.shape[:3]
    if log_alpha is None:
        gate = 0
    elif log_alpha.ndim == 3:
        gate = 1
        assert log_alpha.shape == q.shape[:3]
    else:
        gate = 2
        assert log_alpha.shape == q.shape
    if a is not None:
        assert a.shape == q.shape and b.shape == q.shape
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.size - 1
    else:
        N = B
    if S0 is not None:
        assert S0.shape == (N, H, dv, dk)
    O = np.full((B, T, H, dv), np.nan)
    Sf = np.full((N, H, dv, dk), np.nan) if want_state else None
    ch = None
    n_ch = 0
    if chains is not None:
        ch = np.ascontiguousarray(np.asarray(chains, dtype=np.int32).reshape(-1, 2))
        n_ch = ch.shape[0]
    rc = _lib().gdr_ref_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), gate,
                            int(bool(clip)), _ptr(beta), _ptr(S0), _ptr(O), _ptr(Sf), _ptr(cu), N,
                            B, H, T, dk, dv, _ptr(ch), n_ch, int(n_threads))
    if rc != 0:
        raise ValueError(f"gdr_ref_fwd rejected its arguments (code {rc})")
    return O, Sf


def recurrence_bwd(q, k, v, beta, dO, log_alpha=None, a=None, b=None, S0=None, dS_final=None,
                   cu_seqlens=None, chains=None, n_threads: int = 0):
    """Gradients of L = <dO, O> + <dS_final, S_final> for the fp64 recurrence.

    Shapes as in ``recurrence``; dO has O's shape, dS_final S_final's (None: zero).
    Returns a dict with dq, dk, dv, dbeta, dS0 and, when given, da, db and
    dlog_alpha (same shapes as the inputs).  Entries of chains that are not
    computed are NaN.
    """
    q, k, v, beta, dO = _f64(q), _f64(k), _f64(v), _f64(beta), _f64(dO)
    a, b, log_alpha, S0, dSf = _f64(a), _f64(b), _f64(log_alpha), _f64(S0), _f64(dS_final)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert dO.shape == v.shape
    gate = 0 if log_alpha is None else (1 if log_alpha.ndim == 3 else 2)
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.size - 1
    else:
        N = B
    if S0 is not None:
        assert S0.shape == (N, H, dv, dk)
    if dSf is not None:
        assert dSf.shape == (N, H, dv, dk)
    g = {"dq": np.full(q.shape, np.nan), "dk": np.full(q.shape, np.nan),
         "dv": np.full(v.shape, np.nan), "dbeta": np.full(beta.shape, np.nan),
         "dS0": np.full((N, H, dv, dk), np.nan)}
    if a is not None:
        g["da"] = np.full(q.shape, np.nan)
        g["db"] = np.full(q.shape, np.nan)
    if log_alpha is not None:
        g["dlog_alpha"] = np.full(log_alpha.shape, np.nan)
    ch = None
    n_ch = 0
    if chains is not None:
        ch = np.ascontiguousarray(np.asarray(chains, dtype=np.int32).reshape(-1, 2))
        n_ch = ch.shape[0]
    rc = _lib().gdr_ref_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), gate,
                            _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dSf), _ptr(g["dq"]),
                            _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g.get("da")), _ptr(g.get("db")),
                            _ptr(g.get("dlog_alpha")), _ptr(g["dbeta"]), _ptr(g["dS0"]),
                            _ptr(cu), N, B, H, T, dk, dv, _ptr(ch), n_ch, int(n_threads))
    if rc != 0:
        raise ValueError(f"gdr_ref_bwd rejected its arguments (code {rc})")
    return g


def spectral_norm_rank1(eta: float, k: np.ndarray, j: np.ndarray) -> float:
    """||I - eta k j^T||_2 for unit vectors k, j: (eta + sqrt(eta^2 - 4 eta k.j + 4)) / 2.

    "How to make GDN2 more stable", eq. 4 (proved there by reducing to the 2x2
    block on span{k, j} and using ||B||_F^2 and |det B|, eqs. 8-12).
    """
    c = float(np.dot(k, j))
    return 0.5 * (eta + np.sqrt(eta * eta - 4.0 * eta * c + 4.0))
