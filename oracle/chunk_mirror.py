"""The chunk-form algebra of the pages, in fp64 numpy (TEST INFRASTRUCTURE ONLY).

This is a second, independent route to the same result as the token recurrence:
it applies the chunkwise rewrite exactly as the pages write it, with library
matrix products and a library triangular inverse, and no blocking or fusion of
its own.  Tests require it to agree with the recurrence to ~1e-12, which pins
the chunk algebra the GPU kernels are built on, and its per-chunk intermediates
(the inverse, W, U, V_new) are checked against the pages' closed forms.

Notation (all per chunk of C tokens, rows r = 1..C):
  g_r        inclusive prefix sum of log alpha from the chunk start; Gamma = exp(g)
  X<- = X * Gamma,  X-> = X / Gamma    (row-wise, per key channel)
  M  = lower-triangular ones (with the diagonal), M_1 = M - I (strictly lower)

KDA form ("Kimi Delta Attention backward" notes, forward recap):
  Xt = I + Diag(beta)(K<- K->^T * M_1),  At = Xt^-1
  W  = At Diag(beta) K<-,   U = At Diag(beta) V
  V_new = U - W S^T
  S  <- S Diag(gamma_C) + V_new^T K-> Diag(gamma_C)
  O  = Q<- S^T + (Q<- K->^T * M) V_new            (S is the state entering the chunk)

Gated DPLR form ("Diagonal Plus Low Rank", section 2, matrix form), with the write
term scaled by beta (V := Diag(beta) V):
  E  = (I + (B<- A->^T * M_1))^-1,   W = E B<-,   Cm = -E (B<- K->^T * M_1) V
  N  = Cm - W S^T
  S  <- S Diag(gamma_C) + V^T K-> Diag(gamma_C) + N^T A-> Diag(gamma_C)
  O  = Q<- S^T + (Q<- K->^T * M) V + (Q<- A->^T * M) N
"""
from __future__ import annotations

import numpy as np
import scipy.linalg


def _g(log_alpha_rows, n, dk):
    """Inclusive in-chunk prefix sum of log alpha, as an [n, dk] array."""
    if log_alpha_rows is None:
        return np.zeros((n, dk))
    la = np.asarray(log_alpha_rows, dtype=np.float64)
    if la.ndim == 1:
        la = np.repeat(la[:, None], dk, axis=1)
    return np.cumsum(la, axis=0)


def _unit_lower_inverse(X):
    return scipy.linalg.solve_triangular(X, np.eye(X.shape[0]), lower=True, unit_diagonal=True)


def chunk_forward(q, k, v, beta, log_alpha=None, a=None, b=None, S0=None, cu_seqlens=None,
                  C: int = 64, record: bool = False):
    """Chunkwise forward in fp64.  Same argument conventions as ``oracle.recurrence``.

    Returns (O, S_final, records) where records (if ``record``) is a list over
    chains of lists over chunks of dicts with the chunk intermediates.
    """
    q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
    la = None if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)
    a = None if a is None else np.asarray(a, dtype=np.float64)
    b = None if b is None else np.asarray(b, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flat = lambda x: None if x is None else x.reshape((B * T,) + x.shape[2:])
    qf, kf, vf, bf, laf, af, bbf = map(flat, (q, k, v, beta, la, a, b))
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = list(np.asarray(cu_seqlens).tolist())
        bounds = [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    N = len(bounds)
    O = np.zeros((B * T, H, dv))
    Sf = np.zeros((N, H, dv, dk))
    records = []
    M = np.tril(np.ones((C, C)))
    M1 = np.tril(np.ones((C, C)), -1)
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            rec = []
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                m = c1 - c0
                Mm, M1m = M[:m, :m], M1[:m, :m]
                Q, K, V = qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, h]
                bet = bf[c0:c1, h]
                g = _g(None if laf is None else laf[c0:c1, h], m, dk)
                Gam = np.exp(g)
                gC = Gam[-1]
                Ql, Kl, Kr = Q * Gam, K * Gam, K / Gam
                if af is None:
                    Xt = np.eye(m) + bet[:, None] * ((Kl @ Kr.T) * M1m)
                    At = _unit_lower_inverse(Xt)
                    W = At @ (bet[:, None] * Kl)
                    U = At @ (bet[:, None] * V)
                    Vn = U - W @ S.T
                    Oc = Ql @ S.T + ((Ql @ Kr.T) * Mm) @ Vn
                    S = S * gC[None, :] + (Vn.T @ Kr) * gC[None, :]
                    if record:
                        rec.append(dict(A=At, W=W, U=U, V_new=Vn))
                else:
                    A_, B_ = af[c0:c1, h], bbf[c0:c1, h]
                    Ar, Bl = A_ / Gam, B_ * Gam
                    Vb = bet[:, None] * V
                    E = _unit_lower_inverse(np.eye(m) + (Bl @ Ar.T) * M1m)
                    W = E @ Bl
                    Cm = -E @ (((Bl @ Kr.T) * M1m) @ Vb)
                    Nn = Cm - W @ S.T
                    Oc = Ql @ S.T + ((Ql @ Kr.T) * Mm) @ Vb + ((Ql @ Ar.T) * Mm) @ Nn
                    S = (S + Vb.T @ Kr + Nn.T @ Ar) * gC[None, :]
                    if record:
                        rec.append(dict(A=E, W=W, C=Cm, N=Nn))
                O[c0:c1, h] = Oc
            Sf[n, h] = S
            records.append(rec)
    return O.reshape(B, T, H, dv), Sf, records
