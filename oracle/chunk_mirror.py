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


def chunk_bwd(q, k, v, beta, dO, log_alpha=None, S0=None, dS_final=None, cu_seqlens=None,
              C: int = 64, a=None, b=None):
    """Gradients of <dO, O> + <dS_final, S_final> by the chunk-form backward of the
    "Kimi Delta Attention backward" notes (KDA form: a = k, b = beta k), fp64; with a and
    b given, by the gated DPLR backward of the "Diagonal Plus Low Rank" notes (section 3),
    see ``_chunk_bwd_dplr``.

    Notation as above, with the notes' state convention S_[t] = S_[t-1] Diag(gamma_C)
    + V_new^T K-> Diag(gamma_C).  Per chunk, with dS = dL/dS_[t] at its end:
      dU = dV_new = K-> Diag(gamma_C) dS^T + (Q<- K->^T * M)^T dO
      dW = -dU S_[t-1]
      dQ<- = dO S_[t-1] + (dO V_new^T * M) K->,             dQ = dQ<- * Gamma
      dV = Diag(beta) At^T dU
      dAt = dW K<-^T Diag(beta) + dU V^T Diag(beta),          dXt = -At^T dAt At^T
      dK<- = Diag(beta) At^T dW + (Diag(beta) dXt * M_1) K->
      dK-> = V_new dS Diag(gamma_C) + (dO V_new^T * M)^T Q<- + (Diag(beta) dXt * M_1)^T K<-
      dK = dK<- * Gamma + dK-> / Gamma
      dbeta = diag(At^T dW K<-^T + At^T dU V^T + dXt (K<- K->^T * M_1)^T)
      dlog Gamma = dQ * Q + (dK<- * Gamma) * K - (dK-> / Gamma) * K, plus
                   diag(S_[t]^T dS) on the chunk's last row
      dS_[t-1] = dS Diag(gamma_C) + dO^T Q<- - dU^T W
    and dlog alpha is the suffix sum of dlog Gamma inside the chunk (g is the prefix
    sum of log alpha), summed over channels for a head gate.  beta is not divided
    out: the notes' diag(At^T dAt) / beta is written as the diagonal of the first
    line of their derivation, which is the same number and is defined at beta = 0.
    """
    if a is not None:
        return _chunk_bwd_dplr(q, k, v, beta, dO, log_alpha, a, b, S0, dS_final, cu_seqlens, C)
    q, k, v, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, dO))
    la = None if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flat = lambda x: None if x is None else x.reshape((B * T,) + x.shape[2:])
    qf, kf, vf, bf, laf, dOf = map(flat, (q, k, v, beta, la, dO))
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = list(np.asarray(cu_seqlens).tolist())
        bounds = [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    N = len(bounds)
    out = {"dq": np.zeros((B * T, H, dk)), "dk": np.zeros((B * T, H, dk)),
           "dv": np.zeros((B * T, H, dv)), "dbeta": np.zeros((B * T, H)),
           "dS0": np.zeros((N, H, dv, dk))}
    if la is not None:
        out["dlog_alpha"] = np.zeros((B * T,) + la.shape[2:])
    M = np.tril(np.ones((C, C)))
    M1 = np.tril(np.ones((C, C)), -1)
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            # forward over the chunks, keeping what the backward needs
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            chunks = []
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                m = c1 - c0
                Q, K, V, dOc = qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, h], dOf[c0:c1, h]
                bet = bf[c0:c1, h]
                Gam = np.exp(_g(None if laf is None else laf[c0:c1, h], m, dk))
                gC = Gam[-1]
                Ql, Kl, Kr = Q * Gam, K * Gam, K / Gam
                At = _unit_lower_inverse(np.eye(m) + bet[:, None] * ((Kl @ Kr.T) * M1[:m, :m]))
                W = At @ (bet[:, None] * Kl)
                U = At @ (bet[:, None] * V)
                Vn = U - W @ S.T
                Sn = (S + Vn.T @ Kr) * gC[None, :]
                chunks.append(dict(c0=c0, c1=c1, m=m, Q=Q, K=K, V=V, dO=dOc, bet=bet, Gam=Gam,
                                   gC=gC, Ql=Ql, Kl=Kl, Kr=Kr, At=At, W=W, Vn=Vn, Sp=S, Sn=Sn))
                S = Sn
            dS = np.zeros((dv, dk)) if dS_final is None else np.array(dS_final[n, h], dtype=np.float64)
            for ch in reversed(chunks):
                m = ch["m"]
                Mm, M1m = M[:m, :m], M1[:m, :m]
                Ql, Kl, Kr, Gam, gC = ch["Ql"], ch["Kl"], ch["Kr"], ch["Gam"], ch["gC"]
                At, W, Vn, Sp, V, G, bet = ch["At"], ch["W"], ch["Vn"], ch["Sp"], ch["V"], ch["dO"], ch["bet"]
                dU = (Kr * gC[None, :]) @ dS.T + ((Ql @ Kr.T) * Mm).T @ G
                dW = -dU @ Sp
                dOV = (G @ Vn.T) * Mm
                dQl = G @ Sp + dOV @ Kr
                dV = bet[:, None] * (At.T @ dU)
                dAt = (dW @ Kl.T + dU @ V.T) * bet[None, :]
                dXt = -At.T @ dAt @ At.T
                dXm = bet[:, None] * dXt * M1m
                dKl = bet[:, None] * (At.T @ dW) + dXm @ Kr
                dKr = Vn @ dS * gC[None, :] + dOV.T @ Ql + dXm.T @ Kl
                dbeta = np.diag(At.T @ dW @ Kl.T + At.T @ dU @ V.T + dXt @ ((Kl @ Kr.T) * M1m).T)
                dlg = dQl * Ql + dKl * Kl - dKr * Kr
                dlg[-1] += np.sum(ch["Sn"] * dS, axis=0)
                sl = slice(ch["c0"], ch["c1"])
                out["dq"][sl, h] = dQl * Gam
                out["dk"][sl, h] = dKl * Gam + dKr / Gam
                out["dv"][sl, h] = dV
                out["dbeta"][sl, h] = dbeta
                if la is not None:
                    suffix = np.cumsum(dlg[::-1], axis=0)[::-1]
                    out["dlog_alpha"][sl, h] = suffix if la.ndim == 4 else suffix.sum(axis=1)
                dS = dS * gC[None, :] + G.T @ Ql - dU.T @ W
            out["dS0"][n, h] = dS
    res = {key: val.reshape((B, T) + val.shape[1:]) for key, val in out.items() if key != "dS0"}
    res["dS0"] = out["dS0"]
    return res


def _chunk_bwd_dplr(q, k, v, beta, dO, log_alpha, a, b, S0, dS_final, cu_seqlens, C):
    """Gated DPLR backward ("Diagonal Plus Low Rank" notes, section 3), fp64, with the
    write term scaled by beta (V' = Diag(beta) V, the notes' V).  Per chunk, with
    F = I + (B<- A->^T * M_1), E = F^-1, W = E B<-, Cm = -E (B<- K->^T * M_1) V',
    N = Cm - W S_p^T (the notes' V_2), and dS = dL/dS_[t]:
      dN = dCm = A-> Diag(gamma_C) dS^T + (Q<- A->^T * M)^T dO
      dV'1 = K-> Diag(gamma_C) dS^T + (Q<- K->^T * M)^T dO
      dW = -dN S_p
      dE = -dCm V'^T (B<- K->^T * M_1)^T + dW B<-^T,    dF = -E^T dE E^T
      dQ<- = dO S_p + (dO V'^T * M) K-> + (dO N^T * M) A->
      dB<- = E^T dW - (E^T dCm V'^T * M_1) K-> + (dF * M_1) A->
      dK-> = (dO V'^T * M)^T Q<- - (E^T dCm V'^T * M_1)^T B<- + V' dS Diag(gamma_C)
      dA-> = (dO N^T * M)^T Q<- + (dF * M_1)^T B<- + N dS Diag(gamma_C)
      dV' = dV'1 - (B<- K->^T * M_1)^T E^T dCm,          dV = Diag(beta) dV', dbeta = rowsum(dV' * V)
      dlog Gamma = dQ<- Q<- + dB<- B<- - dK-> K-> - dA-> A->, plus diag(S_[t]^T dS) on the last row
      dS_[t-1] = dS Diag(gamma_C) + dO^T Q<- - dCm^T W
    The notes write dW with S_[t] and list dK->, dA-> without their state-update terms;
    the forward definitions fix both (N uses S_[t-1]; V'^T K-> Diag(gamma_C) and
    N^T A-> Diag(gamma_C) enter the state), and the pins against the token reverse pass
    confirm that reading.
    """
    q, k, v, beta, dO, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, dO, a, b))
    la = None if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flat = lambda x: None if x is None else x.reshape((B * T,) + x.shape[2:])
    qf, kf, vf, bf, laf, dOf, af, bbf = map(flat, (q, k, v, beta, la, dO, a, b))
    if cu_seqlens is None:
        bounds = [(n * T, (n + 1) * T) for n in range(B)]
    else:
        cu = list(np.asarray(cu_seqlens).tolist())
        bounds = [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    N_ = len(bounds)
    out = {key: np.zeros((B * T, H, dk)) for key in ("dq", "dk", "da", "db")}
    out["dv"] = np.zeros((B * T, H, dv))
    out["dbeta"] = np.zeros((B * T, H))
    out["dS0"] = np.zeros((N_, H, dv, dk))
    if la is not None:
        out["dlog_alpha"] = np.zeros((B * T,) + la.shape[2:])
    M = np.tril(np.ones((C, C)))
    M1 = np.tril(np.ones((C, C)), -1)
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            chunks = []
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                m = c1 - c0
                Mm, M1m = M[:m, :m], M1[:m, :m]
                Q, K, A_, B_ = qf[c0:c1, h], kf[c0:c1, h], af[c0:c1, h], bbf[c0:c1, h]
                bet = bf[c0:c1, h]
                Vp = bet[:, None] * vf[c0:c1, h]
                Gam = np.exp(_g(None if laf is None else laf[c0:c1, h], m, dk))
                gC = Gam[-1]
                Ql, Kr, Ar, Bl = Q * Gam, K / Gam, A_ / Gam, B_ * Gam
                E = _unit_lower_inverse(np.eye(m) + (Bl @ Ar.T) * M1m)
                W = E @ Bl
                BK = (Bl @ Kr.T) * M1m
                Cm = -E @ (BK @ Vp)
                Nn = Cm - W @ S.T
                Sn = (S + Vp.T @ Kr + Nn.T @ Ar) * gC[None, :]
                chunks.append(dict(c0=c0, c1=c1, m=m, Ql=Ql, Kr=Kr, Ar=Ar, Bl=Bl, Gam=Gam, gC=gC,
                                   E=E, W=W, BK=BK, Nn=Nn, Vp=Vp, bet=bet, V=vf[c0:c1, h],
                                   dO=dOf[c0:c1, h], Sp=S, Sn=Sn))
                S = Sn
            dS = np.zeros((dv, dk)) if dS_final is None else np.array(dS_final[n, h], dtype=np.float64)
            for ch in reversed(chunks):
                m = ch["m"]
                Mm, M1m = M[:m, :m], M1[:m, :m]
                Ql, Kr, Ar, Bl, Gam, gC = ch["Ql"], ch["Kr"], ch["Ar"], ch["Bl"], ch["Gam"], ch["gC"]
                E, W, BK, Nn, Vp, Sp, G = ch["E"], ch["W"], ch["BK"], ch["Nn"], ch["Vp"], ch["Sp"], ch["dO"]
                dC = (Ar * gC[None, :]) @ dS.T + ((Ql @ Ar.T) * Mm).T @ G
                dV1 = (Kr * gC[None, :]) @ dS.T + ((Ql @ Kr.T) * Mm).T @ G
                dW = -dC @ Sp
                dE = -dC @ Vp.T @ BK.T + dW @ Bl.T
                dF = -E.T @ dE @ E.T
                dOV = (G @ Vp.T) * Mm
                dON = (G @ Nn.T) * Mm
                X = (E.T @ dC @ Vp.T) * M1m
                dQl = G @ Sp + dOV @ Kr + dON @ Ar
                dBl = E.T @ dW - X @ Kr + (dF * M1m) @ Ar
                dKr = dOV.T @ Ql - X.T @ Bl + Vp @ dS * gC[None, :]
                dAr = dON.T @ Ql + (dF * M1m).T @ Bl + Nn @ dS * gC[None, :]
                dVp = dV1 - BK.T @ (E.T @ dC)
                dlg = dQl * Ql + dBl * Bl - dKr * Kr - dAr * Ar
                dlg[-1] += np.sum(ch["Sn"] * dS, axis=0)
                sl = slice(ch["c0"], ch["c1"])
                out["dq"][sl, h] = dQl * Gam
                out["db"][sl, h] = dBl * Gam
                out["dk"][sl, h] = dKr / Gam
                out["da"][sl, h] = dAr / Gam
                out["dv"][sl, h] = ch["bet"][:, None] * dVp
                out["dbeta"][sl, h] = np.sum(dVp * ch["V"], axis=1)
                if la is not None:
                    suffix = np.cumsum(dlg[::-1], axis=0)[::-1]
                    out["dlog_alpha"][sl, h] = suffix if la.ndim == 4 else suffix.sum(axis=1)
                dS = dS * gC[None, :] + G.T @ Ql - dC.T @ W
            out["dS0"][n, h] = dS
    res = {key: val.reshape((B, T) + val.shape[1:]) for key, val in out.items() if key != "dS0"}
    res["dS0"] = out["dS0"]
    return res
