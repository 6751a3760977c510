"""Pins for the backward oracle (gradients of the fp64 recurrence).

Each test checks ``oracle.recurrence_bwd`` against something other than itself:
central finite differences of the forward oracle (a separate code path), closed
forms of the linear-attention special case, and the chunk form of the KDA
backward notes written out in numpy.
"""
import numpy as np
import pytest

import oracle
from oracle import chunk_mirror


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(rng, B=1, T=9, H=2, dk=3, dv=2, gate=2, dplr=False, cu=None, s0=True):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0.1, 1.0, (B, T, H))
    la = None
    if gate == 1:
        la = rng.uniform(-0.4, -0.01, (B, T, H))
    elif gate == 2:
        la = rng.uniform(-0.4, -0.01, (B, T, H, dk))
    a = b = None
    if dplr:
        a = _unit(rng.standard_normal((B, T, H, dk)))
        b = beta[..., None] * _unit(a + 0.5 * rng.standard_normal((B, T, H, dk)))
    N = B if cu is None else len(cu) - 1
    S0 = 0.5 * rng.standard_normal((N, H, dv, dk)) if s0 else None
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=la, a=a, b=b, S0=S0,
                cu_seqlens=None if cu is None else np.asarray(cu, dtype=np.int32))


def _loss(c, dO, dSf):
    O, Sf = oracle.recurrence(**c)
    return float(np.sum(O * dO) + np.sum(Sf * dSf))


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "log_alpha": "dlog_alpha",
           "a": "da", "b": "db", "S0": "dS0"}


def _fd_check(c, dO, dSf, g, names, rng=None, n_pick=None, h=1e-6, tol=2e-7):
    for name in names:
        x = c[name]
        idx = list(np.ndindex(x.shape))
        if n_pick is not None and len(idx) > n_pick:
            idx = [idx[i] for i in rng.choice(len(idx), n_pick, replace=False)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += h
            xm[ix] -= h
            fd = (_loss(dict(c, **{name: xp}), dO, dSf) - _loss(dict(c, **{name: xm}), dO, dSf)) / (2 * h)
            an = g[GRAD_OF[name]][ix]
            assert abs(fd - an) <= tol * (1 + abs(an)), (name, ix, fd, an)


@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_gradients_match_finite_differences(gate, dplr):
    """Every input's gradient against central differences of the forward oracle:
    packed sequences (one of length 0), several heads, initial state, dS_final."""
    rng = np.random.default_rng(500 + gate + 3 * dplr)
    cu = [0, 4, 4, 9]
    c = _case(rng, B=1, T=9, H=2, gate=gate, dplr=dplr, cu=cu)
    dO = rng.standard_normal(c["v"].shape)
    dSf = rng.standard_normal(c["S0"].shape)
    g = oracle.recurrence_bwd(dO=dO, dS_final=dSf, **c)
    names = ["q", "k", "v", "beta", "S0"] + (["log_alpha"] if gate else []) + \
        (["a", "b"] if dplr else [])
    _fd_check(c, dO, dSf, g, names)
    # the empty sequence passes dS_final straight through
    np.testing.assert_array_equal(g["dS0"][1], dSf[1])


def test_gradients_across_checkpoint_segments():
    """A sequence longer than the oracle's replay segment (64 tokens): sampled
    entries of every gradient against central differences."""
    rng = np.random.default_rng(510)
    c = _case(rng, B=2, T=150, H=1, dk=4, dv=3, gate=2, dplr=False)
    dO = rng.standard_normal(c["v"].shape)
    dSf = rng.standard_normal(c["S0"].shape)
    g = oracle.recurrence_bwd(dO=dO, dS_final=dSf, **c)
    _fd_check(c, dO, dSf, g, ["q", "k", "v", "beta", "log_alpha", "S0"], rng=rng, n_pick=25)


def test_linear_attention_closed_form_gradients():
    """b = 0, beta = 1, no gate, S0 = 0: O = (Q K^T masked) V and S_final = V^T K.
    Then dV = (Q K^T masked)^T dO + K dSf^T, dQ = (dO V^T masked) K,
    dK = (dO V^T masked)^T Q + V dSf, da = 0 (plain matrix calculus)."""
    rng = np.random.default_rng(520)
    T, d, dv = 11, 4, 3
    c = _case(rng, B=1, T=T, H=1, dk=d, dv=dv, gate=0, dplr=True, s0=False)
    c["b"] = np.zeros_like(c["b"])
    c["beta"] = np.ones_like(c["beta"])
    dO = rng.standard_normal(c["v"].shape)
    dSf = rng.standard_normal((1, 1, dv, d))
    g = oracle.recurrence_bwd(dO=dO, dS_final=dSf, **c)
    Q, K, V, G = c["q"][0, :, 0], c["k"][0, :, 0], c["v"][0, :, 0], dO[0, :, 0]
    M = np.tril(np.ones((T, T)))
    D = dSf[0, 0]
    np.testing.assert_allclose(g["dv"][0, :, 0], ((Q @ K.T) * M).T @ G + K @ D.T, atol=1e-12)
    np.testing.assert_allclose(g["dq"][0, :, 0], ((G @ V.T) * M) @ K, atol=1e-12)
    np.testing.assert_allclose(g["dk"][0, :, 0], ((G @ V.T) * M).T @ Q + V @ D, atol=1e-12)
    np.testing.assert_allclose(g["da"], 0.0, atol=1e-15)
    # beta scales the write: dbeta_i = v_i . (dv_i / beta_i) with beta = 1
    np.testing.assert_allclose(g["dbeta"][0, :, 0], np.sum(V * g["dv"][0, :, 0], axis=-1), atol=1e-12)


@pytest.mark.parametrize("C", [1, 5, 16])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_chunk_backward_of_the_notes_matches(C, gate):
    """The chunk-form backward of the KDA backward notes (numpy, fp64) against the
    token-level reverse pass: every gradient, packed sequences, initial state."""
    rng = np.random.default_rng(530 + C + 7 * gate)
    cu = [0, 23, 23, 40, 61]
    c = _case(rng, B=1, T=61, H=2, dk=5, dv=4, gate=gate, cu=cu)
    dO = rng.standard_normal(c["v"].shape)
    dSf = rng.standard_normal(c["S0"].shape)
    g = oracle.recurrence_bwd(dO=dO, dS_final=dSf, **c)
    m = chunk_mirror.chunk_bwd(dO=dO, dS_final=dSf, C=C, **c)
    for key in ["dq", "dk", "dv", "dbeta", "dS0"] + (["dlog_alpha"] if gate else []):
        np.testing.assert_allclose(m[key], g[key], rtol=0, atol=1e-10, err_msg=key)


@pytest.mark.parametrize("C", [1, 5, 16])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_dplr_chunk_backward_of_the_notes_matches(C, gate):
    """The gated DPLR chunk backward of the DPLR notes (section 3; numpy, fp64) against
    the token-level reverse pass: every gradient, a and b included."""
    rng = np.random.default_rng(560 + C + 7 * gate)
    cu = [0, 23, 23, 40, 61]
    c = _case(rng, B=1, T=61, H=2, dk=5, dv=4, gate=gate, dplr=True, cu=cu)
    dO = rng.standard_normal(c["v"].shape)
    dSf = rng.standard_normal(c["S0"].shape)
    g = oracle.recurrence_bwd(dO=dO, dS_final=dSf, **c)
    m = chunk_mirror.chunk_bwd(dO=dO, dS_final=dSf, C=C, **c)
    for key in ["dq", "dk", "dv", "da", "db", "dbeta", "dS0"] + (["dlog_alpha"] if gate else []):
        np.testing.assert_allclose(m[key], g[key], rtol=0, atol=1e-10, err_msg=key)
