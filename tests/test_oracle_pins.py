"""Pins for the CPU oracle: each test checks the fp64 recurrence (or the chunk
mirror) against something other than itself -- a hand-worked example, a closed
form, an identity proved on the pages, a textbook routine, or an invariant of
the recurrence -- chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_mirror

HERE = os.path.dirname(os.path.abspath(__file__))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(rng, B=1, T=40, H=2, dk=6, dv=5, gate=2, dplr=False, s0=True, la=(-0.3, -0.01)):
    q = _unit(rng.standard_normal((B, T, H, dk)))
    k = _unit(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.random((B, T, H))
    if gate == 0:
        log_alpha = None
    elif gate == 1:
        log_alpha = rng.uniform(*la, size=(B, T, H))
    else:
        log_alpha = rng.uniform(*la, size=(B, T, H, dk))
    a = b = None
    if dplr:
        a = _unit(rng.standard_normal((B, T, H, dk)))
        b = beta[..., None] * _unit(a + 0.3 * rng.standard_normal((B, T, H, dk)))
    S0 = rng.standard_normal((B, H, dv, dk)) * 0.5 if s0 else None
    return dict(q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, a=a, b=b, S0=S0)


def _alpha_full(log_alpha, shape):
    """exp(log alpha) broadcast to [B, T, H, dk]."""
    if log_alpha is None:
        return np.ones(shape)
    al = np.exp(log_alpha)
    return al if al.ndim == 4 else np.broadcast_to(al[..., None], shape)


# ---------------------------------------------------------------------------
# 1. Hand-worked examples (tests/golden/hand_worked.json).
# ---------------------------------------------------------------------------
def _load_hand():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_hand(), ids=lambda c: c["name"])
def test_hand_worked(case):
    dk, dv = case["dk"], case["dv"]
    k = np.array(case["k"])[None, :, None, :]
    T = k.shape[1]
    q = np.array(case["q"])[None, :, None, :]
    v = np.array(case["v"])[None, :, None, :]
    beta = np.array(case["beta"])[None, :, None]
    la = None if case["alpha"] is None else np.log(np.array(case["alpha"]))[None, :, None, :]
    a = b = None
    if "a" in case:
        a = np.array(case["a"])[None, :, None, :]
        b = np.array(case["b"])[None, :, None, :]
    S0 = np.array(case["S0"], dtype=np.float64).reshape(1, 1, dv, dk)
    O, Sf = oracle.recurrence(q, k, v, beta, log_alpha=la, a=a, b=b, S0=S0)
    np.testing.assert_allclose(O[0, :, 0, :], np.array(case["O"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sf[0, 0], np.array(case["S_final"]), rtol=0, atol=1e-12)
    assert T == len(case["O"])


# ---------------------------------------------------------------------------
# 2. Closed forms.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_gla_closed_form(gate):
    """b = 0: the recurrence is gated linear attention ("Gated Linear Attention"
    notes, sections 5.1-5.2): o_r = S0 Diag(gamma_r) q_r + sum_{i<=r} beta_i v_i
    (k_i * gamma_r/gamma_i)^T q_r with gamma the cumulative gate from the start."""
    rng = np.random.default_rng(10 + gate)
    c = _rand_case(rng, B=2, T=23, H=2, dk=5, dv=4, gate=gate)
    zeros = np.zeros_like(c["q"])
    O, Sf = oracle.recurrence(c["q"], c["k"], c["v"], c["beta"], log_alpha=c["log_alpha"],
                              a=zeros, b=zeros, S0=c["S0"])
    B, T, H, dk = c["q"].shape
    al = _alpha_full(c["log_alpha"], c["q"].shape)
    logg = np.cumsum(np.log(al), axis=1)
    ref = np.zeros_like(O)
    Sref = np.zeros_like(Sf)
    for bb in range(B):
        for h in range(H):
            for r in range(T):
                acc = c["S0"][bb, h] @ (np.exp(logg[bb, r, h]) * c["q"][bb, r, h])
                for i in range(r + 1):
                    dec = np.exp(logg[bb, r, h] - logg[bb, i, h])
                    acc = acc + c["beta"][bb, i, h] * c["v"][bb, i, h] * np.dot(
                        c["k"][bb, i, h] * dec, c["q"][bb, r, h])
                ref[bb, r, h] = acc
            S = c["S0"][bb, h] * np.exp(logg[bb, T - 1, h])[None, :]
            for i in range(T):
                dec = np.exp(logg[bb, T - 1, h] - logg[bb, i, h])
                S = S + c["beta"][bb, i, h] * np.outer(c["v"][bb, i, h], c["k"][bb, i, h] * dec)
            Sref[bb, h] = S
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Sf, Sref, rtol=0, atol=1e-12)


def test_linear_attention_closed_form():
    """No gate, b = 0, beta = 1: O = (Q K^T * M) V (causal linear attention,
    "DeltaNet" notes section 3 and "Gated Linear Attention" notes section 3.2)."""
    rng = np.random.default_rng(3)
    c = _rand_case(rng, B=1, T=31, H=3, dk=7, dv=4, gate=0, s0=False)
    zeros = np.zeros_like(c["q"])
    ones = np.ones_like(c["beta"])
    O, _ = oracle.recurrence(c["q"], c["k"], c["v"], ones, a=zeros, b=zeros)
    for h in range(3):
        Q, K, V = c["q"][0, :, h], c["k"][0, :, h], c["v"][0, :, h]
        ref = np.tril(Q @ K.T) @ V
        np.testing.assert_allclose(O[0, :, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_single_token(gate, dplr):
    """T = 1: S1 = S0 Diag(alpha)(I - b a^T) + beta v k^T and o = S1 q, with the
    gate applied before the rank-one factor ("Diagonal Plus Low Rank", section 2)."""
    rng = np.random.default_rng(20 + gate + 3 * dplr)
    c = _rand_case(rng, B=1, T=1, H=1, dk=6, dv=3, gate=gate, dplr=dplr)
    O, Sf = oracle.recurrence(**c)
    k = c["k"][0, 0, 0]
    a = k if c["a"] is None else c["a"][0, 0, 0]
    b = c["beta"][0, 0, 0] * k if c["b"] is None else c["b"][0, 0, 0]
    alpha = _alpha_full(c["log_alpha"], c["q"].shape)[0, 0, 0]
    S1 = c["S0"][0, 0] @ np.diag(alpha) @ (np.eye(6) - np.outer(b, a)) + \
        c["beta"][0, 0, 0] * np.outer(c["v"][0, 0, 0], k)
    np.testing.assert_allclose(Sf[0, 0], S1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O[0, 0, 0], S1 @ c["q"][0, 0, 0], rtol=0, atol=1e-13)
    if gate == 2:
        # The other gate order gives a different state on this case.
        other = c["S0"][0, 0] @ (np.eye(6) - np.outer(b, a)) @ np.diag(alpha) + \
            c["beta"][0, 0, 0] * np.outer(c["v"][0, 0, 0], k)
        assert np.max(np.abs(other - S1)) > 1e-3


@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [1, 2])
def test_total_forgetting(gate, dplr):
    """A gate that falls by e^-300 per token forgets everything before the current
    token: S_t = beta_t v_t k_t^T and o_t = beta_t v_t (k_t . q_t), whatever S0 and the
    rank-one factor (the recurrence with Diag(alpha) = 0 up to e^-300)."""
    rng = np.random.default_rng(40 + gate + 3 * dplr)
    c = _rand_case(rng, B=2, T=7, H=2, dk=5, dv=3, gate=gate, dplr=dplr)
    c["log_alpha"] = np.full_like(c["log_alpha"], -300.0)
    O, Sf = oracle.recurrence(**c)
    bv = c["beta"][..., None] * c["v"]
    kq = np.sum(c["k"] * c["q"], axis=-1)[..., None]
    np.testing.assert_allclose(O, bv * kq, rtol=0, atol=1e-13)
    last = np.einsum("bhi,bhj->bhij", bv[:, -1], c["k"][:, -1])
    np.testing.assert_allclose(Sf, last, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# 3. WY representation of the transition product.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [0, 2])
def test_wy_identity(gate, dplr):
    """With v = 0 and S0 = I the recurrence returns P = prod_t Diag(alpha_t)(I - b_t a_t^T).
    It must equal (a) the explicit product of the factors and (b) the WY form
    P = (I - sum_i w_i (a_i/gamma_i)^T) Diag(gamma_C) with
    w_r = (I - sum_{i<r} w_i (a_i/gamma_i)^T)(gamma_r * b_r)
    ("Diagonal Plus Low Rank", section 2; ungated: "DeltaNet" notes section 4.1,
    P = I - sum w k^T, w_r = beta_r (k_r - sum_{i<r} w_i k_i^T k_r))."""
    rng = np.random.default_rng(40 + gate + 5 * dplr)
    d, T = 6, 13
    c = _rand_case(rng, B=1, T=T, H=1, dk=d, dv=d, gate=gate, dplr=dplr, s0=False)
    c["v"] = np.zeros_like(c["v"])
    c["S0"] = np.eye(d)[None, None]
    _, P = oracle.recurrence(**c)
    P = P[0, 0]
    k = c["k"][0, :, 0]
    beta = c["beta"][0, :, 0]
    A = k if c["a"] is None else c["a"][0, :, 0]
    Bv = beta[:, None] * k if c["b"] is None else c["b"][0, :, 0]
    alpha = _alpha_full(c["log_alpha"], c["q"].shape)[0, :, 0]
    explicit = np.eye(d)
    for t in range(T):
        explicit = explicit @ np.diag(alpha[t]) @ (np.eye(d) - np.outer(Bv[t], A[t]))
    np.testing.assert_allclose(P, explicit, rtol=0, atol=1e-13)
    gam = np.cumprod(alpha, axis=0)
    w = []
    for r in range(T):
        acc = np.eye(d)
        for i in range(r):
            acc = acc - np.outer(w[i], A[i] / gam[i])
        w.append(acc @ (gam[r] * Bv[r]))
    wy = np.eye(d)
    for i in range(T):
        wy = wy - np.outer(w[i], A[i] / gam[i])
    wy = wy @ np.diag(gam[T - 1])
    np.testing.assert_allclose(P, wy, rtol=0, atol=1e-12)
    if gate == 0 and not dplr:
        w2 = []
        for r in range(T):
            w2.append(beta[r] * (k[r] - sum(w2[i] * np.dot(k[i], k[r]) for i in range(r))))
        P2 = np.eye(d) - sum(np.outer(w2[i], k[i]) for i in range(T))
        np.testing.assert_allclose(P, P2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 4. Spectral norm of I - eta k j^T ("How to make GDN2 more stable", eq. 4).
# ---------------------------------------------------------------------------
def test_spectral_norm_formula_vs_svd():
    rng = np.random.default_rng(7)
    for _ in range(200):
        d = int(rng.integers(2, 9))
        k = _unit(rng.standard_normal(d))
        j = _unit(rng.standard_normal(d))
        eta = float(rng.uniform(0, 3))
        svd = np.linalg.norm(np.eye(d) - eta * np.outer(k, j), 2)
        assert abs(oracle.spectral_norm_rank1(eta, k, j) - svd) < 1e-12
    k = _unit(rng.standard_normal(5))
    for eta in [0.0, 0.5, 1.0, 2.0, 2.7]:
        # c = 1: eigen-decomposable, norm max(1, |1 - eta|); c = -1: norm 1 + eta.
        assert abs(oracle.spectral_norm_rank1(eta, k, k) - max(1.0, abs(1 - eta))) < 1e-12
        assert abs(oracle.spectral_norm_rank1(eta, k, -k) - (1.0 + eta)) < 1e-12


def test_spectral_norm_exceeds_one_unless_aligned():
    """Corollary (eqs. 5-6): the norm is > 1 whenever k != j and eta > 0."""
    rng = np.random.default_rng(8)
    for _ in range(50):
        k = _unit(rng.standard_normal(4))
        j = _unit(k + 0.2 * rng.standard_normal(4))
        eta = float(rng.uniform(0.01, 2.0))
        assert oracle.spectral_norm_rank1(eta, k, j) > 1.0


# ---------------------------------------------------------------------------
# 4b. Spectral clipping of the gate inside the recurrence ("How to make GDN2
#     more stable", eq. 7): alpha <- min(alpha, 1/rho), rho = ||I - b a^T||_2.
#     The expected rho always comes from numpy's SVD, never from eq. 4.
# ---------------------------------------------------------------------------
def _rank1_case(rng, d, eta, spread):
    """a unit, b = eta * unit(a + spread * noise): GDN2's j = a and eta k = b."""
    a = _unit(rng.standard_normal(d))
    b = eta * _unit(a + spread * rng.standard_normal(d))
    return a, b


@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_clip_single_step_gate_is_min_with_inverse_norm(gate, dplr):
    """T = 1, S0 = I, no write: S1 = Diag(alpha')(I - b a^T).  Row j of S1 is alpha'_j
    times row j of I - b a^T; alpha'_j must be min(alpha_j, 1/sigma_max(I - b a^T))
    and ||S1||_2 <= 1 (eq. 2)."""
    rng = np.random.default_rng(300 + gate + 3 * dplr)
    d = 6
    c = _rand_case(rng, B=1, T=1, H=1, dk=d, dv=d, gate=gate, dplr=dplr, s0=False)
    c["S0"] = np.eye(d)[None, None]
    c["v"] = np.zeros_like(c["v"])
    if dplr:
        a, b = _rank1_case(rng, d, 1.6, 0.8)
        c["a"], c["b"] = a[None, None, None], b[None, None, None]
        c["beta"] = np.zeros_like(c["beta"])  # no write; b carries its own scale
    else:
        c["beta"] = np.full_like(c["beta"], 2.6)  # eta = beta |k|^2 > 2: rho = eta - 1
        a, b = c["k"][0, 0, 0], 2.6 * c["k"][0, 0, 0]
    if gate == 2:
        c["log_alpha"] = np.linspace(-1.5, -0.001, d)[None, None, None]
    elif gate == 1:
        c["log_alpha"] = np.full((1, 1, 1), -0.01)
    M = np.eye(d) - np.outer(b, a)
    rho = np.linalg.norm(M, 2)
    assert rho > 1.1
    alpha = _alpha_full(c["log_alpha"], c["q"].shape)[0, 0, 0]
    want = np.minimum(alpha, 1.0 / rho)
    if gate == 2:
        assert (alpha < 1 / rho).any() and (alpha > 1 / rho).any()  # both sides of the clip
    O, Sf = oracle.recurrence(**c, clip=True)
    S1 = Sf[0, 0]
    got = np.einsum("jk,jk->j", S1, M) / np.einsum("jk,jk->j", M, M)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S1, np.diag(want) @ M, rtol=0, atol=1e-13)
    assert np.linalg.norm(S1, 2) <= 1.0 + 1e-12
    np.testing.assert_allclose(O[0, 0, 0], S1 @ c["q"][0, 0, 0], rtol=0, atol=1e-13)
    if not dplr:
        assert abs(rho - 1.6) < 1e-12  # KDA form: max(eta, 2) - 1 (eq. 5)


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_clip_is_identity_when_the_factor_does_not_expand(gate):
    """Eq. 6: with a = k unit and eta = beta <= 2 the norm is 1, so clipping changes nothing."""
    rng = np.random.default_rng(320 + gate)
    c = _rand_case(rng, B=2, T=30, H=2, dk=5, dv=4, gate=gate, dplr=False)
    O0, S0_ = oracle.recurrence(**c)
    O1, S1 = oracle.recurrence(**c, clip=True)
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S1, S0_, rtol=0, atol=1e-13)


@pytest.mark.parametrize("gate", [0, 2])
def test_clip_makes_the_state_non_expansive(gate):
    """Without writes, S_t = S_{t-1} M_t with ||M_t||_2 <= 1 after clipping, so every
    ||S_t||_2 <= ||S0||_2 and |o_t| <= ||S0||_2 for unit q.  Unclipped, the same
    transitions blow the state up (so the check has teeth)."""
    rng = np.random.default_rng(340 + gate)
    d, T = 8, 60
    c = _rand_case(rng, B=1, T=T, H=1, dk=d, dv=d, gate=gate, dplr=True, la=(-0.02, -0.001))
    a = np.stack([_rank1_case(rng, d, float(rng.uniform(1.0, 3.0)), 1.0) for _ in range(T)])
    c["a"] = a[:, 0][None, :, None]
    c["b"] = a[:, 1][None, :, None]
    c["beta"] = np.zeros_like(c["beta"])
    s0 = np.linalg.norm(c["S0"][0, 0], 2)
    _, Sraw = oracle.recurrence(**c)
    assert np.linalg.norm(Sraw[0, 0], 2) > 10 * s0
    O, Sf = oracle.recurrence(**c, clip=True)
    assert np.linalg.norm(Sf[0, 0], 2) <= s0 * (1 + 1e-12)
    assert np.max(np.linalg.norm(O[0, :, 0], axis=-1)) <= s0 * (1 + 1e-12)


@pytest.mark.parametrize("dplr", [False, True])
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_clip_equals_unclipped_run_on_the_clipped_gate(gate, dplr):
    """The clip acts token by token and head by head: the clipped run equals an
    unclipped run whose gate is replaced by min(alpha_t, 1/rho_t), rho_t from the SVD
    of each token's I - b_t a_t^T (packed sequences, several heads, initial state)."""
    rng = np.random.default_rng(360 + gate + 3 * dplr)
    B, T, H, d, dv = 1, 37, 3, 5, 4
    c = _rand_case(rng, B=B, T=T, H=H, dk=d, dv=dv, gate=gate, dplr=dplr, s0=False)
    c["beta"] = rng.uniform(0.0, 4.0, size=(B, T, H))
    if dplr:
        c["b"] = c["beta"][..., None] * _unit(c["a"] + 0.7 * rng.standard_normal(c["a"].shape))
    cu = np.array([0, 11, 11, 30, 37], dtype=np.int32)
    c["cu_seqlens"] = cu
    c["S0"] = rng.standard_normal((len(cu) - 1, H, dv, d)) * 0.5
    k = c["k"][0]
    A = k if c["a"] is None else c["a"][0]
    Bv = c["beta"][0][..., None] * k if c["b"] is None else c["b"][0]
    inv_rho = np.empty((T, H))
    for t in range(T):
        for h in range(H):
            inv_rho[t, h] = 1.0 / np.linalg.norm(np.eye(d) - np.outer(Bv[t, h], A[t, h]), 2)
    alpha = _alpha_full(c["log_alpha"], c["q"].shape)[0]
    clipped = np.minimum(alpha, inv_rho[..., None])
    assert (alpha > inv_rho[..., None]).mean() > 0.2  # the clip is active often
    if gate == 2:
        la = np.log(clipped)[None]
    else:
        la = np.log(clipped[..., 0])[None]  # one value per token and head
    O1, S1 = oracle.recurrence(**c, clip=True)
    O2, S2 = oracle.recurrence(**dict(c, log_alpha=la))
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 5. The chunk rewrite against the definition, and its inverse's closed form.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 7, 16, 64])
@pytest.mark.parametrize("gate", [0, 1, 2])
@pytest.mark.parametrize("dplr", [False, True])
def test_chunk_mirror_matches_recurrence(C, gate, dplr):
    rng = np.random.default_rng(100 + C + 3 * gate + 50 * dplr)
    c = _rand_case(rng, B=2, T=100, H=2, dk=8, dv=6, gate=gate, dplr=dplr)
    O, Sf = oracle.recurrence(**c)
    Om, Sm, _ = chunk_mirror.chunk_forward(**c, C=C)
    scale = max(np.max(np.abs(O)), 1.0)
    assert np.max(np.abs(Om - O)) / scale < 1e-12
    assert np.max(np.abs(Sm - Sf)) / max(np.max(np.abs(Sf)), 1.0) < 1e-12


def test_chunk_mirror_varlen():
    rng = np.random.default_rng(5)
    c = _rand_case(rng, B=1, T=150, H=2, dk=8, dv=8, gate=2, s0=False)
    cu = np.array([0, 37, 64, 150], dtype=np.int32)
    c["S0"] = rng.standard_normal((3, 2, 8, 8)) * 0.3
    O, Sf = oracle.recurrence(**c, cu_seqlens=cu)
    Om, Sm, _ = chunk_mirror.chunk_forward(**c, cu_seqlens=cu, C=16)
    assert np.max(np.abs(Om - O)) < 1e-12 * max(1, np.max(np.abs(O)))
    assert np.max(np.abs(Sm - Sf)) < 1e-12 * max(1, np.max(np.abs(Sf)))


@pytest.mark.parametrize("gate", [0, 2])
def test_inverse_entries_bounded_and_closed_form(gate):
    """For unit k and beta in [0, 1], every entry of the UT inverse
    At = (I + Diag(beta)(K<- K->^T * M_1))^-1 lies in [-1, 1] (the claim quoted by
    "How to make GDN2 more stable").  The reason is the closed form, which
    follows from expanding (I + L)^-1 as the finite Neumann series of the
    "DeltaNet" notes (section 4.2):
      At_ri = -beta_r k_r^T D_r (I - beta_{r-1} k k^T) D_{r-1} ... (I - beta_{i+1} k k^T) D_{i+1} k_i
    (D_j = Diag(alpha_j)), a product of factors of spectral norm <= 1."""
    rng = np.random.default_rng(60 + gate)
    C, d = 16, 8
    c = _rand_case(rng, B=1, T=C, H=1, dk=d, dv=3, gate=gate, s0=False, la=(-0.5, -0.01))
    _, _, rec = chunk_mirror.chunk_forward(**c, C=C, record=True)
    At = rec[0][0]["A"]
    assert np.all(np.abs(At) <= 1.0 + 1e-12)
    np.testing.assert_allclose(np.diag(At), 1.0, atol=1e-14)
    assert np.all(np.triu(At, 1) == 0)
    k = c["k"][0, :, 0]
    beta = c["beta"][0, :, 0]
    alpha = _alpha_full(c["log_alpha"], c["q"].shape)[0, :, 0]
    for r in range(C):
        for i in range(r):
            M = np.diag(alpha[r])
            for j in range(r - 1, i, -1):
                M = M @ (np.eye(d) - beta[j] * np.outer(k[j], k[j])) @ np.diag(alpha[j])
            closed = -beta[r] * k[r] @ M @ k[i]
            assert abs(At[r, i] - closed) < 1e-13


def test_inverse_matches_textbook_inverse():
    rng = np.random.default_rng(61)
    c = _rand_case(rng, B=1, T=32, H=1, dk=8, dv=3, gate=2, s0=False, dplr=True)
    _, _, rec = chunk_mirror.chunk_forward(**c, C=32, record=True)
    E = rec[0][0]["A"]
    # E must be the inverse of I + (B<- A->^T * M_1): check E X = I with numpy's own inverse.
    al = _alpha_full(c["log_alpha"], c["q"].shape)[0, :, 0]
    gam = np.cumprod(al, axis=0)
    Bl = c["b"][0, :, 0] * gam
    Ar = c["a"][0, :, 0] / gam
    X = np.eye(32) + np.tril(Bl @ Ar.T, -1)
    np.testing.assert_allclose(E, np.linalg.inv(X), atol=1e-10)
