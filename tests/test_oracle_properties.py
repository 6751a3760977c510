"""Property tests of the oracle over random shapes (hypothesis): invariants that follow
from the recurrence S_t = S_{t-1} Diag(alpha_t)(I - b_t a_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t ("Diagonal Plus Low Rank" notes, section 2) hold for every draw of sizes,
gate layout, form (a = k, b = beta k, or a, b given) and initial state:

* state passing: running [0, s) and then [s, T) from the carried state is one run;
* packed sequences (cu_seqlens, empty ones included) equal separate runs;
* the map (v, S0) -> (O, S_final) is linear for fixed keys, gates and beta;
* the reverse pass: <dL/dx, d> for a random direction d matches a central finite
  difference of L = <dO, O> + <dS_final, S_final>.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = dict(max_examples=100, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw, max_T=24):
    """A random small problem: sizes, gate layout, form, initial state; values from a seed."""
    B = draw(st.integers(1, 2))
    T = draw(st.integers(1, max_T))
    H = draw(st.integers(1, 3))
    dk = draw(st.integers(1, 6))
    dv = draw(st.integers(1, 5))
    gate = draw(st.sampled_from([0, 1, 2]))
    dplr = draw(st.booleans())
    has_s0 = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    c = dict(q=unit(rng.standard_normal((B, T, H, dk))), k=unit(rng.standard_normal((B, T, H, dk))),
             v=rng.standard_normal((B, T, H, dv)), beta=rng.random((B, T, H)))
    c["log_alpha"] = (None if gate == 0 else
                      rng.uniform(-0.5, 0.0, size=(B, T, H) if gate == 1 else (B, T, H, dk)))
    c["a"] = unit(rng.standard_normal((B, T, H, dk))) if dplr else None
    c["b"] = (c["beta"][..., None] * unit(c["a"] + 0.3 * rng.standard_normal((B, T, H, dk)))
              if dplr else None)
    c["S0"] = 0.5 * rng.standard_normal((B, H, dv, dk)) if has_s0 else None
    return c


def _slice(c, sl):
    return {k: (v[:, sl] if (v is not None and k != "S0") else v) for k, v in c.items()}


@settings(**SETTINGS)
@given(problems(), st.floats(0.0, 1.0))
def test_state_passing_any_split(c, frac):
    T = c["q"].shape[1]
    s = int(round(frac * T))
    O, Sf = oracle.recurrence(**c)
    O1, S1 = oracle.recurrence(**_slice(c, slice(0, s))) if s > 0 else (None, c["S0"])
    tail = _slice(c, slice(s, T))
    tail["S0"] = S1 if s > 0 else c["S0"]
    if s < T:
        O2, S2 = oracle.recurrence(**tail)
    else:
        O2, S2 = np.zeros(O[:, :0].shape), S1
    Ocat = O2 if s == 0 else np.concatenate([O1, O2], axis=1)
    np.testing.assert_allclose(Ocat, O, rtol=0, atol=1e-11)
    np.testing.assert_allclose(S2, Sf, rtol=0, atol=1e-11)


@settings(**SETTINGS)
@given(problems(max_T=30), st.lists(st.integers(0, 12), min_size=1, max_size=5))
def test_packed_sequences_equal_separate_runs(c, lens):
    # one batch row holds the sequences back to back (lengths may be zero)
    total = sum(lens)
    if total == 0:
        lens = [1] + lens[1:]
        total = sum(lens)
    c = {k: (v[:1] if v is not None else None) for k, v in c.items()}
    T = c["q"].shape[1]
    reps = -(-total // T)
    packed = {k: (np.concatenate([v] * reps, axis=1)[:, :total] if (v is not None and k != "S0") else v)
              for k, v in c.items()}
    n = len(lens)
    H, dv, dk = c["v"].shape[2], c["v"].shape[3], c["q"].shape[3]
    rng = np.random.default_rng(total)
    packed["S0"] = 0.5 * rng.standard_normal((n, H, dv, dk))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    O, Sf = oracle.recurrence(**packed, cu_seqlens=cu)
    for i in range(n):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        if t1 == t0:  # an empty sequence returns its initial state
            np.testing.assert_array_equal(Sf[i], packed["S0"][i])
            continue
        part = _slice(packed, slice(t0, t1))
        part["S0"] = packed["S0"][i:i + 1]
        On, Sn = oracle.recurrence(**part)
        np.testing.assert_allclose(On, O[:, t0:t1], rtol=0, atol=1e-11)
        np.testing.assert_allclose(Sn[0], Sf[i], rtol=0, atol=1e-11)


@settings(**SETTINGS)
@given(problems(), st.floats(-3.0, 3.0), st.floats(-3.0, 3.0))
def test_linear_in_values_and_initial_state(c, x, y):
    rng = np.random.default_rng(7)
    B, T, H, dv = c["v"].shape
    dk = c["q"].shape[3]
    v2 = rng.standard_normal(c["v"].shape)
    s1 = rng.standard_normal((B, H, dv, dk))
    s2 = rng.standard_normal((B, H, dv, dk))
    Oa, Sa = oracle.recurrence(**dict(c, S0=s1))
    Ob, Sb = oracle.recurrence(**dict(c, v=v2, S0=s2))
    Oc, Sc = oracle.recurrence(**dict(c, v=x * c["v"] + y * v2, S0=x * s1 + y * s2))
    scale = 1.0 + abs(x) + abs(y)
    np.testing.assert_allclose(Oc, x * Oa + y * Ob, rtol=0, atol=1e-10 * scale)
    np.testing.assert_allclose(Sc, x * Sa + y * Sb, rtol=0, atol=1e-10 * scale)


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(problems(max_T=12), st.integers(0, 2 ** 31 - 1))
def test_reverse_pass_matches_directional_finite_difference(c, seed):
    rng = np.random.default_rng(seed)
    B, T, H, dv = c["v"].shape
    dk = c["q"].shape[3]
    dO = rng.standard_normal((B, T, H, dv))
    dSf = rng.standard_normal((B, H, dv, dk))
    S0 = c["S0"] if c["S0"] is not None else np.zeros((B, H, dv, dk))
    c = dict(c, S0=S0)
    g = oracle.recurrence_bwd(**c, dO=dO, dS_final=dSf)
    names = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "S0": "dS0", "a": "da", "b": "db",
             "log_alpha": "dlog_alpha"}
    dirs = {k: rng.standard_normal(np.shape(c[k])) for k in names if c.get(k) is not None}

    def loss(t):
        cc = {k: (v + t * dirs[k] if k in dirs else v) for k, v in c.items()}
        O, Sf = oracle.recurrence(**cc)
        return float(np.sum(O * dO) + np.sum(Sf * dSf))

    eps = 1e-5
    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    an = sum(float(np.sum(g[names[k]] * d)) for k, d in dirs.items())
    assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (fd, an)
