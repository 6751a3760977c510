"""Seeded synthetic inputs for the gated delta-rule forward pass.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, so both the CPU oracle tests and the GPU tests can use it.

Seven workloads are defined, each a sampled stand-in for the shapes and value
ranges used to study the method (the pages report no dataset for this path):

1. ``deltanet_f32``  DeltaNet, no gate, fp32:   B=1  H=2  T=256   dk=dv=64
2. ``gdn``           Gated DeltaNet, head gate:  B=4  H=16 T=4096  dk=dv=128
3. ``kda``           KDA, per-channel gate:      B=2  H=32 T=8192  dk=dv=128
4. ``dplr``          gated DPLR, distinct a, b:  B=1  H=16 T=16384 dk=dv=128; the drawn
                     beta scales b only and the write term is unscaled (beta = 1 is passed)
5. ``kda_varlen``    KDA, 8 packed sequences:    32768 tokens, H=32, dk=dv=128
6. ``gdn2_clip``     GDN2 form with the spectral gate clip: the ``dplr`` shapes, with
                     the write key tied to b (b = beta k, as in the GDN2 form)
7. ``kda_strong``    the ``kda`` shapes with -log alpha log-uniform in [1e-3, 8] per
                     (token, channel): chunks whose gate falls beyond the range of the
                     scaled operands (the log-domain prep's workload)

Draw order (fixed, so every consumer sees the same bytes): [lengths], q, k, v,
beta, log_alpha, [a_raw, b_noise], [S0].  All draws are float32; q and k (and a,
b) are L2-normalised over the head dimension in float32, then rounded to the
input dtype (bf16 by round-to-nearest-even) where the workload says so.  In the
GDN2 form (``gdn2``) the drawn k is discarded for k = unit(a + 0.1 noise), so
that b = beta k carries the same key as the write term.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

GATE_NONE, GATE_HEAD, GATE_CHANNEL = 0, 1, 2


@dataclasses.dataclass
class Problem:
    """One forward-pass problem. Tensors are CPU torch tensors.

    Layout: q, k, a, b ``[B, T, H, dk]``; v ``[B, T, H, dv]``;
    log_alpha ``[B, T, H]`` (head gate) or ``[B, T, H, dk]`` (channel gate) fp32;
    beta ``[B, T, H]`` fp32; S0 ``[N, H, dv, dk]`` fp32 where N is B, or the number
    of packed sequences when ``cu_seqlens`` is given (then B == 1).
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    beta: torch.Tensor
    log_alpha: Optional[torch.Tensor]
    a: Optional[torch.Tensor]
    b: Optional[torch.Tensor]
    S0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    gate: int
    chunk: int = 64
    clip: bool = False  # spectral clipping of the gate, alpha <- min(alpha, 1/||I - b a^T||)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def dk(self):
        return self.q.shape[3]

    @property
    def dv(self):
        return self.v.shape[3]

    @property
    def n_seq(self):
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def dtype(self):
        return self.q.dtype

    def tokens(self):
        return self.B * self.T

    def seq_bounds(self):
        """(start, end) token offsets into the flattened [B*T] token axis."""
        if self.cu_seqlens is None:
            return [(i * self.T, (i + 1) * self.T) for i in range(self.B)]
        cu = self.cu_seqlens.tolist()
        return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def _l2n(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _cast(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def dirichlet_lengths(rng: np.random.Generator, n_seq: int, total: int, min_len: int) -> np.ndarray:
    """Split ``total`` tokens into ``n_seq`` lengths, each >= ``min_len``.

    p ~ Dirichlet(1); L_i = min_len + floor(p_i * (total - n_seq*min_len)); the
    remaining tokens go one each to the largest fractional parts (ties to the
    lower index), so the lengths sum to ``total`` exactly.
    """
    p = rng.dirichlet(np.ones(n_seq))
    spare = total - n_seq * min_len
    assert spare >= 0
    raw = p * spare
    base = np.floor(raw).astype(np.int64)
    rem = int(spare - base.sum())
    frac = raw - base
    order = sorted(range(n_seq), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    return (base + min_len).astype(np.int64)


def make_problem(kind: str, *, seed: Optional[int] = None, B=None, H=None, T=None, dk=None,
                 dv=None, n_seq=None, total=None, min_len=None, dtype=None,
                 s0_scale=None, gate=None, dplr=None, clip=None, la_range=None,
                 chunk: int = 64) -> Problem:
    """Build a seeded problem of workload ``kind`` (see module doc).

    Keyword overrides shrink or reshape a workload while keeping its value
    distributions, so small parity cases and the full-size workloads share one
    recipe.  ``gate`` swaps the gate mode (the log-decay range stays the
    workload's); ``dplr=True`` adds distinct a, b drawn as in the ``dplr`` workload;
    ``clip`` turns the spectral gate clipping on or off; ``la_range`` replaces the
    uniform range of log alpha.
    """
    spec = dict(WORKLOADS[kind])
    spec.update({k: v for k, v in dict(B=B, H=H, T=T, dk=dk, dv=dv, n_seq=n_seq, total=total,
                                        min_len=min_len, dtype=dtype, s0_scale=s0_scale,
                                        gate=gate, dplr=dplr, clip=clip, la_range=la_range).items()
                 if v is not None})
    if seed is None:
        seed = spec["seed"]
    rng = np.random.default_rng(seed)
    dt = spec["dtype"]
    H_, dk_, dv_ = spec["H"], spec["dk"], spec["dv"]
    cu = None
    if spec.get("varlen"):
        lens = dirichlet_lengths(rng, spec["n_seq"], spec["total"], spec["min_len"])
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B_, T_ = 1, int(spec["total"])
    else:
        B_, T_ = spec["B"], spec["T"]
    shp = (B_, T_, H_)
    q = _l2n(rng.standard_normal(shp + (dk_,), dtype=np.float32))
    k = _l2n(rng.standard_normal(shp + (dk_,), dtype=np.float32))
    v = rng.standard_normal(shp + (dv_,), dtype=np.float32)
    beta = rng.random(shp, dtype=np.float32)
    gate = spec["gate"]
    log_alpha = None
    gshape = shp if gate == GATE_HEAD else shp + (dk_,)
    if gate != GATE_NONE and spec.get("la_loguniform") and la_range is None:
        # decay rates spread over orders of magnitude: -log alpha log-uniform in [lo, hi]
        lo, hi = spec["la_loguniform"]
        log_alpha = (-np.exp(rng.uniform(np.log(lo), np.log(hi), size=gshape))).astype(np.float32)
    elif gate != GATE_NONE:
        log_alpha = rng.uniform(*spec["la_range"], size=gshape).astype(np.float32)
    a = b = None
    if spec.get("dplr"):
        a32 = _l2n(rng.standard_normal(shp + (dk_,), dtype=np.float32))
        noise = rng.standard_normal(shp + (dk_,), dtype=np.float32)
        kb = _l2n(a32 + np.float32(0.1) * noise)
        b32 = (beta[..., None] * kb).astype(np.float32)
        a, b = _cast(a32, dt), _cast(b32, dt)
        if spec.get("gdn2"):
            k = kb
        if spec.get("unit_write"):
            # the drawn beta lives on in b only: the write term is v k^T, unscaled
            beta = np.ones_like(beta)
    S0 = None
    if spec.get("s0_scale"):
        n = len(cu) - 1 if cu is not None else B_
        S0 = torch.from_numpy(
            (np.float32(spec["s0_scale"]) * rng.standard_normal((n, H_, dv_, dk_), dtype=np.float32)))
    return Problem(
        name=kind, q=_cast(q, dt), k=_cast(k, dt), v=_cast(v, dt), beta=torch.from_numpy(beta),
        log_alpha=None if log_alpha is None else torch.from_numpy(log_alpha), a=a, b=b, S0=S0,
        cu_seqlens=None if cu is None else torch.from_numpy(cu), gate=gate, chunk=chunk,
        clip=bool(spec.get("clip", False)))


def make_problem_on_device(kind: str, device, *, seed: Optional[int] = None, B=None, H=None,
                           T=None, dk=None, dv=None, dtype=None) -> Problem:
    """A workload's recipe drawn on ``device`` with a seeded torch generator, for sizes
    whose host copy would be too large (tensors beyond 2^31 elements).

    The forms without a, b and without packing only (kda, gdn): q, k ~ N(0, 1)
    L2-normalised per token, v ~ N(0, 1), beta ~ U(0, 1), log alpha ~ U(la_range), drawn
    in that order, one tensor at a time.  Same distributions as ``make_problem``, other
    values (another generator).  The returned Problem holds device tensors.
    """
    spec = dict(WORKLOADS[kind])
    assert not spec.get("varlen") and not spec.get("dplr") and "la_range" in spec
    spec.update({k: v for k, v in dict(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype).items()
                 if v is not None})
    gen = torch.Generator(device=device)
    gen.manual_seed(spec["seed"] if seed is None else seed)
    shp = (spec["B"], spec["T"], spec["H"])
    dt = spec["dtype"]

    def unit_rows(d):
        x = torch.randn(shp + (d,), generator=gen, device=device, dtype=torch.float32)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dt)

    q = unit_rows(spec["dk"])
    k = unit_rows(spec["dk"])
    v = torch.randn(shp + (spec["dv"],), generator=gen, device=device, dtype=torch.float32).to(dt)
    beta = torch.rand(shp, generator=gen, device=device, dtype=torch.float32)
    gate = spec["gate"]
    gshape = shp if gate == GATE_HEAD else shp + (spec["dk"],)
    lo, hi = spec["la_range"]
    log_alpha = torch.rand(gshape, generator=gen, device=device, dtype=torch.float32)
    log_alpha.mul_(hi - lo).add_(lo)
    return Problem(name=kind, q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, a=None, b=None,
                   S0=None, cu_seqlens=None, gate=gate)


def make_cotangents(P: Problem, seed: int, ds_scale: float = 0.1):
    """Seeded dO (P's dtype, shape of O) and dS_final (fp32, shape of S_final) for the
    backward pass: dO ~ N(0, 1), dS_final ~ ds_scale N(0, 1), drawn in that order."""
    rng = np.random.default_rng(seed)
    dO = _cast(rng.standard_normal((P.B, P.T, P.H, P.dv), dtype=np.float32), P.dtype)
    dSf = torch.from_numpy(np.float32(ds_scale) *
                           rng.standard_normal((P.n_seq, P.H, P.dv, P.dk), dtype=np.float32))
    return dO, dSf


WORKLOADS = {
    "deltanet_f32": dict(seed=1, B=1, H=2, T=256, dk=64, dv=64, dtype=torch.float32,
                         gate=GATE_NONE),
    "gdn": dict(seed=2, B=4, H=16, T=4096, dk=128, dv=128, dtype=torch.bfloat16,
                gate=GATE_HEAD, la_range=(-0.1, -0.001)),
    "kda": dict(seed=3, B=2, H=32, T=8192, dk=128, dv=128, dtype=torch.bfloat16,
                gate=GATE_CHANNEL, la_range=(-0.2, -0.001)),
    # the DPLR notes' form (section 2): b = beta unit(a + 0.1 noise), write term v k^T
    # unscaled, so the library's write scale is 1
    "dplr": dict(seed=4, B=1, H=16, T=16384, dk=128, dv=128, dtype=torch.bfloat16,
                 gate=GATE_CHANNEL, la_range=(-0.1, -0.001), dplr=True, unit_write=True),
    "kda_varlen": dict(seed=5, varlen=True, n_seq=8, total=32768, min_len=256, H=32, dk=128,
                       dv=128, dtype=torch.bfloat16, gate=GATE_CHANNEL, la_range=(-0.2, -0.001),
                       s0_scale=0.1),
    "gdn2_clip": dict(seed=6, B=1, H=16, T=16384, dk=128, dv=128, dtype=torch.bfloat16,
                      gate=GATE_CHANNEL, la_range=(-0.1, -0.001), dplr=True, gdn2=True, clip=True),
    # KDA shapes with per-channel decay rates over four orders of magnitude, as a forget
    # gate exp(-w softplus(x)) gives: most chunks hold channels whose gate falls by far more
    # than the scaled operands' exponent range, so they take the log-domain prep
    "kda_strong": dict(seed=7, B=2, H=32, T=8192, dk=128, dv=128, dtype=torch.bfloat16,
                       gate=GATE_CHANNEL, la_range=(-0.2, -0.001), la_loguniform=(1e-3, 8.0)),
}

# The tolerance on max|X - X_ref| / max|X_ref| for O and for the final state.
TOLERANCE = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
