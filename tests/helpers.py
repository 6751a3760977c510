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
                             chains=chains, n_threads=n_threads, clip=P.clip)


def rel_err(x, ref):
    """max|x - ref| / max|ref| over all finite reference entries."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = np.isfinite(ref)
    denom = np.max(np.abs(ref[m])) if m.any() else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(x[m]))) if m.any() else 0.0
    return float(np.max(np.abs(x[m] - ref[m])) / denom)


def gpu_run(P, device="cuda", **kw):
    """Run the HIP path on a Problem; returns (O, S_final) as float64 numpy."""
    from chunkwise_gated_delta_amd import gdr
    to = lambda t: None if t is None else t.to(device)
    O, Sf = gdr.chunk_fwd(to(P.q), to(P.k), to(P.v), to(P.beta), log_alpha=to(P.log_alpha),
                          a=to(P.a), b=to(P.b), S0=to(P.S0), cu_seqlens=to(P.cu_seqlens),
                          chunk_size=P.chunk, clip=P.clip, **kw)
    torch.cuda.synchronize()
    return (O.to(torch.float64).cpu().numpy(),
            None if Sf is None else Sf.to(torch.float64).cpu().numpy())


def chain_slices(P, chains):
    """For each (sequence, head): (batch row, token slice, head) into O[B, T, H, dv]."""
    out = []
    for n, h in chains:
        if P.cu_seqlens is None:
            out.append((n, slice(0, P.T), h))
        else:
            cu = P.cu_seqlens.tolist()
            out.append((0, slice(cu[n], cu[n + 1]), h))
    return out


def compare(P, O, Sf, chains=None, n_threads=0):
    """Relative errors (O, S_final) of a GPU result against the oracle,
    over all chains or over the given (sequence, head) chains."""
    Oref, Sref = oracle_of(P, chains=chains, n_threads=n_threads)
    if chains is None:
        return rel_err(O, Oref), (None if Sf is None else rel_err(Sf, Sref))
    og, orf, sg, srf = [], [], [], []
    for (n, h), (b, sl, hh) in zip(chains, chain_slices(P, chains)):
        og.append(O[b, sl, hh].ravel())
        orf.append(Oref[b, sl, hh].ravel())
        if Sf is not None:
            sg.append(Sf[n, h].ravel())
            srf.append(Sref[n, h].ravel())
    eo = rel_err(np.concatenate(og), np.concatenate(orf))
    es = None if Sf is None else rel_err(np.concatenate(sg), np.concatenate(srf))
    return eo, es
