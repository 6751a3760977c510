"""Parity beyond 2^31 elements per tensor (every global offset of the HIP path is 64-bit).

KDA form in bf16, B = 1, H = 1024, T = 16448 (257 chunks, the last one ragged), dk = dv =
128: q, k, v, log alpha, O and every input gradient hold 2,155,872,256 elements (> 2^31),
the forward blocks 16.3 GB and each per-chunk state buffer 8.6 GB of the workspace.  The
fp32 kernels the same way: GDN form, H = 1024, T = 32832 (513 chunks), dk = dv = 64, 2^31
+ 2^23 elements per tensor.  The inputs are drawn on the device; the oracle recomputes the
first, a middle and the last head (the largest offsets) from the same values, to the bar
of the input precision (1e-2 bf16, 1e-4 fp32).  Every element of O and of the gradients
is checked to have been written (NaN canaries).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from chunkwise_gated_delta_amd import gdr, inputs
from helpers import rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2
H, T = 1024, 16448
HEADS = (0, 517, H - 1)


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield


@pytest.fixture(scope="module")
def big():
    P = inputs.make_problem_on_device("kda", "cuda", B=1, H=H, T=T, seed=11)
    assert P.q.numel() > 2**31 and P.log_alpha.numel() > 2**31
    yield P
    del P
    torch.cuda.empty_cache()


def _head(t, h):
    """One head of a [B, T, H, ...] device tensor as a float64 [B, T, 1, ...] array."""
    return t[:, :, h:h + 1].to(torch.float64).cpu().numpy()


def test_forward_beyond_2_31_elements(big):
    P = big
    ws = torch.zeros(gdr.workspace_bytes(1, H, T, 128, 128), dtype=torch.uint8, device="cuda")
    out = torch.full((1, T, H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    O, Sf = gdr.chunk_fwd(P.q, P.k, P.v, P.beta, log_alpha=P.log_alpha, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert gdr.check_workspace_error(ws) == 0
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(Sf).all())
    del ws
    for h in HEADS:
        Oref, Sref = oracle.recurrence(_head(P.q, h), _head(P.k, h), _head(P.v, h), _head(P.beta, h),
                                       log_alpha=_head(P.log_alpha, h))
        eo = rel_err(_head(O, h), Oref)
        es = rel_err(Sf[:, h:h + 1].to(torch.float64).cpu().numpy(), Sref)
        print(f"[gpu-case] head {h}: rel err O {eo:.3e} S_final {es:.3e}", file=sys.__stderr__, flush=True)
        assert eo <= TOL and es <= TOL
    del O, Sf, out
    torch.cuda.empty_cache()


def test_backward_beyond_2_31_elements(big):
    P = big
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    dO = torch.randn((1, T, H, 128), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dSf = 0.1 * torch.randn((1, H, 128, 128), generator=gen, device="cuda", dtype=torch.float32)
    ws = torch.zeros(gdr.bwd_workspace_bytes(1, H, T, 128, 128), dtype=torch.uint8, device="cuda")
    g = gdr.chunk_bwd(P.q, P.k, P.v, P.beta, dO, log_alpha=P.log_alpha, dS_final=dSf, workspace=ws)
    torch.cuda.synchronize()
    assert gdr.check_workspace_error(ws) == 0
    del ws
    for key, val in g.items():
        assert bool(torch.isfinite(val).all()), key
    for h in HEADS:
        ref = oracle.recurrence_bwd(_head(P.q, h), _head(P.k, h), _head(P.v, h), _head(P.beta, h),
                                    _head(dO, h), log_alpha=_head(P.log_alpha, h),
                                    dS_final=dSf[:, h:h + 1].to(torch.float64).cpu().numpy())
        errs = {}
        for key in ("dq", "dk", "dv", "dbeta", "dlog_alpha"):
            errs[key] = rel_err(_head(g[key], h), ref[key])
        errs["dS0"] = rel_err(g["dS0"][:, h:h + 1].to(torch.float64).cpu().numpy(), ref["dS0"])
        print(f"[gpu-case] head {h}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()),
              file=sys.__stderr__, flush=True)
        assert max(errs.values()) <= TOL, errs
    del g, dO, dSf
    torch.cuda.empty_cache()


def test_fp32_forward_beyond_2_31_elements():
    T32 = 32832
    P = inputs.make_problem_on_device("gdn", "cuda", B=1, H=H, T=T32, dk=64, dv=64,
                                      dtype=torch.float32, seed=13)
    assert P.q.numel() > 2**31
    ws = torch.zeros(gdr.workspace_bytes(1, H, T32, 64, 64, dtype=torch.float32, gate=gdr.GATE_HEAD),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((1, T32, H, 64), float("nan"), dtype=torch.float32, device="cuda")
    O, Sf = gdr.chunk_fwd(P.q, P.k, P.v, P.beta, log_alpha=P.log_alpha, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert gdr.check_workspace_error(ws) == 0
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(Sf).all())
    del ws
    for h in HEADS:
        Oref, Sref = oracle.recurrence(_head(P.q, h), _head(P.k, h), _head(P.v, h), _head(P.beta, h),
                                       log_alpha=_head(P.log_alpha, h))
        eo = rel_err(_head(O, h), Oref)
        es = rel_err(Sf[:, h:h + 1].to(torch.float64).cpu().numpy(), Sref)
        print(f"[gpu-case] fp32 head {h}: rel err O {eo:.3e} S_final {es:.3e}", file=sys.__stderr__, flush=True)
        assert eo <= 1e-4 and es <= 1e-4
    del O, Sf, out, P
    torch.cuda.empty_cache()
