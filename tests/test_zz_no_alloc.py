"""gdr_chunk_fwd_noalloc: the forward without a workspace argument, on the library's
fixed per-GPU scratch array, for callers that cannot allocate.  Its output is held to
gdr_chunk_fwd's on the same inputs (the same kernels: the same bits) and to the oracle
at the bf16 / fp32 bar, over two calls in a row, the second one smaller.
"""
import sys

import numpy as np
import pytest
import torch

from chunkwise_gated_delta_amd import gdr, inputs
from helpers import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield


def _run(P, no_alloc, flags=None):
    to = lambda t: None if t is None else t.to("cuda")
    O, Sf = gdr.chunk_fwd(to(P.q), to(P.k), to(P.v), to(P.beta), log_alpha=to(P.log_alpha),
                          a=to(P.a), b=to(P.b), S0=to(P.S0), cu_seqlens=to(P.cu_seqlens),
                          chunk_size=P.chunk, clip=P.clip, no_alloc=no_alloc, flags=flags)
    torch.cuda.synchronize()
    return O, Sf


def _check_pair(P):
    O1, S1 = _run(P, no_alloc=False)
    O2, S2 = _run(P, no_alloc=True)
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
    eo, es = compare(P, O2.double().cpu().numpy(), S2.double().cpu().numpy())
    tol = inputs.TOLERANCE[P.dtype]
    print(f"[gpu-case] rel err O {eo:.3e} S_final {es:.3e} tol {tol}", file=sys.__stderr__, flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("kind,first,second", [
    ("kda", dict(B=2, H=4, T=1000, s0_scale=0.3), dict(B=1, H=2, T=130)),
    ("dplr", dict(B=1, H=4, T=2100, s0_scale=0.3), dict(B=1, H=2, T=65)),  # segmented pass
    ("deltanet_f32", dict(), dict(T=100, H=1)),                            # fp32 kernels
])
def test_noalloc_two_calls_match_workspace_entry(kind, first, second):
    # two calls in a row on the one scratch array, the second on a smaller input
    for spec in (first, second):
        _check_pair(inputs.make_problem(kind, **spec))


def test_noalloc_packed_sequences_and_flags():
    P = inputs.make_problem("kda_varlen", n_seq=4, total=700, min_len=1, H=2)
    P.cu_seqlens = torch.tensor([0, 1, 300, 300, 700], dtype=torch.int32)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    O1, S1 = _run(P, no_alloc=False)
    O2, S2 = _run(P, no_alloc=True, flags=flags)
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
    assert int(flags.item()) == 0
    # malformed offsets are clamped and reported through `flags`
    P.cu_seqlens = torch.tensor([0, 100, 50, 650, 5000], dtype=torch.int32)
    P.S0 = None
    O3, _ = _run(P, no_alloc=True, flags=flags)
    assert int(flags.item()) == 1
    assert torch.isfinite(O3[:, :650].float()).all()


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    # the benchmark workload needs ~500 MB of workspace: refused before any launch
    need = gdr.workspace_bytes(2, 32, 8192, 128, 128)
    assert need > gdr.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(2, 8192, 32, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(2, 8192, 32, 128, dtype=torch.bfloat16, device="cuda")
    beta = torch.zeros(2, 8192, 32, dtype=torch.float32, device="cuda")
    la = torch.zeros(2, 8192, 32, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_fwd(q, q, v, beta, log_alpha=la, no_alloc=True)
    assert e.value.code == -4


def test_noalloc_graph_capture_replays():
    # captured in a HIP graph and replayed on new inputs copied into the captured tensors:
    # every replay gives the bits of the workspace entry point on the same inputs
    problems = [inputs.make_problem("kda", seed=70 + i, B=1, H=2, T=300, s0_scale=0.3) for i in range(3)]
    P0 = problems[0]
    names = ("q", "k", "v", "beta", "log_alpha", "S0")
    dev = {n: getattr(P0, n).to("cuda").clone() for n in names}
    out = torch.empty_like(dev["v"])
    fs = torch.empty_like(dev["S0"])
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        gdr.chunk_fwd(dev["q"], dev["k"], dev["v"], dev["beta"], log_alpha=dev["log_alpha"],
                      S0=dev["S0"], no_alloc=True, flags=flags, out=out, final_state=fs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for P in problems[1:] + problems[:1]:
        for n in names:
            dev[n].copy_(getattr(P, n).to("cuda"))
        graph.replay()
        torch.cuda.synchronize()
        O1, S1 = _run(P, no_alloc=False)
        assert torch.equal(out, O1) and torch.equal(fs, S1)
    assert int(flags.item()) == 0
