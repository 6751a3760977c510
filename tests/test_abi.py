"""C-ABI contract tests that run without a GPU: the library loads, exports
every function include/gdr.h declares, sizes workspaces, and rejects bad
arguments on the host before anything is enqueued.

Every call below that passes non-NULL pointers is one that validation rejects,
so no kernel is ever launched with them."""
import ctypes
import os
import re

import pytest

from chunkwise_gated_delta_amd import gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

P = ctypes.c_void_p
FAKE = 1 << 40  # never dereferenced: every such call fails validation first


def _header_functions():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gdr.load_library()


def test_exports_every_declared_function(lib):
    names = _header_functions()
    assert set(names) == set(gdr.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.gdr_version() >= 100
    for code in range(-7, 1):
        s = lib.gdr_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.gdr_status_string(-99).decode() == "unknown status"


def _align(x):
    return -(-x // 256) * 256


def test_workspace_sizes(lib):
    ws = gdr.workspace_bytes
    # KDA family (bf16): the error-flag header plus one 61952-byte block per (chunk, head)
    # at dk = 128 (37120 at dk = 64); with a gate, one int per (chunk, head) flags chunks
    # for the log-domain prep; then, with few chains, the segmented-pass area
    kda = lambda chains_chunks, blk, gated=True: _align(256 + chains_chunks * blk) + \
        (chains_chunks * 4 if gated else 0)
    assert ws(2, 32, 8192, 128, 128) == _align(kda(32 * 256, 61952))
    assert ws(4, 16, 4096, 128, 128, gate=gdr.GATE_HEAD) == _align(kda(16 * 256, 61952))
    assert ws(1, 2, 100, 64, 64, gate=gdr.GATE_NONE) == 256 + 2 * 2 * 37120
    # ... and, for packed sequences, the chunk offsets and room for every sequence
    # to end in a partial chunk
    assert ws(1, 32, 32768, 128, 128, n_seq=8) == _align(256 + 256 + 32 * 520 * 61952) + 32 * 520 * 4
    # DPLR (bf16, distinct a, b, C = 64): the same blocks plus Diag(beta) K^ (16 KiB).
    # With 16 (sequence, head) chains the state pass is cut into 3 runs (on 256 CUs):
    # start states of runs 1, 2, and R, P of run 1, fp32 [128][128] each, per chain
    assert ws(1, 16, 16384, 128, 128, has_ab=True) == \
        _align(kda(16 * 256, 61952 + 16384)) + 16 * 4 * 128 * 128 * 4
    assert ws(1, 2, 100, 64, 64, has_ab=True) == _align(kda(2 * 2, 37120 + 8192))
    # two chains of 32 chunks: 4 runs (3 start states, 2 R, 2 P per chain)
    assert ws(1, 2, 2048, 128, 128) == _align(kda(2 * 32, 61952)) + 2 * 7 * 128 * 128 * 4
    # the fp32 kernels (fp32 inputs, or other chunk sizes with a, b) keep one fp32 block
    # per (chunk, head): W', Q~, K^ (+ Diag(beta) K^) [C][dk], two [C][C], gamma [dk],
    # rounded up to 64 floats
    blk = lambda C, dk, dp: -(-((4 if dp else 3) * C * dk + 2 * C * C + dk) // 64) * 64 * 4
    assert ws(1, 2, 256, 64, 64, dtype=__import__("torch").float32, gate=0) == 256 + 2 * 4 * blk(64, 64, False)
    assert ws(1, 16, 16384, 128, 128, C=32, has_ab=True) == 256 + 16 * 512 * blk(32, 128, True)
    # unsupported / invalid -> 0
    assert ws(1, 2, 256, 96, 64) == 0
    assert ws(1, 2, 256, 128, 48) == 0
    assert ws(1, 2, 256, 128, 128, C=32) == 0           # bf16 KDA family: C = 64 only
    assert ws(0, 2, 256, 128, 128) == 0
    assert ws(2, 2, 256, 128, 128, n_seq=3) == 0        # packed sequences need B == 1


def _call(lib, q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), a=None, b=None,
          la=FAKE + (3 << 30), beta=FAKE + (4 << 30), S0=None, O=FAKE + (5 << 30),
          Sf=FAKE + (6 << 30), cu=None, n_seq=0, B=1, H=2, T=64, dk=128, dv=128, C=64,
          dtype=1, gate=2, ws=FAKE + (7 << 30), ws_bytes=1 << 20):
    return lib.gdr_chunk_fwd(P(q), P(k), P(v), P(a), P(b), P(la), P(beta), P(S0), P(O), P(Sf),
                             P(cu), n_seq, B, H, T, dk, dv, C, dtype, gate, P(ws), ws_bytes, None)


def test_backward_workspace_sizes(lib):
    # bf16, C = 64 only; DPLR needs larger forward blocks than KDA
    kda = lib.gdr_chunk_bwd_workspace(2, 4, 300, 128, 128, 64, 0, 1, 2, 0)
    dplr = lib.gdr_chunk_bwd_workspace(2, 4, 300, 128, 128, 64, 0, 1, 2, 1)
    assert kda > 0 and dplr > kda
    assert lib.gdr_chunk_bwd_workspace(2, 4, 300, 128, 128, 32, 0, 1, 2, 0) == 0  # C
    assert lib.gdr_chunk_bwd_workspace(2, 4, 300, 128, 128, 64, 0, 0, 2, 0) == 0  # fp32
    assert lib.gdr_chunk_bwd_workspace(2, 4, 300, 96, 128, 64, 0, 1, 2, 0) == 0   # dk
    assert lib.gdr_chunk_bwd_workspace(2, 4, 300, 128, 128, 64, 0, 1, 2 | gdr.GATE_CLIP, 0) == 0


def test_clip_flag_accepted_with_every_layout(lib):
    # the clip flag changes no buffer size, except that an ungated bf16 call gains the
    # per-chunk flags of the log-domain prep (a clipped gate can fall far)
    for dt, C, ab in [(1, 64, 0), (1, 64, 1), (0, 32, 0), (1, 16, 1)]:
        for layout in (0, 1, 2):
            plain = lib.gdr_chunk_fwd_workspace(2, 4, 300, 128, 128, C, 0, dt, layout, ab)
            assert plain > 0
            clipped = lib.gdr_chunk_fwd_workspace(2, 4, 300, 128, 128, C, 0, dt,
                                                  layout | gdr.GATE_CLIP, ab)
            if dt == 1 and C == 64 and layout == 0:
                assert clipped == _align(plain + 2 * 4 * 5 * 4)  # 40 (chunk, head) flags
            else:
                assert clipped == plain
    assert lib.gdr_chunk_fwd_workspace(2, 4, 300, 128, 128, 64, 0, 1, 3 | gdr.GATE_CLIP, 0) == 0
    assert lib.gdr_chunk_fwd_workspace(2, 4, 300, 128, 128, 64, 0, 1, 16, 0) == 0


def test_null_pointers_rejected(lib):
    assert _call(lib, q=None) == -1
    assert _call(lib, O=None) == -1
    assert _call(lib, beta=None) == -1
    assert _call(lib, a=FAKE + (9 << 30)) == -1           # only one of a, b
    assert _call(lib, la=None, gate=2) == -1              # gate without log_alpha
    assert _call(lib, gate=0) == -1                       # log_alpha without a gate
    assert _call(lib, gate=0 | gdr.GATE_CLIP) == -1       # ... also with the clip flag
    assert _call(lib, la=None, gate=2 | gdr.GATE_CLIP) == -1


def test_bad_shapes_rejected(lib):
    assert _call(lib, T=0) == -2
    assert _call(lib, B=0) == -2
    assert _call(lib, gate=3) == -2
    assert _call(lib, gate=3 | gdr.GATE_CLIP) == -2
    assert _call(lib, gate=8 | 2) == -2                   # unknown flag bit
    assert _call(lib, gate=-1) == -2
    assert _call(lib, cu=FAKE + (8 << 30), n_seq=2, B=2) == -2
    assert _call(lib, cu=FAKE + (8 << 30), n_seq=0) == -2


def test_size_bound(lib):
    # tokens x H x max(dk, dv) must stay below 2^40 elements per tensor (every global
    # offset is 64-bit; job and chain indices stay 32-bit inside that bound)
    ws = gdr.workspace_bytes
    assert ws(1, 1 << 10, (1 << 23) - 64, 128, 128) > 0
    assert ws(1, 1 << 10, 1 << 23, 128, 128) == 0
    assert ws(1 << 10, 1 << 10, 1 << 13, 64, 128) == 0      # the larger head size counts
    assert ws(1 << 20, 1 << 20, 1 << 20, 64, 64) == 0       # no 32-bit wrap in the check
    assert _call(lib, B=1, H=1 << 10, T=1 << 23) == -2
    assert gdr.bwd_workspace_bytes(1, 1 << 10, 1 << 23, 128, 128) == 0
    # and fewer than 2^27 (sequence, head) chains (the serial kernels count workgroups in
    # 32 bits)
    assert ws((1 << 17) - 1, 1 << 10, 1, 64, 64) > 0
    assert ws(1 << 17, 1 << 10, 1, 64, 64) == 0
    assert ws(1, 1 << 10, 1 << 20, 64, 64, n_seq=1 << 17) == 0
    assert ws(1, 1 << 10, 1 << 20, 64, 64, n_seq=(1 << 17) - 1) > 0


def test_unsupported_rejected(lib):
    assert _call(lib, dk=96) == -3
    assert _call(lib, dv=40) == -3
    assert _call(lib, C=32) == -3
    assert _call(lib, dtype=5) == -3


def test_workspace_checked(lib):
    assert _call(lib, ws=None) == -4
    assert _call(lib, ws_bytes=100) == -4


def test_aliasing_rejected(lib):
    assert _call(lib, O=FAKE) == -5                       # O on top of q
    assert _call(lib, Sf=FAKE + (2 << 30)) == -5          # S_final on top of v
    assert _call(lib, S0=FAKE + (10 << 30), Sf=FAKE + (10 << 30) + 64) == -5  # partial overlap
    assert _call(lib, ws=FAKE + (5 << 30)) == -5          # workspace on top of O


def test_misaligned_pointers_rejected(lib):
    # every tensor and the workspace must start on a 16-byte boundary: a contiguous view
    # with a storage offset (here 2 bytes: one bf16 element) is refused before any launch
    assert _call(lib, q=FAKE + 2) == -7
    assert _call(lib, v=FAKE + (2 << 30) + 8) == -7
    assert _call(lib, beta=FAKE + (4 << 30) + 4) == -7
    assert _call(lib, O=FAKE + (5 << 30) + 2) == -7
    assert _call(lib, ws=FAKE + (7 << 30) + 2) == -7
    assert _call_for_bwd(lib, q=FAKE + 2) == -7
    assert lib.gdr_status_string(-7).decode() != "unknown status"
    # the backward: dq offset by one bf16 element
    ptrs = [P(FAKE + (i << 30)) for i in range(19)]
    ptrs[3] = ptrs[4] = ptrs[13] = ptrs[14] = P(None)  # no a, b (and no da, db)
    ptrs[18] = P(None)                                  # no cu_seqlens
    ptrs[10] = P(FAKE + (10 << 30) + 2)
    args = ptrs + [0, 1, 2, 64, 128, 128, 64, 1, 2]
    assert lib.gdr_chunk_bwd(*args, 0, P(FAKE + (30 << 30)), 1 << 40, None) == -7


def _call_noalloc(lib, **kw):
    """gdr_chunk_fwd_noalloc with _call's defaults (B=1, H=2, T=64, channel gate)."""
    d = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), a=None, b=None,
             la=FAKE + (3 << 30), beta=FAKE + (4 << 30), S0=None, O=FAKE + (5 << 30),
             Sf=FAKE + (6 << 30), cu=None, n_seq=0, B=1, H=2, T=64, dk=128, dv=128, C=64,
             dtype=1, gate=2, flags=None)
    d.update(kw)
    return lib.gdr_chunk_fwd_noalloc(P(d["q"]), P(d["k"]), P(d["v"]), P(d["a"]), P(d["b"]),
                                     P(d["la"]), P(d["beta"]), P(d["S0"]), P(d["O"]), P(d["Sf"]),
                                     P(d["cu"]), d["n_seq"], d["B"], d["H"], d["T"], d["dk"],
                                     d["dv"], d["C"], d["dtype"], d["gate"], P(d["flags"]), None)


def test_noalloc_validated_before_any_setup(lib):
    # the host checks of gdr_chunk_fwd, in the same order, then the scratch size: none of
    # these calls reaches the device (the scratch is set up only after them)
    assert _call_noalloc(lib, q=None) == -1
    assert _call_noalloc(lib, T=0) == -2
    assert _call_noalloc(lib, C=32) == -3
    assert _call_noalloc(lib, q=FAKE + 2) == -7
    assert _call_noalloc(lib, flags=FAKE + (8 << 30) + 2) == -7   # an int: 4-byte aligned
    assert _call_noalloc(lib, O=FAKE) == -5
    # more than the fixed array holds: refused, whatever the inputs
    big = dict(B=2, H=32, T=8192)
    assert lib.gdr_chunk_fwd_workspace(2, 32, 8192, 128, 128, 64, 0, 1, 2, 0) > gdr.NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(lib, **big) == -4
    # the documented size of the array matches the binding's constant
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    m = re.search(r"#define GDR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdr.NOALLOC_SCRATCH_BYTES


def test_backward_flags_validated(lib):
    # pointers are never dereferenced: validation fails before any launch
    ptrs = [P(FAKE + (i << 30)) for i in range(19)]
    ptrs[3] = ptrs[4] = ptrs[13] = ptrs[14] = P(None)  # no a, b (and no da, db)
    ptrs[18] = P(None)                                  # no cu_seqlens
    args = ptrs + [0, 1, 2, 64, 128, 128, 64, 1, 2]
    for flags, want in [(4, -2), (8, -2), (-1, -2)]:
        assert lib.gdr_chunk_bwd(*args, flags, P(FAKE + (30 << 30)), 16, None) == want
    # valid flags get past that check (and then fail on the too-small workspace)
    for flags in (1, 2, 3):
        assert lib.gdr_chunk_bwd(*args, flags, P(FAKE + (30 << 30)), 16, None) == -4


def _call_for_bwd(lib, **kw):
    """gdr_chunk_fwd_for_bwd with _call's defaults (B=1, H=2, T=64, channel gate)."""
    d = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), a=None, b=None,
             la=FAKE + (3 << 30), beta=FAKE + (4 << 30), S0=None, O=FAKE + (5 << 30),
             Sf=FAKE + (6 << 30), cu=None, n_seq=0, B=1, H=2, T=64, dk=128, dv=128, C=64,
             dtype=1, gate=2, ws=FAKE + (7 << 30), ws_bytes=1 << 20)
    d.update(kw)
    return lib.gdr_chunk_fwd_for_bwd(P(d["q"]), P(d["k"]), P(d["v"]), P(d["a"]), P(d["b"]),
                                     P(d["la"]), P(d["beta"]), P(d["S0"]), P(d["O"]), P(d["Sf"]),
                                     P(d["cu"]), d["n_seq"], d["B"], d["H"], d["T"], d["dk"],
                                     d["dv"], d["C"], d["dtype"], d["gate"], P(d["ws"]),
                                     d["ws_bytes"], None)


def test_forward_for_backward_validated(lib):
    # the forward that keeps its states for the backward takes only what the backward
    # supports, and the backward's workspace; every case fails before any launch
    fwd = lib.gdr_chunk_fwd_workspace(1, 2, 64, 128, 128, 64, 0, 1, 2, 0)
    bwd = lib.gdr_chunk_bwd_workspace(1, 2, 64, 128, 128, 64, 0, 1, 2, 0)
    assert bwd > fwd > 0
    assert _call_for_bwd(lib, ws_bytes=fwd) == -4               # the forward's size is short
    assert _call_for_bwd(lib, ws=None) == -4
    assert _call_for_bwd(lib, gate=2 | gdr.GATE_CLIP) == -3     # no clipped backward
    assert _call_for_bwd(lib, dtype=0, C=32) == -3              # fp32: forward only
    assert _call_for_bwd(lib, q=None) == -1
    assert _call_for_bwd(lib, O=FAKE) == -5
