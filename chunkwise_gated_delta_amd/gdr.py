"""Python binding of libgdr.so: argument marshalling only.

Every step of the forward pass runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_F32, GDR_BF16 = 0, 1
GATE_NONE, GATE_HEAD, GATE_CHANNEL = 0, 1, 2
GATE_CLIP = 4  # flag: spectral clipping of the gate, alpha <- min(alpha, 1/||I - b a^T||_2)
STATUS = {0: "GDR_OK", -1: "GDR_ERR_NULL", -2: "GDR_ERR_SHAPE", -3: "GDR_ERR_UNSUPPORTED",
          -4: "GDR_ERR_WORKSPACE", -5: "GDR_ERR_ALIAS", -6: "GDR_ERR_HIP", -7: "GDR_ERR_ALIGN"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDR_NOALLOC_SCRATCH_BYTES
EXPORTS = ("gdr_chunk_fwd", "gdr_chunk_fwd_for_bwd", "gdr_chunk_fwd_noalloc",
           "gdr_chunk_fwd_workspace", "gdr_chunk_bwd",
           "gdr_chunk_bwd_workspace",
           "gdr_workspace_error", "gdr_status_string", "gdr_version")

_lib = None
_lock = threading.Lock()
_ws_cache = {}


class GdrError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libgdr.so and declare its C signatures (no GPU is touched)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.gdr_chunk_fwd.restype = I
        lib.gdr_chunk_fwd.argtypes = [P] * 11 + [I] * 9 + [P, Z, P]
        lib.gdr_chunk_fwd_for_bwd.restype = I
        lib.gdr_chunk_fwd_for_bwd.argtypes = [P] * 11 + [I] * 9 + [P, Z, P]
        lib.gdr_chunk_fwd_noalloc.restype = I
        lib.gdr_chunk_fwd_noalloc.argtypes = [P] * 11 + [I] * 9 + [P, P]
        lib.gdr_chunk_fwd_workspace.restype = Z
        lib.gdr_chunk_fwd_workspace.argtypes = [I] * 10
        lib.gdr_chunk_bwd.restype = I
        lib.gdr_chunk_bwd.argtypes = [P] * 19 + [I] * 10 + [P, Z, P]
        lib.gdr_chunk_bwd_workspace.restype = Z
        lib.gdr_chunk_bwd_workspace.argtypes = [I] * 10
        lib.gdr_workspace_error.restype = I
        lib.gdr_workspace_error.argtypes = [P, P]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_status_string.argtypes = [I]
        lib.gdr_version.restype = I
        lib.gdr_version.argtypes = []
        _lib = lib
        return lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return GDR_F32
    if dt == torch.bfloat16:
        return GDR_BF16
    raise TypeError(f"unsupported element type {dt}; use float32 or bfloat16")


def workspace_bytes(B, H, T, dk, dv, C=64, n_seq=0, dtype=torch.bfloat16, gate=GATE_CHANNEL,
                    has_ab=False) -> int:
    """Workspace bytes for these arguments (gate may carry GATE_CLIP); 0 if unsupported."""
    lib = load_library()
    return int(lib.gdr_chunk_fwd_workspace(B, H, T, dk, dv, C, n_seq, _dtype_code(dtype), gate,
                                           int(bool(has_ab))))


def _ws_key(device: torch.device):
    return (device.type, device.index, torch.cuda.current_stream(device).cuda_stream)


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """The default workspace of the current stream on `device` (grown on demand).

    One buffer per (device, stream): calls that pass no workspace on different
    streams never share one.  The buffer is allocated on that stream and used only
    there, so when it is replaced by a larger one the caching allocator hands the old
    memory out again only to work ordered after everything already enqueued on it.
    """
    key = _ws_key(device)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              log_alpha: Optional[torch.Tensor] = None, a: Optional[torch.Tensor] = None,
              b: Optional[torch.Tensor] = None, S0: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_final_state: bool = True, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              clip: bool = False, for_backward: bool = False, no_alloc: bool = False,
              flags: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise forward of S_t = S_{t-1} Diag(alpha_t)(I - b_t a_t^T) + beta_t v_t k_t^T, o_t = S_t q_t.

    clip=True clips the gate per token to min(alpha_t, 1/||I - b_t a_t^T||_2)
    (spectral clipping of the GDN2 stability notes, eq. 7; GATE_CLIP in the C ABI).

    for_backward=True (gdr_chunk_fwd_for_bwd): also leave the per-chunk states in
    `workspace` (required, sized by bwd_workspace_bytes) for a chunk_bwd call with
    forward_states=True on the same inputs.

    no_alloc=True (gdr_chunk_fwd_noalloc): the library's fixed per-GPU scratch array
    replaces the workspace (no workspace argument; at most NOALLOC_SCRATCH_BYTES of it);
    `flags`, a zeroed int32 device tensor of one element or None, receives the device
    error bits.  Calls that overlap on one GPU race on that array.  Pass `out` and
    `final_state` to keep the call free of allocations altogether.

    q, k, (a, b): [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H] fp32;
    log_alpha: None, [B, T, H] (head gate) or [B, T, H, dk] (channel gate), fp32;
    S0: None or [N, H, dv, dk] fp32; cu_seqlens: None or int32 [N+1] (then B == 1).
    Returns (O [B, T, H, dv] in q's dtype, S_final [N, H, dv, dk] fp32 or None).
    """
    lib = load_library()
    if not q.is_cuda:
        raise RuntimeError("chunk_fwd runs on the GPU only; move the tensors to a cuda device")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    tensors = dict(q=q, k=k, v=v, a=a, b=b, log_alpha=log_alpha, beta=beta, S0=S0,
                   cu_seqlens=cu_seqlens)
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name in ("k", "a", "b"):
        t = tensors[name]
        if t is not None and (t.shape != q.shape or t.dtype != q.dtype):
            raise ValueError(f"{name} must match q in shape and dtype")
    if v.shape[:3] != q.shape[:3] or v.dtype != q.dtype:
        raise ValueError("v must be [B, T, H, dv] in q's dtype")
    if beta.shape != q.shape[:3] or beta.dtype != torch.float32:
        raise ValueError("beta must be [B, T, H] float32")
    if log_alpha is None:
        gate = GATE_NONE
    elif log_alpha.dim() == 3 and log_alpha.shape == q.shape[:3]:
        gate = GATE_HEAD
    elif log_alpha.shape == q.shape:
        gate = GATE_CHANNEL
    else:
        raise ValueError("log_alpha must be [B, T, H] or [B, T, H, dk]")
    if log_alpha is not None and log_alpha.dtype != torch.float32:
        raise ValueError("log_alpha must be float32")
    if clip:
        gate |= GATE_CLIP
    n_seq = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        n_seq = cu_seqlens.numel() - 1
    N = n_seq if cu_seqlens is not None else B
    if S0 is not None and (S0.shape != (N, H, dv, dk) or S0.dtype != torch.float32):
        raise ValueError(f"S0 must be [{N}, {H}, {dv}, {dk}] float32")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    if not output_final_state:
        final_state = None
    with torch.cuda.device(q.device):  # the size depends on the device's CU count
        need = int(lib.gdr_chunk_fwd_workspace(B, H, T, dk, dv, chunk_size, n_seq, dt, gate,
                                               int(a is not None)))
    if need == 0:
        raise GdrError(-3, f"no kernel for dtype={q.dtype} dk={dk} dv={dv} C={chunk_size}")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if no_alloc:
        if for_backward or workspace is not None:
            raise ValueError("no_alloc=True takes neither a workspace nor for_backward")
        if flags is not None and (flags.dtype != torch.int32 or flags.device != q.device):
            raise ValueError("flags must be an int32 tensor on q's device")
        with torch.cuda.device(q.device):
            rc = lib.gdr_chunk_fwd_noalloc(
                _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha), _ptr(beta),
                _ptr(S0), _ptr(out), _ptr(final_state), _ptr(cu_seqlens), n_seq, B, H, T, dk, dv,
                chunk_size, dt, gate, _ptr(flags), ctypes.c_void_p(stream))
        if rc != 0:
            raise GdrError(rc, lib.gdr_status_string(rc).decode())
        return out, final_state
    if workspace is None:
        if for_backward:
            raise ValueError("for_backward=True needs the workspace the backward will use")
        workspace = _workspace(q.device, need)
    entry = lib.gdr_chunk_fwd_for_bwd if for_backward else lib.gdr_chunk_fwd
    with torch.cuda.device(q.device):
        rc = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha),
                               _ptr(beta), _ptr(S0), _ptr(out), _ptr(final_state),
                               _ptr(cu_seqlens), n_seq, B, H, T, dk, dv, chunk_size, dt, gate,
                               _ptr(workspace), workspace.numel(), ctypes.c_void_p(stream))
    if rc != 0:
        raise GdrError(rc, lib.gdr_status_string(rc).decode())
    return out, final_state


def check_workspace_error(workspace: Optional[torch.Tensor] = None, device=None) -> int:
    """Synchronise and return (and clear) the device error flag of a workspace."""
    lib = load_library()
    if workspace is None:
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        workspace = _ws_cache.get(_ws_key(dev))
        if workspace is None:
            return 0
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    return int(lib.gdr_workspace_error(_ptr(workspace), ctypes.c_void_p(stream)))


def bwd_workspace_bytes(B, H, T, dk, dv, C=64, n_seq=0, dtype=torch.bfloat16,
                        gate=GATE_CHANNEL, has_ab=False) -> int:
    """Workspace bytes of chunk_bwd for these arguments; 0 if unsupported."""
    lib = load_library()
    return int(lib.gdr_chunk_bwd_workspace(B, H, T, dk, dv, C, n_seq, _dtype_code(dtype), gate,
                                           int(bool(has_ab))))


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
              dO: torch.Tensor, log_alpha: Optional[torch.Tensor] = None,
              a: Optional[torch.Tensor] = None, b: Optional[torch.Tensor] = None,
              S0: Optional[torch.Tensor] = None, dS_final: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              want_dS0: bool = True, workspace: Optional[torch.Tensor] = None,
              forward_workspace: bool = False, forward_states: bool = False) -> dict:
    """Gradients of <dO, O> + <dS_final, S_final> for chunk_fwd.

    Shapes as in chunk_fwd; dO like O, dS_final like S_final (None: zero).
    Returns a dict with dq, dk, dv (q's dtype), dbeta, da and db (with a, b),
    dlog_alpha (when a gate is given) and dS0 (fp32, when want_dS0).

    forward_workspace=True: `workspace` is the one the chunk_fwd call on the same inputs
    filled (sized for both, see bwd_workspace_bytes); its per-chunk factors are reused
    (GDR_BWD_FORWARD_WORKSPACE).  The caller guarantees the inputs are the same.
    forward_states=True: the same for a workspace chunk_fwd(for_backward=True) filled; its
    per-chunk states are reused too (GDR_BWD_FORWARD_STATES).
    """
    lib = load_library()
    if not q.is_cuda:
        raise RuntimeError("chunk_bwd runs on the GPU only; move the tensors to a cuda device")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q.dtype)
    tensors = dict(q=q, k=k, v=v, a=a, b=b, beta=beta, dO=dO, log_alpha=log_alpha, S0=S0,
                   dS_final=dS_final, cu_seqlens=cu_seqlens)
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name in ("k", "a", "b"):
        t = tensors[name]
        if t is not None and (t.shape != q.shape or t.dtype != q.dtype):
            raise ValueError(f"{name} must match q in shape and dtype")
    if (a is None) != (b is None):
        raise ValueError("give both a and b, or neither")
    if v.shape[:3] != q.shape[:3] or v.dtype != q.dtype:
        raise ValueError("v must be [B, T, H, dv] in q's dtype")
    if dO.shape != v.shape or dO.dtype != q.dtype:
        raise ValueError("dO must match v in shape and dtype")
    if beta.shape != q.shape[:3] or beta.dtype != torch.float32:
        raise ValueError("beta must be [B, T, H] float32")
    if log_alpha is None:
        gate = GATE_NONE
    elif log_alpha.dim() == 3 and log_alpha.shape == q.shape[:3]:
        gate = GATE_HEAD
    elif log_alpha.shape == q.shape:
        gate = GATE_CHANNEL
    else:
        raise ValueError("log_alpha must be [B, T, H] or [B, T, H, dk]")
    if log_alpha is not None and log_alpha.dtype != torch.float32:
        raise ValueError("log_alpha must be float32")
    n_seq = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        n_seq = cu_seqlens.numel() - 1
    N = n_seq if cu_seqlens is not None else B
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and (t.shape != (N, H, dv, dk) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be [{N}, {H}, {dv}, {dk}] float32")
    with torch.cuda.device(q.device):  # the size depends on the device's CU count
        need = int(lib.gdr_chunk_bwd_workspace(B, H, T, dk, dv, chunk_size, n_seq, dt, gate,
                                               int(a is not None)))
    if need == 0:
        raise GdrError(-3, f"no backward kernel for dtype={q.dtype} dk={dk} dv={dv} C={chunk_size}")
    if (forward_workspace or forward_states) and workspace is None:
        raise ValueError("forward_workspace / forward_states need the workspace chunk_fwd used")
    flags = 2 if forward_states else (1 if forward_workspace else 0)
    if workspace is None:
        workspace = _workspace(q.device, need)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dbeta": torch.empty_like(beta)}
    if a is not None:
        out["da"] = torch.empty_like(a)
        out["db"] = torch.empty_like(b)
    if log_alpha is not None:
        out["dlog_alpha"] = torch.empty_like(log_alpha)
    if want_dS0:
        out["dS0"] = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = lib.gdr_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(log_alpha),
                               _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]),
                               _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("da")),
                               _ptr(out.get("db")), _ptr(out.get("dlog_alpha")),
                               _ptr(out["dbeta"]), _ptr(out.get("dS0")), _ptr(cu_seqlens),
                               n_seq, B, H, T, dk, dv,
                               chunk_size, dt, gate, flags, _ptr(workspace),
                               workspace.numel(), ctypes.c_void_p(stream))
    if rc != 0:
        raise GdrError(rc, lib.gdr_status_string(rc).decode())
    return out
