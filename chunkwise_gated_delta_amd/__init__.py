"""Chunkwise gated delta-rule forward pass for AMD MI355X (gfx950).

``chunk_fwd`` runs the hand-written HIP kernels of ``libgdr.so`` through its C ABI.
The library is loaded on first use; importing this package touches no GPU.
"""
__all__ = ["chunk_fwd", "workspace_bytes"]


def __getattr__(name):
    if name in ("chunk_fwd", "workspace_bytes"):
        from . import gdr
        return getattr(gdr, name)
    raise AttributeError(name)
