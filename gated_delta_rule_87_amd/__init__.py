"""Chunkwise gated delta-rule forward for AMD MI355X (gfx950).

The compute path is ``libgdr.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/gdr.h``); :mod:`.binding` is a thin ctypes layer over it
that takes torch tensors for device memory and streams.  Importing this
package does not load the library; the first call into :mod:`.binding` does,
and fails loudly if it is missing.
"""
__all__ = ["binding", "inputs"]
