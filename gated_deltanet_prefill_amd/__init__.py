"""Gated delta rule (gated DeltaNet) forward pass for AMD Instinct MI355X.

The computation lives in ``libgdn.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/gdn.h``):

* :func:`chunk_fwd` -- T tokens in chunks of C against one read of the state
  (C = 0: the library chooses the kernel and the chunk length);
* :func:`seq_fwd`   -- T tokens one by one against one read of the state
  (short T);
* :func:`step`      -- one token (decode).

This package only marshals torch tensors (device memory, streams) into
those calls.
"""
from ._binding import (GDN_BF16, GDN_F16, GDN_F32, GDNError, LIB_PATH,  # noqa: F401
                       SUPPORTED_CHUNKS, SUPPORTED_DIMS, chunk_fwd, load, seq_fwd, status_string,
                       step)

__all__ = ["chunk_fwd", "seq_fwd", "step", "load", "status_string", "GDNError"]
