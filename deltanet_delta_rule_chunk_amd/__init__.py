"""MI355X (gfx950) DeltaNet delta-rule forward and decode step.

The computation lives in hand-written HIP kernels behind the C ABI of
``libdeltanet.so`` (include/deltanet.h); ``binding`` marshals PyTorch tensors
to it.  The library is loaded on first use and its absence is an error.
"""

from .binding import chunk_fwd, decode_step, delta_rule, load, workspace_bytes  # noqa: F401

__all__ = ["chunk_fwd", "decode_step", "delta_rule", "load", "workspace_bytes"]
