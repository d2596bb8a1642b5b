"""MI355X (gfx950) causal linear attention: chunkwise forward (optionally from
raw projections, or normalised), its backward pass, decode step and the Gated
DeltaProduct forward and backward.

The compute runs in hand-written HIP kernels behind the C ABI of
``include/linattn.h`` (``liblinattn.so``); this package only marshals torch
tensors to it.  Importing the package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
from ._binding import (EXPORTS, LIB_PATH, LinattnError, abi_version, chunk_bwd,  # noqa: F401
                       chunk_bwd_workspace_bytes, chunk_fwd, chunk_fwd_normalized, chunk_fwd_save,
                       chunk_states_shape, chunk_workspace_bytes, decode_step, deltaproduct_bwd,
                       deltaproduct_bwd_workspace_bytes, deltaproduct_fwd,
                       deltaproduct_workspace_bytes, load, normalized_workspace_bytes,
                       status_string)

__all__ = ["chunk_fwd", "chunk_fwd_save", "chunk_bwd", "chunk_bwd_workspace_bytes",
           "chunk_states_shape", "chunk_fwd_normalized", "decode_step", "deltaproduct_fwd", "deltaproduct_bwd",
           "deltaproduct_bwd_workspace_bytes",
           "chunk_workspace_bytes", "normalized_workspace_bytes", "deltaproduct_workspace_bytes",
           "abi_version", "status_string", "load", "LinattnError", "LIB_PATH", "EXPORTS"]
