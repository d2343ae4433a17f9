"""MI355X (gfx950) Mamba-2 SSD layer core.

``forward`` (chunked / dual mode) and ``step`` (recurrent mode) call the
C ABI of include/ssd.h, whose four chunked-mode stages are also exposed one
by one (``dA_cumsum``, ``chunk_state``, ``state_passing``, ``chunk_scan``).
``backward`` gives the gradients of ``forward`` (the training pass).
``forward_noalloc`` is ``forward`` on the library's static scratch (no workspace, no
allocation).  ``forward_varlen`` runs packed variable-length batches (state reset at every
sequence start); ``forward_fused`` the same forward as one pass over the sequence per
(batch, head) with the state on chip.  ``selective_scan`` runs the Mamba-1 layer the SSD form replaces, for
comparison.
All computation runs in the library's hand-written HIP kernels; torch only
provides device memory and the stream.
"""
from .ssd import (SSD_BF16, SSD_F32, SSDError, backward, chunk_scan, chunk_state, dA_cumsum, forward,
                  forward_fused, forward_noalloc, forward_varlen, load_library, num_chunks, selective_scan, state_passing, status_string, step,
                  workspace_bytes)

__all__ = [
    "SSD_BF16", "SSD_F32", "SSDError", "backward", "chunk_scan", "chunk_state", "dA_cumsum", "forward", "forward_fused",
    "forward_noalloc",
    "forward_varlen",
    "load_library",
    "num_chunks", "selective_scan", "state_passing", "status_string", "step", "workspace_bytes",
]
