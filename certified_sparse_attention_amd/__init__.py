"""Certified sparse attention via perturbed retrieval: the decode step of one layer, or of
a batch of items (requests, layers), on MI355X (gfx950), as hand-written HIP kernels
behind the C ABI in include/csa.h.

The Python layer only marshals torch tensors into the C ABI; the library must be
built (``_build.build()``) and there is no CPU fallback.
"""

from .api import (  # noqa: F401
    Event,
    PackedKV,
    allocate_workspace,
    certified_decode_attention,
    certified_decode_attention_batch,
    certified_decode_attention_noalloc,
    dense_decode_attention,
    pack_kv_4bit,
    scan_bounds,
    stream_read,
    workspace_bytes,
    workspace_bytes_batch,
)
