"""Compressed-domain KV-cache attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libtq.so`` (``include/tq.h``):
argument marshalling only.  Every step of the write and read paths runs in
the library's HIP kernels; PyTorch provides device memory (tensors) and the
stream (``torch.cuda.current_stream()``).  Importing this package without a
built ``libtq.so`` raises: there is no fallback.

Build the library with ``python compressed_domain_attention_kv_amd/build.py``.
"""

from ._binding import (  # noqa: F401
    CB_LLOYD_MAX,
    CB_QUANTILE_MEAN,
    FMT_GQ2V,
    FMT_GQ4V,
    FMT_PQ3,
    FMT_PQ4,
    FMT_TQ3K,
    Codebook,
    Layout,
    RING_CAP_MAX,
    STATIC_SCRATCH_BYTES,
    TQError,
    build_codebook,
    cache_bytes,
    decode_attention,
    decode_attention_static,
    decode_attention_hybrid,
    decode_combine,
    decode_hybrid_workspace_bytes,
    decode_partial,
    decode_partial_from_query,
    decode_partial_sparse_v,
    decode_step,
    decode_splits,
    decode_workspace,
    decode_workspace_bytes,
    decode_workspace_init,
    lib,
    library_path,
    quantize_append,
    quantize_rotated,
    ring_append,
    ring_bytes,
    ring_flush,
    rotate_sketch_query,
    strerror,
    vector_bytes,
    version,
)
