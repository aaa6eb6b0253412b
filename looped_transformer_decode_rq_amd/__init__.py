"""ResidualQuant decode attention on MI355X: Python binding of librq.so.

Every entry point mirrors a C function of ``include/rq.h`` and only marshals
arguments (device pointers from torch tensors, the current HIP stream); all
computation runs in the HIP kernels of the library. Importing this package
does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    RQ_DTYPE_BF16, RQ_DTYPE_F16, RQ_DTYPE_F32, RQ_MODE_RESIDUAL, RQ_MODE_DIRECT, RqError, RqLayout, RqDecodeOpts,
    lib, library_path, make_layout, layout_check, pool_bytes, record_bytes, record_offset,
    encode_pack, encode_workspace_bytes, decode_workspace_bytes, decode_auto_split_pages, decode_attention, decode_attention_noalloc,
    RQ_NOALLOC_SCRATCH_BYTES, bf16_workspace_bytes,
    bf16_auto_split_pages, chunk_workspace_bytes, chunk_attention,
    bf16_decode_attention, bf16_write, status_string, fit_rotation, fit_rotation_device, fit_workspace_bytes,
    decode_stream_probe, read_probe, EXPORTED,
)
