"""LoopVQ encoder and quantised decode attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libloopvq.so (C ABI in include/loopvq.h);
this package only marshals arguments to it.  There is no CPU fallback: the
functions raise if the library is missing.
"""
from ._lib import (  # noqa: F401
    LOOPVQ_DTYPE_BF16, LOOPVQ_DTYPE_F32, LoopVQError, loopvq_dims, lib, EXPORTED, LIB_PATH,
    loopvq_status_string, loopvq_row_bytes, loopvq_build_codebook_slices, loopvq_rope_table,
    loopvq_encode, loopvq_decode_workspace_bytes, loopvq_decode_attn, loopvq_decode_split,
    loopvq_decode_combine, loopvq_decode_attn_noalloc, NOALLOC_SCRATCH_BYTES, loopvq_bf16_window, loopvq_decode_attn_window, loopvq_encode_pages,
    loopvq_tasq, loopvq_encode_tasq_workspace_bytes, loopvq_encode_tasq, loopvq_decode_attn_tasq,
    loopvq_kmeans_workspace_bytes, loopvq_kmeans_update,
)
