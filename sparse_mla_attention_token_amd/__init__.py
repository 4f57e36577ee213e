"""Sparse MLA prefill attention for AMD MI355X (gfx950).

The attention (and the FP8 lightning indexer with its top-k stage that
produces the attention's index lists, and the dense MLA prefill with a
block-scaled FP8 K_rope) runs in hand-written HIP kernels behind the C ABI declared in
include/smla.h (libsmla.so); this package is the thin Python binding.
"""

from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    QK_DEPTH,
    V_DEPTH,
    SmlaDenseDims,
    SmlaDims,
    SmlaError,
    SmlaIndexDims,
    auto_splits,
    call_raw,
    load_library,
    make_dense_dims,
    make_dims,
    mla_dense_prefill,
    make_index_dims,
    noalloc_scratch_bytes,
    sparse_mla_gather_debug,
    sparse_mla_index_scores,
    sparse_mla_index_topk,
    sparse_mla_prefill,
    sparse_mla_prefill_split_noalloc,
    split_workspace_bytes,
    status_string,
    validate_dense_args,
    validate_index_scores_args,
    validate_index_topk_args,
    validate_prefill_args,
    version,
)
