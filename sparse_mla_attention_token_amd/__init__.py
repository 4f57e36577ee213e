"""Sparse MLA prefill attention for AMD MI355X (gfx950).

The attention runs in hand-written HIP kernels behind the C ABI declared in
include/smla.h (libsmla.so); this package is the thin Python binding.
"""

from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    LIB_PATH,
    QK_DEPTH,
    V_DEPTH,
    SmlaDims,
    SmlaError,
    auto_splits,
    call_raw,
    load_library,
    make_dims,
    sparse_mla_gather_debug,
    sparse_mla_prefill,
    split_workspace_bytes,
    status_string,
    version,
)
