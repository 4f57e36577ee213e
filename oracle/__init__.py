"""CPU float64 oracle for sparse MLA prefill attention.

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this package.  The product path never imports it.
"""

from .sparse_mla import (  # noqa: F401
    QK_DEPTH,
    V_DEPTH,
    decode_bf16,
    decode_e4m3fn,
    dequant_rows,
    error_metrics,
    gather_rows,
    sparse_mla_prefill,
    token_sequences,
    translate_rows,
)
