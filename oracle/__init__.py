"""CPU float64 oracles for sparse MLA prefill attention, the FP8 indexer and
dense MLA prefill with a block-scaled FP8 K_rope.

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline may use this package.  The product path never imports it.
"""

from .dense_mla import ROPE_DEPTH, dense_flops, mla_dense_prefill, rope_scale_columns  # noqa: F401
from .indexer import INDEX_DEPTH, UNUSED_SLOT, causal_counts, indexer_scores, key_rows, topk_select  # noqa: F401
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
