"""Plain CPU oracle of the predictive sparse-KV decode path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.
"""
from .dd_oracle import (  # noqa: F401
    BF16,
    F32,
    F64,
    append_rows,
    attend_rows,
    attention_weights,
    bookkeeping,
    chunk_rows,
    default_scale,
    gather_rows,
    landmarks,
    layer_step,
    masked_attention,
    resident_fetches,
    scaled_logits,
    select_topk,
    upcast,
)
