"""FP64 CPU oracle (test infrastructure only; never used by the product path)."""
from .oracle import (append_ref, bf16_to_f64, decode_ref, fill_ref, merge_ref, partial_ref,  # noqa: F401
                     prefill_ref, prefill_rows_ref, scores_and_values)
