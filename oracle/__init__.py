"""CPU float64 oracle (test infrastructure only; see mla_oracle's header)."""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (attend, combine, bf16_to_f64, e4m3_value, e4m3_to_f64, E4M3_TABLE,  # noqa: F401
                         visible_range, logical_rows, decode_paged, decode_paged_f64,
                         decode_sparse, decode_sparse_f64, sparse_rows, prefill_paged,
                         prefill_paged_f64)
