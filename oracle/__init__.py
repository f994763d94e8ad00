"""CPU float64 oracle for exact attention: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The HIP library never does, and this package imports nothing
from it.
"""
from .attention_oracle import (  # noqa: F401
    as_f64, to_bhnd, from_bhnd, kv_head_of, sdpa_ref, prefill_rows_ref,
    online_softmax_ref, pages_needed, gather_kv_ref, decode_ref, kv_cache_bytes,
)
