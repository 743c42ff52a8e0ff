"""Float64 CPU oracle for exact attention. TEST INFRASTRUCTURE ONLY: imported by
the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
HIP library or its Python binding."""
from .attention import (  # noqa: F401
    MiB, kv_cache_bytes, attention_head_rows, attention_ref, score_bytes, softmax_stats, softmax_weights,
    visible_pairs, gather_paged, attention_paged_ref, e4m3_value, dequant_e4m3, attention_fp8kv_ref,
)
from .backward import attention_backward_ref  # noqa: F401,E402
