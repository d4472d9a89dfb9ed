"""fp64 CPU oracle for paged decode attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg import this
package; the product path never does.
"""
from .pkv_oracle import (  # noqa: F401
    DTYPE_BYTES,
    E4M3_MAX,
    KV_FORMATS,
    STORAGE_DTYPES,
    dequantize,
    e4m3_decode,
    e4m3_encode,
    gather_dequantized,
    kv_append_quantized,
    paged_decode_attention_quantized,
    quantize_row,
    gather_kv,
    kv_append,
    kv_bytes_per_token,
    kv_cache_bytes,
    merge_partitions,
    online_softmax_attention,
    online_softmax_partial,
    paged_decode_attention,
    paged_multi_query_attention,
    read_kv,
    softmax_two_pass,
    storage_to_f64,
)
