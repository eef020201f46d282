"""CPU oracle for paged decode and its cache edits -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library and the HIP
library never calls it.
"""
from .oracle import (  # noqa: F401
    bf16_bits_to_f64,
    copy_blocks,
    dense_attention,
    gather_sequence,
    kv_cache_write,
    paged_attention_decode,
    paged_attention_decode_partitioned,
    paged_attention_decode_rows,
    slot_of,
    to_f64,
)
