"""Plain, slow fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library; both sides only receive the same seeded inputs.

Every function is pinned by CPU tests against facts fixed outside this code
(worked examples from the pages, closed forms, a 50-digit brute-force
softmax, torch's scaled_dot_product_attention in fp64, bit-exact round
trips, invariances).  No function here is "parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    as_f64,
    cache_write,
    combine_splits,
    decode,
    decode_split_partials,
    gather,
    kv_head_of,
    prefill_chunk,
    slot_mapping,
    softmax_attention,
)
