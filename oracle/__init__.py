"""Float64 CPU oracle for paged single-query decode attention.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the bench's CPU-baseline
leg are the only callers. The product path (the HIP library and its Python
binding) never imports anything from here, and nothing here imports the product.
"""

from .paged_attention import (  # noqa: F401
    block_and_slot,
    gather_sequence,
    dense_decode_attention,
    paged_decode_attention,
    paged_multi_query_attention,
    pool_after_append,
    pool_after_append_multi,
    pool_after_copy,
    pool_after_swap,
)
from .fp8 import (  # noqa: F401
    decode as fp8_decode,
    encode as fp8_encode,
    quantize as fp8_quantize,
    pool_after_append_fp8,
    pool_after_append_multi_fp8,
    dequantize_pool as fp8_dequantize_pool,
)
