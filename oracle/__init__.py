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
    pool_after_append,
    pool_after_copy,
)
