"""Plain CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import or run anything in this package;
the product path never does.  It is deliberately slow and written straight
from the definitions (see ``oracle.reference``), in float64.
"""
from .reference import (  # noqa: F401
    allowed_keys,
    append,
    attend_rows,
    attend_rows_matrix,
    bf16_to_f64,
    combine_partials,
    decode,
    decode_partials,
    gather,
    prefill_varlen,
    slot_mapping,
    split_page_range,
)
from .allocator import (  # noqa: F401
    ALLOC_OK,
    ALLOC_OUT_OF_PAGES,
    ALLOC_TABLE_FULL,
    FREE_OVERFLOW,
    page_alloc,
    page_free,
)
