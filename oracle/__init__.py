"""CPU oracles for row-wise top-k index selection and the C128A metadata
build (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP path.
"""

from .topk_oracle import (  # noqa: F401
    check_row,
    is_untied,
    oracle_topk,
    oracle_page_slots,
    oracle_topk_row,
    row_view,
)
from .c128a_oracle import (  # noqa: F401
    active_width,
    next_pow2,
    oracle_c128a_metadata,
    visible_entries,
)
