"""Oracle package: test infrastructure only (see fa_back_oracle's header)."""
from .fa_back_oracle import (  # noqa: F401
    flash_attn_back, flash_attn_back_loops, key_rows, nmse, problem_arrays, query_rows,
    run_problem, widen,
)
