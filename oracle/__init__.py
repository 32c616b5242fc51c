"""Plain fp64 CPU oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke entry point
and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

What it computes and which passage of the source pages each function follows
is stated in the docstrings of ``attention_ref`` and ``fp8_ref``.  Every
function here is pinned by CPU tests against values the pages print, closed
forms, invariants, a library routine and pure-Python brute force
(tests/test_oracle.py, tests/test_oracle_fp8.py).
"""

from .attention_ref import (  # noqa: F401
    attention_fp64,
    attention_fp64_keys,
    attention_bwd_fp64,
    attention_bwd_fp64_rows,
    attention_fp64_key_range,
    attention_fp64_kv_cache,
    attention_fp64_paged,
    gather_paged,
    attention_bruteforce,
    attention_online_blocked,
    probabilities_fp64,
    kv_head_of,
    allowed_keys,
)
from .fp8_ref import (  # noqa: F401
    e4m3_decode,
    dequantize_e4m3,
    attention_fp8_fp64,
    fp8_p_rounding_bound,
    fp8_tolerances,
)
