"""fp64 CPU oracle for the attention forward pass (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    LN2,
    LOG2E,
    attention_backward_blocked,
    attention_backward_sampled,
    attention_blocked,
    attention_fp8_blocked,
    attention_key_range,
    attention_naive,
    attention_online_tiled,
    attention_probs_naive,
    attention_rows,
    classify_tiles,
    fp8_e4m3_decode,
    kv_head_of,
    key_visibility,
    merge_partials,
    tile_plan,
)
