"""float64 CPU oracle for the fused exact attention forward and its
backward pass.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke
check and the benchmark's CPU-baseline leg, never by the GPU library.
"""
from .attention import (  # noqa: F401
    visible_mask, column_visible, kv_head_of, reference_attention, tiled_online_attention,
    splitkv_partials, merge_partials, splitkv_attention, split_bounds,
)
from .backward import (  # noqa: F401
    reference_attention_backward, recompute_backward,
)
from .paged import paged_rows, paged_attention, kvlen_attention  # noqa: F401
from .fp8 import decode_e4m3, reference_attention_fp8  # noqa: F401
