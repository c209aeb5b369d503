"""fp64 CPU oracle for masked attention forward.

TEST INFRASTRUCTURE: only the test suite, the smoke entry point and the benchmark's CPU
baseline leg use it. The product library never imports it, and it imports nothing from the
product.
"""

from .attention import (  # noqa: F401
    ALIBI_MODES,
    alibi_bias,
    attention,
    attention_head,
    attention_rows,
    band_batch_index,
    count_visible_loops,
    tiled_attention,
    visible,
    visible_matrix,
)
from .backward import attention_backward, attention_head_backward  # noqa: F401
