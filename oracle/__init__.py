"""CPU oracle for bidirectional varlen multi-head attention with rotary
position embedding, forward and backward, in float64; key-range partials and
their merge; size-aware bucket batching (batching.py).

TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

Every function is the plain definition written out with numpy, one
(sequence, head) slice at a time, with no tiling, fusion or reordering.
"""

from .attention import (  # noqa: F401
    bf16_bits_to_f64,
    round_to_bf16,
    rope_frequencies,
    rope_rotate,
    rope_rotate_f32,
    query_operand_bf16,
    attention_forward_slice,
    attention_forward_partial_slice,
    merge_partials,
    attention_backward_slice,
    attention_rows_slice,
    forward,
    backward,
)
from . import tolerances  # noqa: F401
