"""Plain, slow CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The GPU library never imports, links or calls it, and it shares no
code with the GPU library.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, invariants, finite differences and an independent library
routine); nothing in this package is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_forward_gqa,
    attention_backward_gqa,
    attention_probs,
    key_range,
    keys_per_row,
    softmax_block_stats,
    merge_softmax_blocks,
    merge_partial_outputs,
    forward_rows,
    backward_dq_rows,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_round,
    fwht_f32,
    quantize_head,
    attention_forward_fp8,
)
from .pattern import (  # noqa: F401
    Pattern,
    attention_forward_pattern,
    attention_backward_pattern,
)
