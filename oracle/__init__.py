"""CPU fp64 oracle for exact attention.  Test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The GPU library never imports, links or calls it.
"""
from .attention import (  # noqa: F401
    attention_forward,
    attention_backward,
    forward_head,
    backward_head,
    forward_rows,
    dq_rows,
    online_softmax_row,
    online_attention_row,
    scores_head,
)
