"""fp64 CPU oracle for exact attention. Test infrastructure: only tests/,
the smoke check and the bench's CPU-baseline leg may use it."""
from .attention import (  # noqa: F401
    attention_backward,
    attention_forward,
    attention_head,
    causal_offset,
    online_softmax_stats,
    row_softmax,
    softmax_three_pass,
)
