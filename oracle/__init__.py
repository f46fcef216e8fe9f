"""CPU float64 oracle for exact attention: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product (the HIP library and its binding) never does.
"""
from .attention import (  # noqa: F401
    attention_backward,
    attention_backward_key_tail,
    attention_backward_rows,
    attention_cross,
    attention_decode,
    attention_forward,
    attention_forward_gqa,
    attention_forward_varlen,
    attention_forward_online,
    attention_rows,
    attention_split_k,
    backward_delta,
    merge_partials,
    online_softmax_stats,
    scores,
    softmax_stats,
    split_partial,
)
from . import fp8  # noqa: F401,E402  (block-scaled E4M3 quantizer and the FP8 Q K^T reference)
