"""Float64 CPU oracle for online-softmax attention.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library or its binding.
"""
from .attention import (  # noqa: F401
    NEG_INF,
    attention_bwd_ref,
    attention_monoid,
    attention_ref,
    block_state,
    decode_combine,
    decode_paged_ref,
    decode_partials,
    decode_ref,
    finalize,
    identity_state,
    mask_matrix,
    merge,
    online_softmax_recurrence,
    paged_gather,
    scores,
    split_bounds,
)
