"""fp64 CPU oracle for the fused attention forward and its gradients.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg. The product (scaled_dot_product_03_amd) never imports it, and it imports nothing from the
product. Every function states the passage of the pages it follows; the tests in
tests/test_oracle.py pin it to brute force, a library special case, closed forms, invariants and
hand-derived golden values.
"""
from .sdpa_ref import (  # noqa: F401
    MASK_NONE, MASK_CAUSAL, MASK_SLIDING, BIAS_NONE, BIAS_T5, BIAS_FULL, BIAS_ALIBI, BIAS_T5U,
    T5_NUM_BUCKETS, T5_MAX_DISTANCE,
    t5_bucket, t5u_bucket, visible, attend_rows, attention_weights, sdpa_rows, sdpa_forward,
    default_threads,
)
from .sdpa_bwd_ref import head_backward, sdpa_backward  # noqa: F401
from .sdpa_varlen_ref import sdpa_forward_varlen  # noqa: F401
