"""Oracle for dynamic-mask attention with an additive bias -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation in fp64 (numpy) of what the
device path computes.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import it; the library itself never does, and the two share no
code.  See ``oracle/attention.py`` for the definitions and their sources.

Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself (PyTorch's scaled_dot_product_attention in fp64, finite
differences, closed forms, brute force and invariants).
"""
from .attention import (  # noqa: F401
    BLOCK,
    BF16_LOWEST_BITS,
    SKIP,
    PARTIAL,
    FULL,
    bf16_to_f64,
    attends,
    valid_rows,
    classify,
    classify_plane_rows,
    forward_rows,
    backward_rows,
    forward,
    backward,
    topk_mask,
)
