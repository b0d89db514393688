"""fp64 CPU oracle for MLA decode -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library does not use it and the
two share no code.
"""
from .mla_oracle import (  # noqa: F401
    D_LATENT,
    D_ROPE,
    SPLIT_BLOCK_ROWS,
    attend,
    cache_rows,
    combine,
    mla_decode_ref,
    mla_decode_split_ref,
    scores,
    softmax_stats,
    split_partial,
    split_ranges,
    to_f64,
    visible_rows,
    weighted_values,
)
