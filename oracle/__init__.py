"""CPU fp64 oracle for the attention forward (+lse) and backward.

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import anything under oracle/. The HIP
library and its Python binding never import it, and it imports nothing of
theirs.
"""
from .sdpa_oracle import (  # noqa: F401
    allowed_block,
    head_rows,
    rows_attending,
    sampled_keys,
    sampled_rows,
    sdpa_forward,
    sdpa_fwd_bwd,
)
