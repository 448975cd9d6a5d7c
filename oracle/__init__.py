"""CPU oracle for generalized paged attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  It shares no code with the
HIP library in ``paged_kv_token_amd``.
"""

from .definitions import (  # noqa: F401
    append_kv,
    causal_attention,
    default_positions,
    e4m3_decode,
    e4m3_encode,
    e4m3_value,
    E4M3_MAX,
    E4M3_VALUES,
    quantize_e4m3,
    gather_kv,
    kv_head_of,
    causal_visible,
    row_positions,
    paged_attention,
    partial_attention,
    partition_token_ranges,
    split_merge,
    split_partial,
    to_f64,
)
