"""Seeded synthetic inputs for generalized paged attention.

This package only draws inputs: request lengths, block placement, slot
mappings, query positions and Q/K/V values.  It holds none of the attention
arithmetic, so both the CPU oracle (``oracle/``) and the GPU path can consume
the same batches without sharing any computation.
"""

from .batches import (  # noqa: F401
    Batch,
    CONFIG_NAMES,
    DTYPE_BYTES,
    bf16_bits_from_f32,
    config_batch,
    conversation_script,
    custom_batch,
    draw_rows,
    storage_dtype,
)
