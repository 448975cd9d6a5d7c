"""Test-side glue: run the CPU oracle on a seeded batch."""

from __future__ import annotations

import numpy as np

import oracle
from workloads import Batch, storage_dtype

BF16_NAN = np.uint16(0x7FC0)


def poison_fill(dtype: str):
    return BF16_NAN if dtype == "bf16" else np.nan


def oracle_pools(batch: Batch, impl=oracle, poison=True, include_new=True, kv_fp8=None):
    """Pools [NB][Hkv][B][d] (K and V) filled through ``impl.append_kv``.

    Every slot starts as NaN (poison), then cached history and (optionally)
    the step's new rows are appended.  kv_fp8 = (k_scale, v_scale): the pools
    hold E4M3 codes (uint8) of the rows divided by the scales.
    """
    nb, hkv, B, d = batch.num_blocks, batch.num_kv_heads, batch.block_size, batch.head_dim
    if kv_fp8 is None:
        sd, fill = storage_dtype(batch.dtype), (poison_fill(batch.dtype) if poison else 0)
        enc_k = enc_v = lambda x: x
    else:
        sd, fill = np.uint8, (0x7F if poison else 0)
        enc_k = lambda x: oracle.quantize_e4m3(x, batch.dtype, kv_fp8[0])
        enc_v = lambda x: oracle.quantize_e4m3(x, batch.dtype, kv_fp8[1])
    k_pool = np.full((nb, hkv, B, d), fill, dtype=sd)
    v_pool = np.full((nb, hkv, B, d), fill, dtype=sd)
    for r, k, v, slots, pos in batch.iter_requests():
        impl.append_kv(k_pool, v_pool, enc_k(k[pos]), enc_v(v[pos]), slots, B)
    if include_new:
        k_new, v_new = batch.new_kv()
        impl.append_kv(k_pool, v_pool, enc_k(k_new), enc_v(v_new), batch.new_slots, B)
    return k_pool, v_pool


def fp8_kw(kv_fp8):
    """Keyword arguments of the oracle's attention for E4M3 pools with scales kv_fp8."""
    return {} if kv_fp8 is None else dict(kv_dtype="e4m3", k_scale=kv_fp8[0], v_scale=kv_fp8[1])


def batch_q_pos(batch: Batch):
    return None if batch.has_default_positions else batch.q_pos


def oracle_output(batch: Batch, impl=oracle, pools=None, **kw):
    k_pool, v_pool = pools if pools is not None else oracle_pools(batch, impl)
    return impl.paged_attention(batch.q_all(), k_pool, v_pool, batch.block_tables, batch.context_lens,
                                batch.cu_q_lens, batch_q_pos(batch), batch.softmax_scale, batch.dtype, **kw)


def oracle_split(batch: Batch, num_partitions: int, impl=oracle, pools=None, **kw):
    k_pool, v_pool = pools if pools is not None else oracle_pools(batch, impl)
    return impl.split_partial(batch.q_all(), k_pool, v_pool, batch.block_tables, batch.context_lens,
                              batch.cu_q_lens, batch_q_pos(batch), batch.softmax_scale, batch.dtype,
                              num_partitions, **kw)


def request_rows_reference(batch: Batch, r: int, h: int, impl=oracle):
    """Oracle rows of (request r, query head h) from the request's logical K/V (no pool)."""
    q = oracle.to_f64(batch.request_q(r)[:, h, :], batch.dtype)
    k, v = batch.request_kv(r)
    g = impl.kv_head_of(h, batch.num_heads, batch.num_kv_heads)
    kk = oracle.to_f64(k[:, g, :], batch.dtype)
    vv = oracle.to_f64(v[:, g, :], batch.dtype)
    return impl.causal_attention(q, kk, vv, batch.query_positions(r), batch.softmax_scale)
