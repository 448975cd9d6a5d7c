"""CPU oracle for generalized paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path never calls it; it
shares no code, tables or helpers with the HIP library.

What it computes (plain definitions, slow on purpose; float64 by default, and float32 on
request -- the same code with its operands cast, used only to time the oracle as a CPU
baseline):

* ``append_kv`` -- each new token's K and V rows are copied into the pool
  slot the caller names.  Paging stores KV in fixed-size blocks allocated on
  demand anywhere in memory ("LLM上下文缓存与状态复用机制的分析和探索",
  section 3.1 PagedAttention); a slot is ``block * B + offset``.
* ``paged_attention`` -- every query row of a request attends to that
  request's KV, gathered through its block table from non-contiguous blocks,
  with a causal mask over history-plus-new positions ("Stateful Large
  Language Model Serving with Pensieve", Abstract and Methodology: the
  generalized PagedAttention computes attention between multiple new tokens
  and a cache spread over non-contiguous memory, also when part of the cache
  was dropped and its tokens are recomputed).  The attention itself is the
  textbook softmax(Q K^T * scale + mask) V.
* ``split_partial`` / ``split_merge`` -- the same attention with each
  request's KV cut into P partitions processed independently and merged
  ("PersistentKV: Page-Aware Decode Scheduling ...", section 2, the split of
  one long context into 32 chapters handled in parallel).

Pool layout (the library's contract; the same for K and V):
  K pool, V pool  [num_blocks][Hkv][B][d]   one block = B token rows of d values
Q and O are [T][Hq][d], rows packed request by request via ``cu_q_lens``.
Query head h reads KV head ``h // (Hq // Hkv)``.  A row at position p sees
keys at positions ``t <= p``.

Readings where the pages are silent are listed in the design notes of the
repository (context length counts every resident position including the new
rows; query rows default to the last q_r positions; scale 1/sqrt(d); no
positional terms in the score; contiguous GQA head groups; empty or fully
masked split partitions carry m = -inf, l = 0, O_p = 0).
"""

from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode a storage array (float32, float16, bfloat16 bit patterns in uint16, E4M3 codes in uint8)."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return e4m3_decode(a)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV storage
# ---------------------------------------------------------------------------
# The KV cache may be stored as 8-bit floats, halving its memory
# ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3): KV cache quantised to
# FP8).  The pages do not fix the format; the reading taken is the OCP 8-bit
# float E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; an
# exponent field of 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there
# are no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
# Each pool carries one float32 scale: stored code = E4M3(x / scale), value
# read back = decoded code * scale.

def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the bit fields."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Values (float64) of an array of E4M3 codes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code; beyond +-448 saturates; NaN -> 0x7F.

    The sign bit follows the sign of the input (so -0.0 and small negatives that
    round to zero give 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    grid = E4M3_VALUES[:0x7F]                     # codes 0 .. 0x7E, ascending magnitudes
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 0, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_e4m3(x: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Storage codes of values x (storage dtype ``dtype``): E4M3 of x / scale, the division in float32."""
    xf = to_f64(x, dtype).astype(np.float32)
    return e4m3_encode(xf / np.float32(scale))


# ---------------------------------------------------------------------------
# KV append
# ---------------------------------------------------------------------------
def append_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              slot_mapping: np.ndarray, block_size: int) -> None:
    """Write token t's K/V rows ([Hkv][d] each) into slot ``slot_mapping[t]``; negative slots are skipped.

    In place; the pools keep their storage dtype, so the copy is exact.
    """
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        k_pool[block, :, offset, :] = k_new[t]
        v_pool[block, :, offset, :] = v_new[t]


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def gather_kv(k_pool, v_pool, block_table_row, context_len: int, kv_head: int, block_size: int,
              dtype: str, k_scale: float = 1.0, v_scale: float = 1.0):
    """Follow a block table: return this request's K and V as contiguous [L][d] float64 arrays.

    Decoded pool values are multiplied by the pool's scale (1 for float pools).
    """
    n_blocks = -(-context_len // block_size)
    k_rows, v_rows = [], []
    for j in range(n_blocks):
        phys = int(block_table_row[j])
        k_rows.append(to_f64(k_pool[phys, kv_head], dtype))            # [B][d]
        v_rows.append(to_f64(v_pool[phys, kv_head], dtype))            # [B][d]
    d = k_pool.shape[-1]
    if n_blocks == 0:
        return np.zeros((0, d)), np.zeros((0, d))
    k = np.concatenate(k_rows, axis=0)[:context_len] * float(k_scale)
    v = np.concatenate(v_rows, axis=0)[:context_len] * float(v_scale)
    return k, v


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Query head h shares KV head h // (Hq / Hkv): contiguous groups (MHA when Hq == Hkv)."""
    return h // (num_heads // num_kv_heads)


def causal_visible(key_positions: np.ndarray, row_positions: np.ndarray) -> np.ndarray:
    """[n][L] boolean: key t is visible to the row at position p iff t <= p."""
    return np.asarray(key_positions)[None, :] <= np.asarray(row_positions)[:, None]


def causal_attention(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, positions: np.ndarray,
                     scale: float) -> np.ndarray:
    """softmax(q k^T * scale, keys t <= position of the row) v, in the operands' float type.

    q_rows [n][d], k/v [L][d], positions [n] (each < L).  Masked keys get a
    weight of exactly zero.
    """
    ct = np.result_type(q_rows, k, v, np.float32)
    n = q_rows.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=ct)
    if n == 0:
        return out
    scores = (q_rows.astype(ct, copy=False) @ k.T.astype(ct, copy=False)) * ct.type(scale)   # [n][L]
    visible = causal_visible(np.arange(k.shape[0]), positions)         # [n][L]
    masked = np.where(visible, scores, -np.inf)
    row_max = masked.max(axis=1, keepdims=True)
    weights = np.where(visible, np.exp(masked - row_max), 0.0)
    denom = weights.sum(axis=1, keepdims=True)
    return (weights @ v) / denom


def default_positions(context_len: int, q_len: int) -> np.ndarray:
    """Rows are the request's last q_len positions."""
    return np.arange(context_len - q_len, context_len, dtype=np.int64)


def row_positions(q_pos: Optional[np.ndarray], lo: int, hi: int, context_len: int) -> np.ndarray:
    """Positions of rows [lo, hi): the caller's q_pos when given, else the last hi - lo positions."""
    if q_pos is not None:
        return np.asarray(q_pos[lo:hi], dtype=np.int64)
    return default_positions(context_len, hi - lo)


def paged_attention(q: np.ndarray, k_pool, v_pool, block_tables: np.ndarray,
                    context_lens: np.ndarray, cu_q_lens: np.ndarray, q_pos: Optional[np.ndarray],
                    softmax_scale: float, dtype: str, *, requests: Optional[Iterable[int]] = None,
                    heads: Optional[Iterable[int]] = None, kv_dtype: Optional[str] = None,
                    k_scale: float = 1.0, v_scale: float = 1.0, compute=np.float64) -> np.ndarray:
    """O [T][Hq][d] float64 for the unified batch (rows of skipped requests/heads are NaN).

    ``dtype`` is the storage type of Q; the pools hold ``kv_dtype`` (default: the
    same), read back as decoded value times k_scale / v_scale.  ``compute`` is the
    float type the attention is carried out in (the decoded operands are cast to it).
    """
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    block_size = k_pool.shape[2]
    out = np.full((T, Hq, d), np.nan)
    reqs = range(len(context_lens)) if requests is None else requests
    head_list = list(range(Hq)) if heads is None else list(heads)
    for r in reqs:
        lo, hi = int(cu_q_lens[r]), int(cu_q_lens[r + 1])
        L = int(context_lens[r])
        pos = row_positions(q_pos, lo, hi, L)
        for h in head_list:
            g = kv_head_of(h, Hq, Hkv)
            k, v = gather_kv(k_pool, v_pool, block_tables[r], L, g, block_size, kv_dtype, k_scale, v_scale)
            qr = to_f64(q[lo:hi, h, :], dtype)
            out[lo:hi, h, :] = causal_attention(qr.astype(compute, copy=False), k.astype(compute, copy=False),
                                                v.astype(compute, copy=False), pos, softmax_scale)
    return out


# ---------------------------------------------------------------------------
# Split-KV partial / merge
# ---------------------------------------------------------------------------
def partition_token_ranges(context_len: int, num_partitions: int, block_size: int):
    """Partition k covers logical blocks [k*S, (k+1)*S), S = ceil(ceil(L/B)/P), clipped to [0, L)."""
    n_blocks = -(-context_len // block_size)
    per = -(-n_blocks // num_partitions) if n_blocks else 0
    ranges = []
    for k in range(num_partitions):
        start = min(k * per * block_size, context_len)
        end = min((k + 1) * per * block_size, context_len)
        ranges.append((start, end))
    return ranges


def partial_attention(q_rows, k, v, positions, scale, start: int, end: int):
    """Attention restricted to keys [start, end): returns (O_p normalised, m, l) per row.

    m is the largest visible scaled score, l the sum of exp(score - m) over
    visible keys; a row with no visible key in the range gets m = -inf,
    l = 0, O_p = 0.
    """
    ct = np.result_type(q_rows, k, v, np.float32)
    n, dv = q_rows.shape[0], v.shape[1]
    o = np.zeros((n, dv), ct); m = np.full(n, -np.inf, ct); l = np.zeros(n, ct)
    if n == 0 or end <= start:
        return o, m, l
    scores = (q_rows.astype(ct, copy=False) @ k[start:end].T.astype(ct, copy=False)) * ct.type(scale)
    visible = causal_visible(np.arange(start, end), positions)
    any_vis = visible.any(axis=1)
    masked = np.where(visible, scores, -np.inf)
    m_rows = np.where(any_vis, masked.max(axis=1), -np.inf)
    safe_m = np.where(any_vis, m_rows, 0.0)
    weights = np.where(visible, np.exp(masked - safe_m[:, None]), 0.0)
    l_rows = weights.sum(axis=1)
    num = weights @ v[start:end]
    o = np.where(any_vis[:, None], num / np.where(l_rows > 0, l_rows, 1.0)[:, None], 0.0)
    return o, m_rows, l_rows


def split_partial(q: np.ndarray, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos,
                  softmax_scale: float, dtype: str, num_partitions: int, *,
                  requests: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None,
                  kv_dtype: Optional[str] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                  compute=np.float64):
    """Partials part_o [T][Hq][P][d], part_m [T][Hq][P], part_l [T][Hq][P] (float64 arrays; the
    attention is carried out in ``compute``)."""
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    block_size = k_pool.shape[2]
    P = num_partitions
    part_o = np.full((T, Hq, P, d), np.nan)
    part_m = np.full((T, Hq, P), np.nan)
    part_l = np.full((T, Hq, P), np.nan)
    reqs = range(len(context_lens)) if requests is None else requests
    head_list = list(range(Hq)) if heads is None else list(heads)
    for r in reqs:
        lo, hi = int(cu_q_lens[r]), int(cu_q_lens[r + 1])
        L = int(context_lens[r])
        pos = row_positions(q_pos, lo, hi, L)
        ranges = partition_token_ranges(L, P, block_size)
        for h in head_list:
            g = kv_head_of(h, Hq, Hkv)
            k, v = gather_kv(k_pool, v_pool, block_tables[r], L, g, block_size, kv_dtype, k_scale, v_scale)
            k, v = k.astype(compute, copy=False), v.astype(compute, copy=False)
            qr = to_f64(q[lo:hi, h, :], dtype).astype(compute, copy=False)
            for p_idx, (s, e) in enumerate(ranges):
                o, m, l = partial_attention(qr, k, v, pos, softmax_scale, s, e)
                part_o[lo:hi, h, p_idx, :] = o
                part_m[lo:hi, h, p_idx] = m
                part_l[lo:hi, h, p_idx] = l
    return part_o, part_m, part_l


def split_merge(part_o: np.ndarray, part_m: np.ndarray, part_l: np.ndarray, compute=np.float64) -> np.ndarray:
    """O = sum_k w_k O_k / sum_k w_k with w_k = l_k exp(m_k - max_k m_k); empty partitions weigh 0."""
    m = np.asarray(part_m, dtype=compute)
    l = np.asarray(part_l, dtype=compute)
    part_o = np.asarray(part_o, dtype=compute)
    live = l > 0
    m_star = np.where(live, m, -np.inf).max(axis=-1, keepdims=True)
    w = np.where(live, l * np.exp(np.where(live, m, 0.0) - np.where(np.isfinite(m_star), m_star, 0.0)), 0.0)
    num = (w[..., None] * np.where(live[..., None], part_o, 0.0)).sum(axis=-2)
    den = w.sum(axis=-1)[..., None]
    return num / den


__all__ = [
    "to_f64", "e4m3_value", "e4m3_decode", "e4m3_encode", "quantize_e4m3", "E4M3_VALUES", "E4M3_MAX", "append_kv", "gather_kv", "kv_head_of", "causal_visible", "causal_attention",
    "default_positions", "row_positions", "paged_attention",
    "partition_token_ranges", "partial_attention", "split_partial", "split_merge",
]
