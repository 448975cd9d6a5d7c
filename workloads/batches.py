"""Seeded batch generator for the unified prefill/decode/recompute attention batch.

Workload shapes follow the multi-turn serving setting of "Stateful Large
Language Model Serving with Pensieve" (Methodology; Key Results: OPT-13B,
Llama 2-13B, Llama 2-70B): every request brings new query tokens that attend
to the cached conversation history, decode requests bring one token, and a
conversation whose leading cache blocks were dropped recomputes those tokens
as extra query rows ahead of its new tokens.  Long single requests follow the
32-way split scenario of "PersistentKV: Page-Aware Decode Scheduling for
Long-Context LLM Serving on Commodity GPUs" (section 2, the split strategy).

Conventions (fixed here, used by both the oracle and the GPU path):

* Position ``t`` of request ``r`` lives in logical block ``t // B`` at offset
  ``t % B``; ``block_tables[r][t // B]`` names the physical block; the slot of
  the token is ``physical * B + t % B``.
* Request ``r`` has ``H_r`` history positions, drops the leading ``E_r`` of
  them (a multiple of ``B``), and brings ``n_r`` new tokens.  After the
  append, its KV covers positions ``[0, L_r)`` with ``L_r = H_r + n_r``.  Its
  query rows are positions ``[0, E_r)`` followed by ``[H_r, H_r + n_r)``, so
  ``q_r = E_r + n_r``.  Rows are packed request by request (``cu_q_lens``).
* Values: rows of each tensor (Q rows, K/V positions) are drawn in chunks
  of 1024 rows; chunk c of tensor tag of request r comes from its own NumPy
  ``default_rng`` stream keyed ``(seed, tag, r, c)``: float32 standard
  normals, multiplied by 0.5, rounded to nearest-even into the storage dtype.
  K and V are drawn for all ``L_r`` positions in position order, so any
  single request (or chunk) can be regenerated alone, and chunks can be
  drawn in parallel threads.
* Storage dtypes: ``f32`` -> ``np.float32``, ``f16`` -> ``np.float16``,
  ``bf16`` -> ``np.uint16`` holding the bfloat16 bit pattern.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Iterator, Optional

import numpy as np

CONFIG_NAMES = (
    "tiny_f32_mha4x64",
    "llama2_13b_mixed_f16",
    "opt13b_decode_heavy_f16",
    "llama2_70b_gqa_recompute_bf16",
    "long_context_split_bf16",
)

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
BASE_SEED = 20231209
_TAG_Q, _TAG_K, _TAG_V = 1, 2, 3
ROW_CHUNK = 1024
_WORKERS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
_pool: Optional[ThreadPoolExecutor] = None


def _thread_pool() -> ThreadPoolExecutor:
    global _pool
    if _pool is None:
        _pool = ThreadPoolExecutor(max_workers=_WORKERS, thread_name_prefix="workloads")
    return _pool


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    return bf16_bits_from_f32(x)


@dataclass
class Batch:
    """One unified attention batch plus the recipe for its values."""

    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seed: int
    hist_lens: np.ndarray
    new_lens: np.ndarray
    evict_lens: np.ndarray
    block_tables: np.ndarray  # int32 [R][stride]
    value_scale: float = 0.5
    # Optional per-request value overrides used by structured tests:
    # fn(r) -> float32 array of the request's shape (rounded to storage here).
    q_fn: Optional[Callable[[int], np.ndarray]] = field(default=None, repr=False)
    k_fn: Optional[Callable[[int], np.ndarray]] = field(default=None, repr=False)
    v_fn: Optional[Callable[[int], np.ndarray]] = field(default=None, repr=False)
    # Optional explicit query positions per request (sorted, distinct, each below the request's
    # context length); they replace the recompute/new-row convention above: the request's rows
    # sit at these positions and every other position of [0, L_r) is cached history.
    positions: Optional[list] = field(default=None, repr=False)

    # ---- shapes -----------------------------------------------------------
    @property
    def num_reqs(self) -> int:
        return int(len(self.hist_lens))

    @property
    def context_lens(self) -> np.ndarray:
        return (self.hist_lens + self.new_lens).astype(np.int32)

    @property
    def q_lens(self) -> np.ndarray:
        if self.positions is not None:
            return np.array([len(p) for p in self.positions], dtype=np.int32)
        return (self.evict_lens + self.new_lens).astype(np.int32)

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_reqs + 1, dtype=np.int32)
        np.cumsum(self.q_lens, out=cu[1:])
        return cu

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def block_table_stride(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    def query_positions(self, r: int) -> np.ndarray:
        if self.positions is not None:
            return np.asarray(self.positions[r], dtype=np.int64)
        e, h, n = int(self.evict_lens[r]), int(self.hist_lens[r]), int(self.new_lens[r])
        return np.concatenate([np.arange(0, e), np.arange(h, h + n)]).astype(np.int64)

    def cached_positions(self, r: int) -> np.ndarray:
        if self.positions is not None:
            return np.setdiff1d(np.arange(int(self.context_lens[r]), dtype=np.int64), self.query_positions(r))
        return np.arange(int(self.evict_lens[r]), int(self.hist_lens[r]), dtype=np.int64)

    @property
    def q_pos(self) -> np.ndarray:
        if self.total_q == 0:
            return np.zeros(0, dtype=np.int32)
        return np.concatenate([self.query_positions(r) for r in range(self.num_reqs)]).astype(np.int32)

    @property
    def has_default_positions(self) -> bool:
        """True when every request's rows are its last q_r positions."""
        if self.positions is not None:
            return all(np.array_equal(self.query_positions(r),
                                      np.arange(int(self.context_lens[r]) - int(self.q_lens[r]),
                                                int(self.context_lens[r])))
                       for r in range(self.num_reqs))
        return bool(np.all(self.evict_lens == 0))

    def slots_for(self, r: int, positions: np.ndarray) -> np.ndarray:
        b = self.block_size
        phys = self.block_tables[r][positions // b].astype(np.int64)
        return (phys * b + positions % b).astype(np.int32)

    @property
    def new_slots(self) -> np.ndarray:
        """Slot of every query row's own K/V (the rows appended this step)."""
        if self.total_q == 0:
            return np.zeros(0, dtype=np.int32)
        return np.concatenate(
            [self.slots_for(r, self.query_positions(r)) for r in range(self.num_reqs)]
        ).astype(np.int32)

    def used_blocks(self) -> np.ndarray:
        used = [self.block_tables[r][: self.num_logical_blocks(r)] for r in range(self.num_reqs)]
        return np.unique(np.concatenate(used)) if used else np.zeros(0, dtype=np.int32)

    def num_logical_blocks(self, r: int) -> int:
        return -(-int(self.context_lens[r]) // self.block_size)

    # ---- values -----------------------------------------------------------
    def _draw_chunk(self, tag: int, r: int, c: int, rows: int, width) -> np.ndarray:
        rng = np.random.default_rng([self.seed, tag, r, c])
        x = rng.standard_normal((rows, *width), dtype=np.float32)
        x *= np.float32(self.value_scale)
        return _to_storage(x, self.dtype)

    def _draw_rows(self, tag: int, r: int, nrows: int, width, parallel: bool) -> np.ndarray:
        out = np.empty((nrows, *width), dtype=storage_dtype(self.dtype))
        nch = -(-nrows // ROW_CHUNK)

        def work(c):
            lo, hi = c * ROW_CHUNK, min(nrows, (c + 1) * ROW_CHUNK)
            out[lo:hi] = self._draw_chunk(tag, r, c, hi - lo, width)

        if parallel and nch > 1:
            list(_thread_pool().map(work, range(nch)))
        else:
            for c in range(nch):
                work(c)
        return out

    def request_q(self, r: int, parallel: bool = True) -> np.ndarray:
        shape = (int(self.q_lens[r]), self.num_heads, self.head_dim)
        if self.q_fn is not None:
            return _to_storage(np.asarray(self.q_fn(r), dtype=np.float32).reshape(shape), self.dtype)
        return self._draw_rows(_TAG_Q, r, shape[0], shape[1:], parallel)

    def request_kv(self, r: int, parallel: bool = True):
        """K and V of every position of request r, [L_r][Hkv][d] each, position order."""
        shape = (int(self.context_lens[r]), self.num_kv_heads, self.head_dim)
        if self.k_fn is not None:
            k = _to_storage(np.asarray(self.k_fn(r), dtype=np.float32).reshape(shape), self.dtype)
        else:
            k = self._draw_rows(_TAG_K, r, shape[0], shape[1:], parallel)
        if self.v_fn is not None:
            v = _to_storage(np.asarray(self.v_fn(r), dtype=np.float32).reshape(shape), self.dtype)
        else:
            v = self._draw_rows(_TAG_V, r, shape[0], shape[1:], parallel)
        return k, v

    def q_all(self) -> np.ndarray:
        sd = storage_dtype(self.dtype)
        if self.total_q == 0:
            return np.zeros((0, self.num_heads, self.head_dim), dtype=sd)
        parts = list(_thread_pool().map(lambda r: self.request_q(r, parallel=False), range(self.num_reqs)))
        return np.concatenate(parts, axis=0)

    def new_kv(self):
        """K/V of the query rows' own positions, [T][Hkv][d], row order."""
        ks, vs = [], []
        for r, k, v, _, _ in self.iter_requests():
            pos = self.query_positions(r)
            ks.append(k[pos])
            vs.append(v[pos])
        sd = storage_dtype(self.dtype)
        empty = np.zeros((0, self.num_kv_heads, self.head_dim), dtype=sd)
        return (np.concatenate(ks, axis=0) if ks else empty, np.concatenate(vs, axis=0) if vs else empty)

    def iter_requests(self, window: Optional[int] = None) -> Iterator[tuple]:
        """Per request: (r, K all positions, V all positions, cached slots, cached positions).

        Requests are drawn ahead in worker threads (at most ``window`` at a
        time) and yielded in order.
        """
        window = window or 2 * _WORKERS

        def one(r):
            k, v = self.request_kv(r, parallel=False)
            pos = self.cached_positions(r)
            return r, k, v, self.slots_for(r, pos), pos

        pending = []
        nxt = 0
        pool = _thread_pool()
        while nxt < self.num_reqs or pending:
            while nxt < self.num_reqs and len(pending) < window:
                pending.append(pool.submit(one, nxt))
                nxt += 1
            yield pending.pop(0).result()


def _place_blocks(rng, need: np.ndarray, num_blocks: int, stride: int) -> np.ndarray:
    """Assign distinct physical blocks request by request from one permutation of the pool."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    total = int(need.sum())
    assert total <= num_blocks, (total, num_blocks)
    bt = np.zeros((len(need), max(stride, 1)), dtype=np.int32)
    off = 0
    for r, nb in enumerate(need):
        bt[r, :nb] = perm[off:off + nb]
        off += nb
    return bt


def custom_batch(
    hist_lens,
    new_lens,
    evict_lens=None,
    *,
    num_heads: int = 4,
    num_kv_heads: int = 4,
    head_dim: int = 64,
    dtype: str = "f32",
    seed: int = 1234,
    block_size: int = 16,
    pool_factor: float = 1.25,
    num_blocks: Optional[int] = None,
    extra_stride: int = 0,
    name: str = "custom",
) -> Batch:
    """Batch with explicit lengths; blocks drawn from one permutation of a pool."""
    hist = np.asarray(hist_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    ev = np.zeros_like(hist) if evict_lens is None else np.asarray(evict_lens, dtype=np.int64)
    assert hist.shape == new.shape == ev.shape
    assert np.all(ev % block_size == 0) and np.all(ev <= hist)
    rng = np.random.default_rng(seed)
    ctx = hist + new
    need = -(-ctx // block_size)
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * int(need.sum()))), 1)
    stride = int(need.max()) + extra_stride if len(need) else 1
    bt = _place_blocks(rng, need, num_blocks, stride)
    return Batch(name, dtype, num_heads, num_kv_heads, head_dim, block_size, int(num_blocks), seed,
                 hist, new, ev, bt)


def config_batch(index: int, *, num_reqs: Optional[int] = None, num_heads: Optional[int] = None,
                 max_hist: Optional[int] = None) -> Batch:
    """The five seeded workloads (0..4), optionally cut down for quick parity runs.

    ``num_reqs`` keeps the first requests of each group, ``num_heads`` keeps the
    first query heads (and the matching share of KV heads) and ``max_hist``
    caps history lengths; the draws themselves are unchanged, so a cut-down
    batch is a sub-problem of the full one up to placement.
    """
    seed = BASE_SEED + index
    rng = np.random.default_rng(seed)
    B = 16
    if index == 0:
        hist = np.array([37, 80, 0]); new = np.array([5, 1, 12]); ev = np.zeros(3, np.int64)
        hq = hkv = 4; d = 64; dt = "f32"
    elif index == 1:
        h_conv = rng.integers(256, 2048, size=32, endpoint=True)
        n_conv = rng.integers(16, 128, size=32, endpoint=True)
        h_dec = rng.integers(256, 2048, size=32, endpoint=True)
        hist = np.concatenate([h_conv, h_dec]); new = np.concatenate([n_conv, np.ones(32, np.int64)])
        ev = np.zeros(64, np.int64); hq = hkv = 40; d = 128; dt = "f16"
        if num_reqs is not None:
            keep = np.r_[0:min(num_reqs, 32), 32:32 + min(num_reqs, 32)]
            hist, new, ev = hist[keep], new[keep], ev[keep]
    elif index == 2:
        h = np.rint(rng.lognormal(mean=math.log(1024.0), sigma=1.0, size=256))
        hist = np.clip(h, 64, 4096).astype(np.int64); new = np.ones(256, np.int64)
        ev = np.zeros(256, np.int64); hq = hkv = 40; d = 128; dt = "f16"
    elif index == 3:
        hist = rng.integers(512, 8192, size=48, endpoint=True)
        dropped = np.array([rng.integers(0, (h // B) // 2, endpoint=True) for h in hist], dtype=np.int64)
        ev = dropped * B
        new = rng.integers(1, 256, size=48, endpoint=True)
        hq, hkv, d, dt = 16, 2, 128, "bf16"
    elif index == 4:
        hist = np.array([32768, 40960, 49152, 65536]); new = np.array([1, 1, 512, 1])
        ev = np.zeros(4, np.int64); hq = hkv = 40; d = 128; dt = "bf16"
    else:
        raise ValueError(index)
    hist = hist.astype(np.int64); new = new.astype(np.int64); ev = ev.astype(np.int64)
    if num_reqs is not None and index != 1:
        hist, new, ev = hist[:num_reqs], new[:num_reqs], ev[:num_reqs]
    if max_hist is not None:
        capped = np.minimum(hist, max_hist)
        ev = np.minimum(ev, (capped // (2 * B)) * B)
        hist = capped
    if num_heads is not None:
        group = hq // hkv
        hq = min(num_heads, hq)
        hkv = max(1, hq // group)
        hq = hkv * group
    ctx = hist + new
    need = -(-ctx // B)
    num_blocks = 32 if index == 0 else int(math.ceil(1.25 * int(need.sum())))
    bt = _place_blocks(rng, need, num_blocks, int(need.max()))
    return Batch(CONFIG_NAMES[index], dt, hq, hkv, d, B, num_blocks, seed, hist, new, ev, bt)


def draw_rows(key, shape, dtype: str, scale: float = 0.5) -> np.ndarray:
    """Standard normals times ``scale`` of the given shape, from ``default_rng(key)``, in storage dtype."""
    rng = np.random.default_rng(list(key))
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    x *= np.float32(scale)
    return _to_storage(x, dtype)


def conversation_script(seed: int, num_convs: int, steps: int, *, prompt=(16, 96), answer=(2, 6),
                        idle=(0, 4)) -> np.ndarray:
    """new_tokens[step][conversation] of a multi-turn serving run.

    Each conversation alternates idle spells and turns.  A turn is one step
    that brings the user's prompt (``prompt`` tokens, inclusive range) followed
    by decode steps of one token each (``answer`` of them); between turns the
    conversation is idle for ``idle`` steps, so its cache sits unused and may
    be dropped.  Draws come from ``default_rng((seed, conversation))``.
    """
    out = np.zeros((steps, num_convs), dtype=np.int32)
    for c in range(num_convs):
        rng = np.random.default_rng([seed, c])
        t = int(rng.integers(idle[0], idle[1], endpoint=True))
        while t < steps:
            out[t, c] = int(rng.integers(prompt[0], prompt[1], endpoint=True))
            t += 1
            for _ in range(int(rng.integers(answer[0], answer[1], endpoint=True))):
                if t >= steps:
                    break
                out[t, c] = 1
                t += 1
            t += int(rng.integers(idle[0], idle[1], endpoint=True))
    return out
