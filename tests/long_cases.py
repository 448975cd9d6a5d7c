"""Structured inputs at the real lengths of the long-context split workload.

"PersistentKV: Page-Aware Decode Scheduling for Long-Context LLM Serving on Commodity GPUs",
section 2 cuts one long context into 32 partitions; the long-context workload has histories of
32768, 40960, 49152 and 65536 tokens with 1, 1, 512 and 1 new rows.  At those lengths the flat
N(0,1)*0.5 values give |O| of about 0.003, below what a 1e-2 gate can see, so these cases use
values whose outputs are fixed in closed form and move far beyond their tolerance when a single
block is read from the wrong place or the causal boundary slips:

* signature_batch -- zero queries (every visible key weighs exactly 1, so O is the mean of the
  visible V rows).  The last dim of V alternates +-A over positions (any one-key slip of the
  causal boundary flips the output between A/(p+1) and 0); every other dim is 0 except at the
  first key of each block, which carries +-A in one dim that depends on the block, its KV head
  and its request, with signs alternating among the blocks sharing a dim, so every partial sum over
  blocks stays in {0, +-A}: dropping, adding or swapping one block moves some output dim by
  A/(p+1) while |O| stays at most A/(p+1).
* onehot_batch -- rows spread over the whole context (one per 64-key tile, in explicit
  positions), random +-1 keys and values, and Q = 4 K at the row's own position: each row's
  own key out-scores every other by about 25 nats, so O is V at the row's own position to well
  inside the gate, and a wrong block gives another V row (some dim off by 2).

Both are used by the GPU parity tests and by the CPU pins that derive the margins.
"""

from __future__ import annotations

import numpy as np

from workloads import custom_batch

LONG_HIST = (32768, 40960, 49152, 65536)
LONG_NEW = (1, 1, 512, 1)
# The largest contexts the structured tests reach: a decode row on 262 144 keys (4 096 tiles of 64)
# beside a 64-row prefill on 131 072 history tokens.
MAX_HIST = (262143, 131072)
MAX_NEW = (1, 64)
A = 256.0


def signature_v(L: int, hkv: int, d: int, r: int) -> np.ndarray:
    """V rows [L][hkv][d] of request r in the signature pattern (float32, exact in f16 and bf16).

    Block b of KV head g puts its mark in dim (b + 31 g + 17 r) mod (d - 1), so the same block
    index of another head or request marks another dim; the blocks sharing a dim within one
    request come d - 1 blocks apart and alternate in sign."""
    t = np.arange(L)
    b = t // 16
    v = np.zeros((L, hkv, d), np.float32)
    v[:, :, d - 1] = (A * (-1.0) ** (t % 2))[:, None]
    first = np.nonzero(t % 16 == 0)[0]
    fb = b[first]
    sign = np.where((fb // (d - 1) + r) % 2 == 0, A, -A).astype(np.float32)
    for g in range(hkv):
        dim = (fb + 31 * g + 17 * r) % (d - 1)
        v[first, g, dim] = sign
    return v


def signature_batch(dtype: str, group: int, hkv: int = 2, d: int = 128, seed: int = 301, hist=LONG_HIST,
                    new=LONG_NEW):
    """Zero queries, signature V, random K; the long-context workload's lengths and rows unless
    hist / new give others."""
    b = custom_batch(list(hist), list(new), num_heads=hkv * group, num_kv_heads=hkv, head_dim=d,
                     dtype=dtype, seed=seed, name=f"long_signature_{dtype}_g{group}")
    b.q_fn = lambda r: np.zeros((int(b.q_lens[r]), b.num_heads, d), np.float32)
    b.v_fn = lambda r: signature_v(int(b.context_lens[r]), hkv, d, r)
    return b


def signature_expected(b) -> np.ndarray:
    """O [T][Hq][d] of a zero-query batch: the float64 mean of the stored V over keys 0..p."""
    out = np.zeros((b.total_q, b.num_heads, b.head_dim))
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        v = signature_v(int(b.context_lens[r]), b.num_kv_heads, b.head_dim, r).astype(np.float64)
        cs = np.cumsum(v, axis=0)
        pos = b.query_positions(r)
        lo = int(b.cu_q_lens[r])
        for h in range(b.num_heads):
            out[lo:lo + len(pos), h, :] = cs[pos, h // G, :] / (pos + 1)[:, None]
    return out


def spread_positions(L: int, seed: int) -> np.ndarray:
    """One row per 64-key tile of [0, L), at offsets that cycle through the tile's four blocks."""
    ntiles = -(-L // 64)
    j = np.arange(ntiles)
    off = (j * 17 + seed) % 64
    pos = np.minimum(64 * j + off, L - 1)
    return np.unique(pos)


def onehot_batch(dtype: str, group: int, hkv: int = 2, d: int = 128, seed: int = 302):
    """Rows in every tile of the long contexts; Q = 4 K[own position]; K, V random +-1."""
    ctx = [h + n for h, n in zip(LONG_HIST, LONG_NEW)]
    positions = [spread_positions(L, r) for r, L in enumerate(ctx)]
    q = [len(p) for p in positions]
    b = custom_batch([L - n for L, n in zip(ctx, q)], q, num_heads=hkv * group, num_kv_heads=hkv, head_dim=d,
                     dtype=dtype, seed=seed, name=f"long_onehot_{dtype}_g{group}")
    b.positions = positions
    rng = np.random.default_rng(seed)
    ks = {r: rng.choice([-1.0, 1.0], size=(L, hkv, d)).astype(np.float32) for r, L in enumerate(ctx)}
    vs = {r: rng.choice([-1.0, 1.0], size=(L, hkv, d)).astype(np.float32) for r, L in enumerate(ctx)}
    b.k_fn = lambda r: ks[r]
    b.v_fn = lambda r: vs[r]
    b.q_fn = lambda r: 4.0 * np.repeat(ks[r][b.query_positions(r)], group, axis=1)
    b._onehot_v = vs
    return b


def onehot_expected(b) -> np.ndarray:
    """O [T][Hq][d] ~= V at each row's own position."""
    out = np.zeros((b.total_q, b.num_heads, b.head_dim))
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        pos = b.query_positions(r)
        lo = int(b.cu_q_lens[r])
        for h in range(b.num_heads):
            out[lo:lo + len(pos), h, :] = b._onehot_v[r][pos, h // G, :]
    return out


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output type at |x| (0 at x = 0); normal range only (enough here)."""
    mant = {"bf16": 7, "f16": 10, "f32": 23}[dtype]
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - mant), 0.0)


def signature_tol(expected: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element gate of the signature test: 4 output ulps at |O| plus 2^-20 (the sums are exact)."""
    return 4.0 * ulp(expected, dtype) + 2.0 ** -20


ONEHOT_TOL = 1e-2
