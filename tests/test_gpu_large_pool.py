"""Pools larger than 4 GiB on the GPU.

Every byte offset of a block past 2^32 must be formed in 64 bits by the append, both attention
kernels, the split pair and the swap.  1 200 000 blocks of f16 K (and V) for 2 KV heads at
head_dim 128 make each pool 9.8 GB; the batch's blocks are drawn from the whole pool, so more
than half of them lie past the first 4 GiB ("Stateful Large Language Model Serving with Pensieve",
Methodology: a request's cache is scattered over a large shared pool).  Each (request, query
head) is checked against the oracle's attention over the request's own K/V rows, which needs no
pool on the host.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, run_split, to_f64, to_host_storage, upload
from oracle_helpers import request_rows_reference
from workloads import custom_batch

pytestmark = pytest.mark.gpu

NUM_BLOCKS = 1_200_000
TOL = 1e-2


def _say(msg):
    print(f"[large_pool] {msg}", flush=True)


def _batch():
    return custom_batch([3000, 700, 0, 1500], [40, 1, 20, 130], num_heads=4, num_kv_heads=2, head_dim=128,
                        dtype="f16", seed=81, num_blocks=NUM_BLOCKS, name="large_pool_f16")


def _used_blocks(b):
    out = []
    for r in range(b.num_reqs):
        out += b.block_tables[r, :-(-int(b.context_lens[r]) // 16)].tolist()
    return out


def _check(b, got, what):
    assert np.all(np.isfinite(got)), what
    worst = 0.0
    for r in range(b.num_reqs):
        lo, hi = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
        for h in range(b.num_heads):
            ref = request_rows_reference(b, r, h)
            worst = max(worst, float(np.max(np.abs(got[lo:hi, h, :] - ref))) if hi > lo else 0.0)
    _say(f"  {what}: max abs err {worst:.3e}")
    assert worst <= TOL, what


def test_pools_beyond_4_gib():
    import torch
    b = _batch()
    block_bytes = b.num_kv_heads * 16 * b.head_dim * 2
    used = _used_blocks(b)
    far = sum(1 for x in used if x * block_bytes >= 2 ** 32)
    _say(f"pool {NUM_BLOCKS * block_bytes / 2**30:.2f} GiB per tensor; {far} of {len(used)} blocks past 4 GiB")
    assert NUM_BLOCKS * block_bytes > 2 ** 32 and far > len(used) // 2
    gb = upload(b)
    # The 130-row request (260 query vectors per KV head) puts this small call on eight-wave
    # matrix-core items, so their offsets past 4 GiB are checked too.
    plan = pk.pensieve_debug_plan(gb.make_desc(0))
    live = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
    assert int((live[:, 4] * (b.num_heads // b.num_kv_heads)).max()) == 256
    _check(b, to_f64(run_attn(gb, 0)), "default plan")
    _check(b, to_f64(run_attn(gb, pk.PENSIEVE_FLAG_VECTOR_ONLY)), "vector kernel")
    _check(b, to_f64(run_split(gb, 4)[3]), "split pair, 4 partitions")
    # Swap round trip of the eight highest blocks: out to the host tier, poisoned on the device,
    # back in; attention is bitwise unchanged.
    before = to_host_storage(run_attn(gb, 0), b.dtype)
    hi_blocks = sorted(used)[-8:]
    k_host = torch.empty((8,) + tuple(gb.k_pool.shape[1:]), dtype=gb.k_pool.dtype).pin_memory()
    v_host = torch.empty((8,) + tuple(gb.v_pool.shape[1:]), dtype=gb.v_pool.dtype).pin_memory()
    pk.pensieve_kv_swap_out(gb.k_pool, gb.v_pool, k_host, v_host, hi_blocks, list(range(8)))
    torch.cuda.synchronize()
    idx = torch.tensor(hi_blocks, dtype=torch.long, device="cuda")
    gb.k_pool[idx] = float("nan")
    gb.v_pool[idx] = float("nan")
    pk.pensieve_kv_swap_in(gb.k_pool, gb.v_pool, k_host, v_host, list(range(8)), hi_blocks)
    torch.cuda.synchronize()
    after = to_host_storage(run_attn(gb, 0), b.dtype)
    assert np.array_equal(before, after)
    _say("  swap round trip of the 8 highest blocks: bitwise equal")
