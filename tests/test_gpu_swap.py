"""GPU block swap with a pinned host tier.

Round trip: every block a batch uses goes out to scattered host blocks, the device pools are
poisoned with NaN, the blocks come back into different device blocks and the block tables are
rewritten.  Attention over the moved cache must be bitwise identical to the original (physical
placement does not enter the arithmetic), and the tier contents must equal the device blocks bit
for bit.  A swap-in on a second stream runs beside an attention launch without disturbing it.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, to_f64, to_host_storage, upload
from oracle_helpers import oracle_output, oracle_pools
from workloads import config_batch, custom_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[swap] {msg}", flush=True)


def _host_tier(gb, blocks):
    import torch
    kp, vp = gb.k_pool, gb.v_pool
    k_host = torch.empty((blocks,) + tuple(kp.shape[1:]), dtype=kp.dtype).pin_memory()
    v_host = torch.empty((blocks,) + tuple(vp.shape[1:]), dtype=vp.dtype).pin_memory()
    return k_host, v_host


def _bits(t):
    import torch
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


CASES = {
    "mixed_f16": lambda: config_batch(1, num_reqs=6, num_heads=8),
    "gqa_recompute_bf16": lambda: config_batch(3, num_reqs=3, max_hist=900),
    "tiny_f32": lambda: config_batch(0),
    "d64_gqa_f16": lambda: custom_batch([300, 45, 0], [20, 1, 33], num_heads=8, num_kv_heads=2, head_dim=64,
                                        dtype="f16", seed=71),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_round_trip_leaves_attention_bitwise_unchanged(name):
    import torch
    b = CASES[name]()
    gb = upload(b)
    before = run_attn(gb).clone()
    used = b.used_blocks()
    rng = np.random.default_rng(7)
    k_host, v_host = _host_tier(gb, len(used) + 5)
    host_ids = rng.permutation(len(used) + 5)[:len(used)].astype(np.int32)
    _say(f"{name}: {len(used)} blocks out to the host tier")
    pk.pensieve_kv_swap_out(gb.k_pool, gb.v_pool, k_host, v_host, used, host_ids)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k_host[torch.from_numpy(host_ids).long()]),
                          _bits(gb.k_pool[torch.from_numpy(used).cuda().long()]))
    assert np.array_equal(_bits(v_host[torch.from_numpy(host_ids).long()]),
                          _bits(gb.v_pool[torch.from_numpy(used).cuda().long()]))
    gb.k_pool.fill_(float("nan"))
    gb.v_pool.fill_(float("nan"))
    new_ids = rng.permutation(b.num_blocks)[:len(used)].astype(np.int32)
    pk.pensieve_kv_swap_in(gb.k_pool, gb.v_pool, k_host, v_host, host_ids, new_ids)
    remap = np.full(b.num_blocks, -1, np.int64)
    remap[used] = new_ids
    bt = b.block_tables.copy()
    for r in range(b.num_reqs):
        nl = b.num_logical_blocks(r)
        bt[r, :nl] = remap[bt[r, :nl]]
    gb.block_tables = torch.from_numpy(bt).cuda()
    torch.cuda.synchronize()
    after = run_attn(gb)
    assert np.array_equal(_bits(before), _bits(after)), "attention changed after the round trip"
    # Against the oracle: the moved blocks hold exactly what the oracle's append put in the original
    # ones (NaN poison in stale slots included), and attention over them meets the gate.
    ok_pool, ov_pool = oracle_pools(b)
    idx = torch.from_numpy(new_ids).cuda().long()
    for got, want in ((gb.k_pool[idx], ok_pool[used]), (gb.v_pool[idx], ov_pool[used])):
        got = to_host_storage(got, b.dtype)
        assert got.shape == want.shape
        assert np.array_equal(got, want, equal_nan=b.dtype != "bf16"), "moved blocks differ from the oracle's"
    tol = 1e-4 if b.dtype == "f32" else 1e-2
    err = float(np.max(np.abs(to_f64(after) - oracle_output(b))))
    _say(f"{name}: blocks bit-exact vs oracle pools, attention max abs err {err:.2e}")
    assert err <= tol


def test_swap_in_on_a_second_stream_beside_attention():
    """Blocks the batch does not use are swapped in on a side stream while attention runs."""
    import torch
    b = config_batch(1, num_reqs=6, num_heads=8)
    gb = upload(b)
    ref = run_attn(gb).clone()
    free = np.setdiff1d(np.arange(b.num_blocks), b.used_blocks()).astype(np.int32)
    n = min(len(free), 64)
    k_host, v_host = _host_tier(gb, n)
    k_host.copy_(torch.randn(k_host.shape, dtype=torch.float32).to(k_host.dtype))
    v_host.copy_(torch.randn(v_host.shape, dtype=torch.float32).to(v_host.dtype))
    side = torch.cuda.Stream()
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(gb.desc), 256), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(gb.q)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        pk.pensieve_kv_swap_in(gb.k_pool, gb.v_pool, k_host, v_host, np.arange(n, dtype=np.int32), free[:n],
                               stream=side)
    pk.pensieve_attn_fwd(gb.desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens, gb.cu_q_lens,
                         gb.q_pos, o, ws)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o), _bits(ref))
    idx = torch.from_numpy(free[:n]).cuda().long()
    assert np.array_equal(_bits(gb.k_pool[idx]), _bits(k_host))
    assert np.array_equal(_bits(gb.v_pool[idx]), _bits(v_host))


def test_swap_rejects_unpinned_host_memory():
    import torch
    b = config_batch(0)
    gb = upload(b)
    k_host = torch.empty((4,) + tuple(gb.k_pool.shape[1:]), dtype=gb.k_pool.dtype)
    v_host = torch.empty((4,) + tuple(gb.v_pool.shape[1:]), dtype=gb.v_pool.dtype)
    with pytest.raises(pk.PensieveError) as ei:
        pk.pensieve_kv_swap_out(gb.k_pool, gb.v_pool, k_host, v_host, [0], [1])
    assert ei.value.status == 1
    from paged_kv_token_amd import binding
    lib = pk.load_library()
    import ctypes
    ids = (ctypes.c_int32 * 1)(0)
    st = lib.pensieve_kv_swap_out(ctypes.c_void_p(gb.k_pool.data_ptr()), ctypes.c_void_p(gb.v_pool.data_ptr()),
                                  b.num_blocks, ctypes.c_void_p(k_host.data_ptr()),
                                  ctypes.c_void_p(v_host.data_ptr()), 4, ids, ids, 1, b.num_kv_heads, b.head_dim,
                                  0, None)
    assert st == binding.PENSIEVE_ERR_INVALID_ARG
