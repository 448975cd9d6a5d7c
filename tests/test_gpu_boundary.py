"""The C-ABI boundary on the GPU: shape checks in the binding, refusal of graph capture, and the
single-stream flag (every launch on the caller's stream gives the same bits as the forked plan)."""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, to_f64, to_host_storage, upload
from workloads import custom_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[boundary] {msg}", flush=True)


def _mixed():
    # Prefill rows (matrix cores) beside decode rows (vector kernel): the default plan forks.
    return custom_batch([300, 1200, 0, 500], [40, 1, 12, 1], num_heads=4, num_kv_heads=4, head_dim=128,
                        dtype="f16", seed=61)


def test_single_stream_flag_is_bitwise_equal():
    b = _mixed()
    gb = upload(b)
    plan = pk.pensieve_debug_plan(gb.desc)
    assert {int(k) for k in plan[:, 0]} == {0, 1}, "the batch should have both kinds of items"
    a = to_host_storage(run_attn(gb), b.dtype)
    s = to_host_storage(run_attn(gb, pk.PENSIEVE_FLAG_SINGLE_STREAM), b.dtype)
    assert np.array_equal(a, s)


def test_binding_rejects_mismatched_shapes():
    import torch
    b = _mixed()
    gb = upload(b)
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(gb.desc), 256), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(gb.q)
    args = dict(q=gb.q, k_pool=gb.k_pool, v_pool=gb.v_pool, block_tables=gb.block_tables,
                context_lens=gb.context_lens, cu_q_lens=gb.cu_q_lens, q_pos=gb.q_pos, o=o, workspace=ws)
    bad = {
        "q": gb.q[:-1].contiguous(),
        "o": torch.empty((b.total_q, b.num_heads, b.head_dim // 2), dtype=gb.q.dtype, device="cuda"),
        "k_pool": gb.k_pool[:-1].contiguous(),
        "v_pool": gb.v_pool.transpose(2, 3).contiguous(),
        "block_tables": gb.block_tables[:, :-1].contiguous(),
        "context_lens": gb.context_lens[:-1].contiguous(),
        "cu_q_lens": gb.cu_q_lens[:-1].contiguous(),
        "q_pos": torch.zeros(b.total_q + 1, dtype=torch.int32, device="cuda"),
    }
    for name, t in bad.items():
        kw = dict(args)
        kw[name] = t
        with pytest.raises(ValueError):
            pk.pensieve_attn_fwd(gb.desc, **kw)
        _say(f"{name}: rejected")
    with pytest.raises(ValueError):
        pk.pensieve_kv_append(gb.k_new, gb.v_new[:-1].contiguous(), gb.k_pool, gb.v_pool, gb.new_slots)
    with pytest.raises(ValueError):
        pk.pensieve_kv_append(gb.k_new, gb.v_new, gb.k_pool, gb.v_pool, gb.new_slots[:-1].contiguous())
    k_host = torch.empty((4,) + tuple(gb.k_pool.shape[1:]), dtype=gb.k_pool.dtype).pin_memory()
    v_host = torch.empty((5,) + tuple(gb.v_pool.shape[1:]), dtype=gb.v_pool.dtype).pin_memory()
    with pytest.raises(ValueError):
        pk.pensieve_kv_swap_out(gb.k_pool, gb.v_pool, k_host, v_host, [0], [1])
    torch.cuda.synchronize()


def test_graph_capture_is_refused():
    """The calls build and upload their work list per call, so a capturing stream is refused before
    anything is enqueued (nothing of ours enters the graph)."""
    import torch
    b = _mixed()
    gb = upload(b)
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(gb.desc), 256), dtype=torch.uint8, device="cuda")
    o = torch.zeros_like(gb.q)
    x = torch.zeros(16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    status = None
    with torch.cuda.stream(side):
        g.capture_begin()
        try:
            x.add_(1.0)
            try:
                pk.pensieve_attn_fwd(gb.desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                                     gb.cu_q_lens, gb.q_pos, o, ws, stream=side)
            except pk.PensieveError as e:
                status = e.status
        finally:
            g.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert status == pk.PENSIEVE_ERR_UNSUPPORTED
    g.replay()
    torch.cuda.synchronize()
    assert float(x[0]) == 1.0
    assert not torch.any(o != 0)


def test_work_list_beyond_a_staging_slot():
    """A work list larger than one staging slot (19 200 items, 600 KB against 512 KiB slots) goes
    up through a page-locked buffer of its own; two calls in a row match the oracle, and a small
    batch afterwards still does."""
    from oracle_helpers import oracle_output
    rng = np.random.default_rng(5)
    R = 600
    big = custom_batch(rng.integers(16, 300, size=R), np.ones(R, np.int64), num_heads=32, num_kv_heads=32,
                       head_dim=64, dtype="f16", seed=91)
    gb = upload(big)
    n_items = len(pk.pensieve_debug_plan(gb.desc))
    assert n_items * 32 > 512 * 1024
    ref = oracle_output(big)
    for call in range(2):
        err = float(np.max(np.abs(to_f64(run_attn(gb)) - ref)))
        _say(f"{n_items} items, call {call}: max abs err {err:.3e}")
        assert err <= 1e-2
    small = _mixed()
    ref_s = oracle_output(small)
    err = float(np.max(np.abs(to_f64(run_attn(upload(small))) - ref_s)))
    _say(f"small batch after: max abs err {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("wait_us", [None, "0"])
def test_staging_ring_reuse_while_the_host_runs_ahead(wait_us, monkeypatch):
    """120 attention calls enqueued back to back on one stream with no host wait, over three
    batches with different work lists, so the host laps the 32-slot staging ring while copies of
    earlier calls may still be pending (a slot is refilled only after the copy kernel that read it
    has reported, through its flags, that it is done); a swap-out after every seventh call takes
    the other way of recycling a slot (an event).  Every output equals bitwise that of a
    synchronised call of its batch.  With the wait limit at zero microseconds, a slot whose flags
    have not arrived is recovered at once through the bounded wait's device synchronisation."""
    import torch
    if wait_us is not None:
        monkeypatch.setenv("PENSIEVE_STAGE_WAIT_US", wait_us)
    rng = np.random.default_rng(11)
    batches = [
        _mixed(),
        custom_batch([3000] * 8, [64] * 8, num_heads=32, num_kv_heads=32, head_dim=128, dtype="bf16", seed=62),
        custom_batch(rng.integers(100, 3000, size=64), np.ones(64, np.int64), num_heads=16, num_kv_heads=4,
                     head_dim=64, dtype="f16", seed=63),
    ]
    gbs = [upload(b) for b in batches]
    refs = [to_host_storage(run_attn(gb), gb.batch.dtype) for gb in gbs]
    wss = [torch.empty(max(pk.pensieve_attn_workspace_size(gb.desc), 256), dtype=torch.uint8, device="cuda")
           for gb in gbs]
    g0 = gbs[0]
    blocks = g0.batch.block_tables[0, :4].tolist()
    k_host = torch.empty((4,) + tuple(g0.k_pool.shape[1:]), dtype=g0.k_pool.dtype).pin_memory()
    v_host = torch.empty((4,) + tuple(g0.v_pool.shape[1:]), dtype=g0.v_pool.dtype).pin_memory()
    outs = []
    for i in range(120):
        j = i % 3
        gb = gbs[j]
        o = torch.empty_like(gb.q)
        pk.pensieve_attn_fwd(gb.desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens, gb.cu_q_lens,
                             gb.q_pos, o, wss[j])
        outs.append((j, o))
        if i % 7 == 6:
            pk.pensieve_kv_swap_out(g0.k_pool, g0.v_pool, k_host, v_host, blocks, list(range(4)))
    torch.cuda.synchronize()
    bad = [i for i, (j, o) in enumerate(outs) if not np.array_equal(to_host_storage(o, gbs[j].batch.dtype), refs[j])]
    _say(f"120 calls enqueued without a wait (wait limit {wait_us} us): {len(bad)} outputs differ")
    assert not bad
    assert np.array_equal(k_host.cpu().numpy().view(np.uint16),
                          g0.k_pool[torch.tensor(blocks, device="cuda")].cpu().numpy().view(np.uint16))
