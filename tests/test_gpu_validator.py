"""The PENSIEVE_DEBUG=1 device-contract validator.

With the variable set, every append and attention call copies its device metadata to the host
and refuses a contract violation with INVALID_ARG before anything is enqueued: slots past the
pool or repeated, block ids outside the pool, device lengths that differ from their host copies,
query positions out of order or past the context.  Each violation below is also memory-safe if
it ever reached a kernel: the pools handed to the library sit inside larger buffers (eight spare
blocks on each side), the bad lengths only shrink what a kernel would read, and bad positions
are clamped by the kernels' own key ranges.  The output buffer must stay untouched.
"""

import ctypes

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, to_host_storage, upload
from workloads import custom_batch

pytestmark = pytest.mark.gpu
PAD = 8   # spare blocks on each side of the pools


def _say(msg):
    print(f"[validator] {msg}", flush=True)


def _batch():
    b = custom_batch([300, 45, 0, 700], [20, 1, 33, 4], evict_lens=[0, 0, 0, 64], num_heads=8, num_kv_heads=2,
                     head_dim=128, dtype="bf16", seed=81)
    return b


def _padded_pools(gb):
    """Copies of the pools inside buffers with PAD spare blocks before and after."""
    import torch
    out = []
    for pool in (gb.k_pool, gb.v_pool):
        big = torch.full((pool.shape[0] + 2 * PAD,) + tuple(pool.shape[1:]), float("nan"), dtype=pool.dtype,
                         device="cuda")
        big[PAD:PAD + pool.shape[0]].copy_(pool)
        out.append(big)
    return out


def _attn_raw(gb, desc, kbig, vbig, bt, ctx, cu, qp, o, ws):
    vp = ctypes.c_void_p
    blk = gb.k_pool[0].numel() * gb.k_pool.element_size()
    return pk.load_library().pensieve_attn_fwd(
        ctypes.byref(desc), vp(gb.q.data_ptr()), vp(kbig.data_ptr() + PAD * blk), vp(vbig.data_ptr() + PAD * blk),
        vp(bt.data_ptr()), vp(ctx.data_ptr()), vp(cu.data_ptr()), vp(qp.data_ptr()) if qp is not None else None,
        vp(o.data_ptr()), vp(ws.data_ptr()), ws.numel(), None)


def test_valid_batch_passes_with_identical_output(monkeypatch):
    b = _batch()
    gb = upload(b)
    ref = to_host_storage(run_attn(gb), b.dtype)
    monkeypatch.setenv("PENSIEVE_DEBUG", "1")
    got = to_host_storage(run_attn(gb), b.dtype)
    assert np.array_equal(ref, got)
    pk.pensieve_kv_append(gb.k_new, gb.v_new, gb.k_pool, gb.v_pool, gb.new_slots)


def test_attention_violations_are_refused(monkeypatch):
    import torch
    b = _batch()
    gb = upload(b)
    assert gb.q_pos is not None
    kbig, vbig = _padded_pools(gb)
    desc = gb.make_desc()
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
    bt0, ctx0, cu0, qp0 = (gb.block_tables.clone(), gb.context_lens.clone(), gb.cu_q_lens.clone(),
                           gb.q_pos.clone())
    o = torch.full_like(gb.q, 7.0)
    monkeypatch.setenv("PENSIEVE_DEBUG", "1")
    assert _attn_raw(gb, desc, kbig, vbig, bt0, ctx0, cu0, qp0, o, ws) == 0
    torch.cuda.synchronize()
    good = to_host_storage(o, b.dtype)
    nb = b.num_blocks

    def case(name, edit):
        bt, ctx, cu, qp = bt0.clone(), ctx0.clone(), cu0.clone(), qp0.clone()
        edit(bt, ctx, cu, qp)
        out = torch.full_like(gb.q, 7.0)
        st = _attn_raw(gb, desc, kbig, vbig, bt, ctx, cu, qp, out, ws)
        torch.cuda.synchronize()
        msg = pk.load_library().pensieve_last_error().decode()
        _say(f"{name}: status {st} ({msg})")
        assert st == pk.PENSIEVE_ERR_INVALID_ARG, name
        assert "PENSIEVE_DEBUG" in msg
        assert bool(torch.all(out == 7.0)), f"{name}: the output was written"

    def set_(t, idx, val):
        t[idx] = val

    case("block id past the pool", lambda bt, ctx, cu, qp: set_(bt, (0, 3), nb))
    case("negative block id", lambda bt, ctx, cu, qp: set_(bt, (3, 0), -1))
    case("last block id past the pool", lambda bt, ctx, cu, qp: set_(bt, (2, -(-33 // 16) - 1), nb + 3))
    case("device context length differs", lambda bt, ctx, cu, qp: set_(ctx, 0, int(b.context_lens[0]) - 5))
    case("device cu_q_lens differs", lambda bt, ctx, cu, qp: set_(cu, 1, int(b.cu_q_lens[1]) - 1))
    lo3 = int(b.cu_q_lens[3])
    case("positions out of order", lambda bt, ctx, cu, qp: set_(qp, lo3 + 1, int(qp0[lo3])))
    case("position at the context length", lambda bt, ctx, cu, qp: set_(qp, int(b.cu_q_lens[4]) - 1,
                                                                         int(b.context_lens[3])))
    case("negative position", lambda bt, ctx, cu, qp: set_(qp, 0, -1))
    # the refusals left nothing behind: the valid call still gives the same bits
    o2 = torch.full_like(gb.q, 7.0)
    assert _attn_raw(gb, desc, kbig, vbig, bt0, ctx0, cu0, qp0, o2, ws) == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host_storage(o2, b.dtype), good)


def test_append_violations_are_refused(monkeypatch):
    import torch
    b = _batch()
    gb = upload(b)
    kbig, vbig = _padded_pools(gb)
    blk = gb.k_pool[0].numel() * gb.k_pool.element_size()
    before = (kbig.clone(), vbig.clone())
    vp = ctypes.c_void_p
    monkeypatch.setenv("PENSIEVE_DEBUG", "1")
    n = b.total_q

    def call(slots):
        st = pk.load_library().pensieve_kv_append(vp(gb.k_new.data_ptr()), vp(gb.v_new.data_ptr()),
                                                  vp(kbig.data_ptr() + PAD * blk), vp(vbig.data_ptr() + PAD * blk),
                                                  vp(slots.data_ptr()), n, b.num_kv_heads, b.head_dim, 16,
                                                  b.num_blocks, pk.PENSIEVE_BF16, None)
        torch.cuda.synchronize()
        return st

    s = gb.new_slots.clone()
    s[5] = b.num_blocks * 16 + 3
    assert call(s) == pk.PENSIEVE_ERR_INVALID_ARG
    s = gb.new_slots.clone()
    s[7] = s[2]
    assert call(s) == pk.PENSIEVE_ERR_INVALID_ARG
    for new, old in zip((kbig, vbig), before):
        assert np.array_equal(to_host_storage(new, b.dtype), to_host_storage(old, b.dtype))
    s = gb.new_slots.clone()
    s[4] = -1                         # skipping a token is allowed
    assert call(s) == 0
