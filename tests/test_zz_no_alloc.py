"""pensieve_attn_fwd_noalloc (the library's own device scratch instead of a caller workspace).

Through the C ABI: two calls in a row, the second with a smaller batch, each bitwise equal to
pensieve_attn_fwd on the same inputs and within the tolerance of the oracle.  The first batch has
a long request that the adaptive plan splits, so its partials and the merge run from the scratch
array; it also mixes matrix-core and vector items, which pensieve_attn_fwd forks onto its side
stream and the no-alloc call keeps on the caller's stream.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import poison_, run_attn, to_f64, to_host_storage, upload
from oracle_helpers import oracle_output
from workloads import custom_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)


def _noalloc(gb):
    import torch
    o = torch.empty_like(gb.q)
    poison_(o, gb.batch.dtype)
    pk.pensieve_attn_fwd_noalloc(gb.desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                                 gb.cu_q_lens, gb.q_pos, o)
    torch.cuda.synchronize()
    return o


def test_noalloc_matches_attn_fwd_on_two_calls():
    big = custom_batch([20000, 300, 0, 1500, 77], [1, 40, 12, 64, 1], num_heads=8, num_kv_heads=2, head_dim=128,
                       dtype="bf16", seed=91)
    small = custom_batch([100, 37], [5, 1], num_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=92)
    for b in (big, small):
        gb = upload(b)
        split_ws = pk.pensieve_attn_workspace_size(gb.desc)
        whole_ws = pk.pensieve_attn_workspace_size(gb.make_desc(pk.PENSIEVE_FLAG_NO_SPLIT))
        _say(f"R={b.num_reqs} T={b.total_q} maxL={int(b.context_lens.max())} workspace {split_ws} B "
             f"(unsplit {whole_ws} B)")
        if b is big:
            assert split_ws > whole_ws, "the long request should be split"
        ref = to_host_storage(run_attn(gb), b.dtype)
        got = _noalloc(gb)
        assert np.array_equal(to_host_storage(got, b.dtype), ref)
        err = float(np.max(np.abs(to_f64(got) - oracle_output(b))))
        _say(f"bitwise equal to attn_fwd; max abs err vs oracle {err:.2e}")
        assert err <= 1e-2


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    """Work list plus partials beyond the 64 MiB scratch: refused on the host before anything is enqueued."""
    import torch
    # A 512-row prefill beside a 200k-token decode request: the decode request is cut into many
    # partitions, and the partials of every split row are sized for the largest count.
    ctx = np.array([49664, 200001], np.int32)
    cu = np.array([0, 512, 513], np.int32)
    nblk = -(-int(ctx.max()) // 16)
    desc = pk.make_desc(num_heads=40, num_kv_heads=40, head_dim=128, num_blocks=int((-(-ctx // 16)).sum()),
                        block_table_stride=nblk,
                        dtype=pk.PENSIEVE_BF16, softmax_scale=128 ** -0.5, context_lens_host=ctx,
                        cu_q_lens_host=cu)
    need = pk.pensieve_attn_workspace_size(desc)
    _say(f"workspace of the oversized batch: {need} B")
    assert need > (64 << 20)
    # Small real buffers stand in for the pools and tables: the call must fail before any launch.
    dummy = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    q = torch.zeros((513, 40, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    import ctypes
    vp = ctypes.c_void_p
    d = vp(dummy.data_ptr())
    st = pk.load_library().pensieve_attn_fwd_noalloc(ctypes.byref(desc), vp(q.data_ptr()), d, d, d, d, d, None,
                                                     vp(o.data_ptr()), None)
    torch.cuda.synchronize()
    assert st == pk.binding.PENSIEVE_ERR_WORKSPACE_TOO_SMALL
