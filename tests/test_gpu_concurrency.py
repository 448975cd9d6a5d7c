"""Several host threads, each on its own stream, call the library at once.

The staging ring, the plan scratch (per thread), the side stream of the fork/join and the
trace state are shared by the process; outputs must be bitwise those of the same calls made
one after another (the kernels' arithmetic does not depend on what runs beside them).
"""

import threading

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import upload
from workloads import config_batch, custom_batch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[threads] {msg}", flush=True)


def test_concurrent_calls_from_host_threads_match_serial_calls():
    import torch
    batches = [config_batch(1, num_reqs=4, num_heads=8),
               config_batch(3, num_reqs=3, max_hist=900),
               custom_batch([5000, 40, 300], [1, 3, 64], num_heads=8, num_kv_heads=2, head_dim=64, dtype="f16",
                            seed=31),
               config_batch(0)]
    gbs = [upload(b) for b in batches]

    def call(gb, o, ws, stream):
        pk.pensieve_attn_fwd(gb.make_desc(), gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                             gb.cu_q_lens, gb.q_pos, o, ws, stream=stream)

    wss = [torch.empty(max(pk.pensieve_attn_workspace_size(gb.make_desc()), 256), dtype=torch.uint8, device="cuda")
           for gb in gbs]
    ref = []
    for gb, ws in zip(gbs, wss):
        o = torch.empty_like(gb.q)
        call(gb, o, ws, torch.cuda.current_stream())
        ref.append(o)
    torch.cuda.synchronize()

    reps = 25
    outs = [[torch.empty_like(gb.q) for _ in range(reps)] for gb in gbs]
    streams = [torch.cuda.Stream() for _ in gbs]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for k in range(reps):
                    call(gbs[i], outs[i][k], wss[i], streams[i])
        except Exception as e:   # reported below; a thread's exception would otherwise vanish
            errors.append(e)

    pk.pensieve_trace_enable(True, 2)         # the shared trace state is exercised too
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(gbs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    records = pk.pensieve_trace_read()
    pk.pensieve_trace_enable(False)
    assert not errors, errors
    _say(f"{len(gbs)} threads x {reps} calls; {len(records)} traced launches")
    for i, gb in enumerate(gbs):
        for k in range(reps):
            assert torch.equal(outs[i][k].view(torch.uint8), ref[i].view(torch.uint8)), (i, k)
