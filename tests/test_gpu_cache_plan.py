"""Serving simulation with eviction and recompute on the GPU.

The host planner's batches (pensieve_cache_plan_evictions / pensieve_cache_build_batch)
drive pensieve_kv_append and pensieve_attn_fwd over a bounded, NaN-poisoned block
pool for 30 steps; every row of every step is compared with plain causal attention
of the CPU oracle over the conversation's whole, never-evicted K/V (for E4M3 pools: its
decoded codes times the scales).  Tolerances: 1e-4 for f32, 1e-2 for f16/bf16 (absolute, per
element).
"""

from __future__ import annotations

import sys

import pytest

import cache_sim


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # dtype, Hq, Hkv, d, conversations, pool blocks, tol
    ("f16", 8, 2, 128, 12, 40, 1e-2),
    ("bf16", 4, 4, 64, 16, 48, 1e-2),
    ("f32", 4, 2, 64, 12, 40, 1e-4),
    ("fp8-bf16", 16, 2, 128, 12, 40, 1e-2),     # E4M3 pools under bf16 queries
    ("fp8-f16", 4, 4, 64, 16, 48, 1e-2),
]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,hq,hkv,d,nc,nb,tol", CASES)
def test_serving_simulation_on_gpu(dtype, hq, hkv, d, nc, nb, tol):
    _say(f"[cache-plan sim] {dtype} Hq={hq} Hkv={hkv} d={d} convs={nc} blocks={nb}")
    backend = cache_sim.GpuFp8Backend if dtype.startswith("fp8-") else cache_sim.GpuBackend
    stats = cache_sim.run(backend, seed=11, num_convs=nc, steps=30, num_blocks=nb, num_heads=hq,
                          num_kv_heads=hkv, head_dim=d, dtype=dtype.replace("fp8-", ""), tol=tol,
                          script_kw=dict(idle=(2, 10)))
    _say(f"  rows={stats.rows} recompute={stats.recompute_rows} dropped={stats.dropped_blocks} "
         f"max_err={stats.max_err:.2e}")
    assert stats.dropped_blocks > 0 and stats.recompute_rows > 0
