"""GPU split-KV partials and merge against the oracle's split definition."""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_split, to_f64, upload
from oracle_helpers import oracle_output, oracle_pools, oracle_split
from workloads import config_batch, custom_batch

pytestmark = pytest.mark.gpu
PATHS = {"default": 0, "vector": pk.PENSIEVE_FLAG_VECTOR_ONLY}


def _say(msg):
    print(f"[split] {msg}", flush=True)


CASES = {
    "long_bf16_cut_p32": (lambda: config_batch(4, num_reqs=4, num_heads=4, max_hist=3000), 32),
    "recompute_bf16_p8": (lambda: config_batch(3, num_reqs=3, max_hist=1000), 8),
    "few_blocks_f16_p16": (lambda: custom_batch([20, 0, 100], [3, 9, 1], num_heads=4, num_kv_heads=2,
                                                head_dim=128, dtype="f16", seed=51), 16),
    "tiny_f32_p4": (lambda: config_batch(0), 4),
    "p1_f16": (lambda: custom_batch([300, 5], [40, 1], num_heads=2, num_kv_heads=2, head_dim=64, dtype="f16",
                                    seed=52), 1),
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", sorted(CASES))
def test_split_partials_and_merge(name, path):
    factory, P = CASES[name]
    b = factory()
    _say(f"{name}/{path}: P={P} R={b.num_reqs} T={b.total_q} {b.dtype}")
    pools = oracle_pools(b)
    ro, rm, rl = oracle_split(b, P, pools=pools)
    ref = oracle_output(b, pools=pools)
    gb = upload(b)
    po, pm, pl, o = run_split(gb, P, PATHS[path])
    po, pm, pl, o = to_f64(po), to_f64(pm), to_f64(pl), to_f64(o)
    tol = 1e-4 if b.dtype == "f32" else 1e-2
    empty = rl == 0
    assert np.array_equal(pl == 0, empty), "empty partitions differ"
    assert np.all(pm[empty] == -np.inf) and np.all(po[empty] == 0)
    live = ~empty
    assert np.all(np.abs(pm[live] - rm[live]) <= 1e-3 + 1e-3 * np.abs(rm[live]))
    assert np.all(np.abs(pl[live] - rl[live]) <= 1e-2 * rl[live])
    assert float(np.max(np.abs(po - ro))) <= tol
    assert np.all(np.isfinite(o))
    err = float(np.max(np.abs(o - ref)))
    _say(f"{name}/{path}: merged max abs err {err:.3e}")
    assert err <= tol
