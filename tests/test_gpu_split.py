"""GPU split-KV partials and merge against the oracle's split definition."""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, run_split, to_f64, upload
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
    # the largest partition count: 256 partitions of a 5000-token prefill and of short requests
    "p256_max_bf16": (lambda: custom_batch([4950, 60, 0], [50, 1, 7], num_heads=4, num_kv_heads=2, head_dim=64,
                                           dtype="bf16", seed=53), 256),
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


ADAPTIVE = {
    # one long decode request among short ones: only it is cut (vector kernel partials)
    "long_decode_among_short_f16": lambda: custom_batch([20000] + [300] * 12, [1] * 13, num_heads=8, num_kv_heads=8,
                                                        head_dim=128, dtype="f16", seed=61),
    # long prefill (matrix-core partials, GQA) and long decode beside a short request
    "long_prefill_gqa_bf16": lambda: custom_batch([6000, 9000, 200], [300, 1, 5], num_heads=8, num_kv_heads=2,
                                                  head_dim=128, dtype="bf16", seed=62),
    # partially evicted history recomputed ahead of new rows, d = 64
    "recompute_d64_f16": lambda: custom_batch([5000, 40], [64, 3], [752, 0], num_heads=4, num_kv_heads=4,
                                              head_dim=64, dtype="f16", seed=63),
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", sorted(ADAPTIVE))
def test_adaptive_split_in_attn_fwd(name, path):
    """pensieve_attn_fwd cuts the long requests (checked on the plan) and still matches the oracle;
    the workspace starts as NaN, so a partial the merge reads without a kernel writing it shows."""
    b = ADAPTIVE[name]()
    gb = upload(b)
    plan = pk.pensieve_debug_plan(gb.make_desc(PATHS[path]))
    parts = {int(row[1]): int(row[6]) for row in plan[plan[:, 4] > 0]}
    longest = int(np.argmax(b.context_lens))
    _say(f"adaptive {name}/{path}: partitions {parts}")
    assert parts[longest] > 1 and min(parts.values()) == 1
    ref = oracle_output(b)
    got = to_f64(run_attn(gb, PATHS[path]))
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    _say(f"adaptive {name}/{path}: max abs err {err:.3e}")
    assert err <= 1e-2


def test_no_split_flag_matches_the_oracle():
    b = ADAPTIVE["long_decode_among_short_f16"]()
    gb = upload(b)
    ref = oracle_output(b)
    got = to_f64(run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT))
    err = float(np.max(np.abs(got - ref)))
    _say(f"no-split flag: max abs err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= 1e-2
