"""The five workloads at full size, in the launch configuration the benchmark
times: sampled (request, head) outputs against the oracle computed one request
at a time from the seeded values, plus properties that hold at any size."""

import numpy as np
import pytest

from gpu_harness import run_attn, run_split, to_f64, upload
from oracle_helpers import request_rows_reference
from workloads import config_batch

pytestmark = pytest.mark.gpu

SAMPLES = {0: (3, 4), 1: (6, 3), 2: (8, 3), 3: (3, 3), 4: (4, 2)}   # (requests, heads) per workload


def _say(msg):
    print(f"[full] {msg}", flush=True)


def _pick_requests(b, k, rng):
    if b.num_reqs <= k:
        return list(range(b.num_reqs))
    cost = b.q_lens.astype(np.int64) * b.context_lens
    cheap = np.argsort(cost)[: max(k, b.num_reqs // 2)]
    picks = set(rng.choice(cheap, size=k - 1, replace=False).tolist())
    picks.add(int(np.argmax(b.context_lens)))     # always include the longest context
    return sorted(picks)


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_full_size_sampled_parity(index):
    b = config_batch(index)
    tol = 1e-4 if b.dtype == "f32" else 1e-2
    _say(f"{b.name}: R={b.num_reqs} T={b.total_q} sumL={int(b.context_lens.sum())}")
    gb = upload(b)
    outs = {"attn": to_f64(run_attn(gb))}
    if index == 4:
        outs["split32"] = to_f64(run_split(gb, 32)[3])
    rng = np.random.default_rng(100 + index)
    nreq, nhead = SAMPLES[index]
    reqs = _pick_requests(b, nreq, rng)
    heads = sorted(set([0, b.num_heads - 1] + rng.choice(b.num_heads, size=nhead, replace=False).tolist()))
    for name, o in outs.items():
        assert np.all(np.isfinite(o)), name
        assert np.max(np.abs(o)) <= 0.5 * 6.5, name   # |O| is bounded by max |V| (|V| <= 0.5 * 6.5 sigma here)
    for r in reqs:
        lo, hi = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
        for h in heads:
            ref = request_rows_reference(b, r, h)
            for name, o in outs.items():
                err = float(np.max(np.abs(o[lo:hi, h, :] - ref)))
                assert err <= tol, (name, r, h, err)
    _say(f"{b.name}: sampled requests {reqs} heads {heads} ok")
