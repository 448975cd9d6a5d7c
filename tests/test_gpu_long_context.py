"""Structured parity at the long-context workload's real lengths (32k-65k keys).

"PersistentKV: Page-Aware Decode Scheduling for Long-Context LLM Serving on Commodity GPUs",
section 2 (one long context cut into partitions).  Zero-query signature values and one-hot rows
(tests/long_cases.py) make a single wrong block or a slipped causal boundary show up far beyond
the gate at every length (the margins are derived on the CPU in test_long_context_pins.py).
Every case runs with both kernels (default routing, vector only) and three plans: never split
(whole partitions of up to 1025 tiles, so the matrix-core kernel streams far past its first 128
tiles), the adaptive split of pensieve_attn_fwd, and the explicit 32-way split pair.  The bf16
cases also run on E4M3 pools ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3)) with both
scales 1, where the structured values are exact codes (pinned on the CPU), so the same closed
forms and gates apply.  The largest context (a decode row on 262 144 keys, 4 096 tiles, beside a
64-row prefill on 131 072 history tokens) runs the signature case through the same plans plus
the 256-way split pair, the most partitions a request can have.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, run_split, to_f64, upload
from long_cases import (MAX_HIST, MAX_NEW, ONEHOT_TOL, onehot_batch, onehot_expected, signature_batch,
                        signature_expected, signature_tol)

pytestmark = pytest.mark.gpu

KERNELS = {"default": 0, "vector": pk.PENSIEVE_FLAG_VECTOR_ONLY}
PLANS = ("no_split", "adaptive", "split32")


def _say(msg):
    print(f"[long] {msg}", flush=True)


def _run(gb, plan, kflag):
    if plan.startswith("split"):
        return to_f64(run_split(gb, int(plan[5:]), kflag)[3])
    return to_f64(run_attn(gb, kflag | (pk.PENSIEVE_FLAG_NO_SPLIT if plan == "no_split" else 0)))


def _longest_matrix_partition_tiles(gb):
    """Tiles (64 keys) of the longest partition any matrix-core item streams, unsplit plan."""
    plan = pk.pensieve_debug_plan(gb.make_desc(pk.PENSIEVE_FLAG_NO_SPLIT))
    b = gb.batch
    best = 0
    for kern, r, g, q0, qc, part, nparts, cost, h0, hc in plan:
        if kern == 1 and qc > 0:
            best = max(best, -(-int(b.context_lens[r]) // 64))
    return best


CASES = [pytest.param(dt, g, f8, id=f"{dt}-g{g}" + ("-e4m3" if f8 else ""))
         for dt, g, f8 in [("bf16", 1, None), ("bf16", 8, None), ("f16", 1, None), ("bf16", 1, (1.0, 1.0)),
                           ("bf16", 8, (1.0, 1.0))]]


@pytest.mark.parametrize("dtype,group,kv_fp8", CASES)
def test_signature_zero_query_at_long_lengths(dtype, group, kv_fp8):
    b = signature_batch(dtype, group)
    _say(f"signature {dtype} G={group} fp8={kv_fp8}: L={b.context_lens.tolist()} T={b.total_q}")
    gb = upload(b, kv_fp8=kv_fp8)
    assert _longest_matrix_partition_tiles(gb) > 128
    exp = signature_expected(b)
    tol = signature_tol(exp, dtype)
    for kname, kflag in KERNELS.items():
        for plan in PLANS:
            got = _run(gb, plan, kflag)
            assert np.all(np.isfinite(got)), (kname, plan)
            bad = np.abs(got - exp) > tol
            worst = float(np.max(np.abs(got - exp) / tol))
            _say(f"  {kname}/{plan}: worst |err|/tol {worst:.3f}")
            assert not bad.any(), (kname, plan, np.argwhere(bad)[:5].tolist())


@pytest.mark.parametrize("dtype,group,kv_fp8", CASES)
def test_onehot_rows_in_every_tile(dtype, group, kv_fp8):
    b = onehot_batch(dtype, group)
    _say(f"one-hot {dtype} G={group} fp8={kv_fp8}: L={b.context_lens.tolist()} rows per request {b.q_lens.tolist()}")
    gb = upload(b, kv_fp8=kv_fp8)
    assert gb.q_pos is not None
    assert _longest_matrix_partition_tiles(gb) > 128
    exp = onehot_expected(b)
    for kname, kflag in KERNELS.items():
        for plan in PLANS:
            got = _run(gb, plan, kflag)
            err = np.abs(got - exp)
            _say(f"  {kname}/{plan}: max abs err {float(err.max()):.3e}")
            assert np.all(np.isfinite(got)) and float(err.max()) <= ONEHOT_TOL, (kname, plan)


@pytest.mark.parametrize("dtype,group", [("bf16", 1), ("bf16", 8)])
def test_signature_zero_query_at_the_largest_context(dtype, group):
    b = signature_batch(dtype, group, hist=MAX_HIST, new=MAX_NEW, seed=303)
    _say(f"largest context {dtype} G={group}: L={b.context_lens.tolist()} T={b.total_q}")
    gb = upload(b)
    assert _longest_matrix_partition_tiles(gb) >= 2049
    exp = signature_expected(b)
    tol = signature_tol(exp, dtype)
    for kname, kflag in KERNELS.items():
        for plan in PLANS + ("split256",):
            got = _run(gb, plan, kflag)
            assert np.all(np.isfinite(got)), (kname, plan)
            worst = float(np.max(np.abs(got - exp) / tol))
            _say(f"  {kname}/{plan}: worst |err|/tol {worst:.3f}")
            assert worst <= 1.0, (kname, plan, np.argwhere(np.abs(got - exp) > tol)[:5].tolist())
