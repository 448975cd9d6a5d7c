"""Host cache planning: leading-block eviction and recompute-batch construction (no GPU).

The planner ("Stateful Large Language Model Serving with Pensieve", Methodology:
block-level dropping weighed by conversation activity and recompute cost;
recompute of dropped tokens with the next turn) is pinned three ways: its
batches follow the unified-batch convention of the seeded generator (recompute
rows for positions [0, E) ahead of the new rows [H, H + n)); its drops are the
least-cost leading-first drops, found by brute force on small instances; and a
multi-step serving simulation over a bounded pool, run through the CPU oracle,
gives every row exactly the attention of the never-evicted conversation.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import paged_kv_token_amd as pk
from workloads import Batch

import cache_sim

B = 16


def _blocks(t):
    return -(-int(t) // B)


def _random_convs(rng, n, max_tokens=120, p_sched=0.5):
    cached = rng.integers(0, max_tokens, size=n, endpoint=True)
    dropped = np.array([rng.integers(0, _blocks(c), endpoint=True) for c in cached])
    new = np.where(rng.random(n) < p_sched, rng.integers(1, 40, size=n, endpoint=True), 0)
    act = rng.random(n).astype(np.float32)
    return pk.conversations(cached, dropped, new, act)


def _tables_for(rng, convs, stride, num_blocks):
    """Resident blocks of every conversation drawn from one permutation of the pool; -1 for dropped ones."""
    perm = list(rng.permutation(num_blocks).astype(np.int32))
    tables = np.full((len(convs), stride), -1, dtype=np.int32)
    for c, v in enumerate(convs):
        for j in range(int(v["dropped_blocks"]), _blocks(v["cached_tokens"])):
            tables[c, j] = perm.pop()
    return tables, perm


@pytest.mark.parametrize("seed", range(6))
def test_build_batch_follows_the_unified_batch_convention(seed):
    rng = np.random.default_rng(seed)
    convs = _random_convs(rng, 9)
    stride = max(_blocks(v["cached_tokens"] + v["new_tokens"]) for v in convs) + 2
    tables, free = _tables_for(rng, convs, stride, 400)
    before = tables.copy()
    out = pk.pensieve_cache_build_batch(convs, tables, free)
    sched = np.nonzero(convs["new_tokens"] > 0)[0]
    assert list(out["request_conv"]) == list(sched)
    # Fresh blocks: exactly the first blocks_used entries of the free list, each used once.
    taken = [int(tables[c, j]) for c in sched for j in range(stride) if before[c, j] != tables[c, j]]
    assert sorted(taken) == sorted(free[:out["blocks_used"]])
    assert len(set(taken)) == len(taken)
    # Resident blocks keep their place; unscheduled conversations are untouched.
    changed = before != tables
    assert np.all(before[changed] == -1)
    for c in range(len(convs)):
        if c not in sched:
            assert np.array_equal(before[c], tables[c])
    # The batch is the generator's unified batch with E = recomputed, H = cached, n = new.
    cached = convs["cached_tokens"][sched].astype(np.int64)
    rec = np.minimum(B * convs["dropped_blocks"][sched].astype(np.int64), cached)
    ref = Batch("planner", "f32", 2, 2, 64, B, 400, 0, cached, convs["new_tokens"][sched].astype(np.int64), rec,
                out["req_block_tables"])
    assert np.array_equal(out["cu_q_lens"], ref.cu_q_lens)
    assert np.array_equal(out["context_lens"], ref.context_lens)
    assert np.array_equal(out["q_pos"], ref.q_pos)
    assert np.array_equal(out["slot_mapping"], ref.new_slots)
    for r, c in enumerate(sched):
        pos = out["q_pos"][out["cu_q_lens"][r]:out["cu_q_lens"][r + 1]]
        assert np.all(np.diff(pos) > 0)
        assert np.array_equal(out["req_block_tables"][r], tables[c])
        # Every logical block the request reads is mapped after the step.
        assert np.all(tables[c, :_blocks(out["context_lens"][r])] >= 0)
    # No two rows share a slot.
    assert len(set(out["slot_mapping"].tolist())) == len(out["slot_mapping"])


def _drop_cost(v, e):
    d = int(v["dropped_blocks"])
    return float(v["activity"]) * sum(j + 1 for j in range(d, d + e))


def _step_need(convs):
    need = 0
    for v in convs:
        if v["new_tokens"] > 0:
            c, n = int(v["cached_tokens"]), int(v["new_tokens"])
            need += int(v["dropped_blocks"]) + _blocks(c + n) - _blocks(c)
    return need


@pytest.mark.parametrize("seed", range(40))
def test_plan_evictions_is_the_least_cost_leading_first_drop(seed):
    rng = np.random.default_rng(1000 + seed)
    convs = _random_convs(rng, int(rng.integers(2, 6, endpoint=True)), max_tokens=64, p_sched=0.35)
    if seed % 5 == 0:
        convs["activity"][rng.integers(0, len(convs))] = 0.0
    need = _step_need(convs)
    idle = [c for c in range(len(convs)) if convs["new_tokens"][c] == 0]
    avail = {c: _blocks(convs["cached_tokens"][c]) - int(convs["dropped_blocks"][c]) for c in idle}
    free = int(rng.integers(0, need + 1)) if need else 0
    k = max(need - free, 0)
    if k > sum(avail.values()):
        with pytest.raises(pk.PensieveError) as ei:
            pk.pensieve_cache_plan_evictions(convs, free)
        assert ei.value.status == pk.PENSIEVE_ERR_UNSUPPORTED
        return
    evict, freed = pk.pensieve_cache_plan_evictions(convs, free)
    assert freed == k == int(evict.sum())
    for c in range(len(convs)):
        if convs["new_tokens"][c] > 0:
            assert evict[c] == 0
        else:
            assert 0 <= evict[c] <= avail[c]
    got = sum(_drop_cost(convs[c], int(evict[c])) for c in idle)
    best = min((sum(_drop_cost(convs[c], e) for c, e in zip(idle, es))
                for es in itertools.product(*[range(avail[c] + 1) for c in idle]) if sum(es) == k),
               default=0.0)
    assert got == pytest.approx(best, rel=1e-12, abs=1e-12)


def test_plan_evictions_drops_nothing_when_the_step_fits():
    convs = pk.conversations([100, 50, 0], [0, 1, 0], [10, 0, 30], [1.0, 0.1, 1.0])
    evict, freed = pk.pensieve_cache_plan_evictions(convs, _step_need(convs))
    assert freed == 0 and not evict.any()


def test_plan_evictions_takes_idle_conversations_first_and_leading_blocks_first():
    # Conversation 1 (idle a long time, activity 0.01) loses all its blocks before conversation 2
    # (activity 1) loses any: dropping block j costs activity * (j + 1).
    convs = pk.conversations([64, 64, 64, 10], [0, 0, 0, 0], [0, 0, 0, 90], [0.5, 0.01, 1.0, 1.0])
    need = _step_need(convs)             # 6 blocks for conversation 3's 90 new tokens
    assert need == 6
    evict, _ = pk.pensieve_cache_plan_evictions(convs, 1)
    # Costs: conv 1: .01,.02,.03,.04; conv 0: .5, 1.0, ...; conv 2: 1, 2, ... -> 4 of conv 1, 1 of conv 0.
    assert list(evict) == [1, 4, 0, 0]


def test_plan_evictions_reports_an_impossible_step():
    convs = pk.conversations([32, 16], [0, 0], [0, 100], [1.0, 1.0])
    with pytest.raises(pk.PensieveError) as ei:
        pk.pensieve_cache_plan_evictions(convs, 1)
    assert ei.value.status == pk.PENSIEVE_ERR_UNSUPPORTED


def test_build_batch_of_a_fully_dropped_conversation_recomputes_every_token():
    # 37 cached tokens, all 3 blocks dropped (the last one partly filled), 5 new tokens.
    convs = pk.conversations([37], [3], [5], [1.0])
    tables = np.full((1, 4), -1, dtype=np.int32)
    out = pk.pensieve_cache_build_batch(convs, tables, [9, 4, 7, 1])
    assert out["blocks_used"] == 3
    assert list(tables[0]) == [9, 4, 7, -1]
    assert list(out["q_pos"]) == list(range(37)) + [37, 38, 39, 40, 41]
    assert out["slot_mapping"][36] == 7 * B + 4 and out["slot_mapping"][37] == 7 * B + 5
    assert list(out["context_lens"]) == [42]


def test_build_batch_with_nothing_scheduled_is_empty():
    convs = pk.conversations([40, 0], [1, 0], [0, 0], [1.0, 1.0])
    tables = np.full((2, 3), -1, dtype=np.int32)
    out = pk.pensieve_cache_build_batch(convs, tables, [])
    assert out["blocks_used"] == 0 and len(out["q_pos"]) == 0 and list(out["cu_q_lens"]) == [0]


@pytest.mark.parametrize("case", ["dropped_past_end", "negative_new", "nan_activity", "negative_activity",
                                  "stride_too_small", "free_list_short"])
def test_cache_calls_reject_bad_input(case):
    cached, dropped, new, act = [40, 20], [0, 0], [8, 0], [1.0, 1.0]
    stride, free = 4, [1, 2, 3]
    if case == "dropped_past_end":
        dropped = [4, 0]
    elif case == "negative_new":
        new = [-1, 0]
    elif case == "nan_activity":
        act = [1.0, float("nan")]
    elif case == "negative_activity":
        act = [1.0, -0.5]
    elif case == "stride_too_small":
        stride = 2
    elif case == "free_list_short":
        dropped, free = [2, 0], [1]
    convs = pk.conversations(cached, dropped, new, act)
    tables = np.full((2, stride), -1, dtype=np.int32)
    before = tables.copy()
    with pytest.raises(pk.PensieveError) as ei:
        pk.pensieve_cache_build_batch(convs, tables, free)
    assert ei.value.status == pk.PENSIEVE_ERR_INVALID_ARG
    assert np.array_equal(tables, before)
    if case not in ("stride_too_small", "free_list_short"):
        with pytest.raises(pk.PensieveError):
            pk.pensieve_cache_plan_evictions(convs, 10)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 4, 4, 64)])
def test_serving_simulation_through_the_oracle(dtype, hq, hkv, d):
    stats = cache_sim.run(cache_sim.OracleBackend, seed=7, num_convs=12, steps=30, num_blocks=40,
                          num_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, tol=1e-12,
                          script_kw=dict(idle=(2, 10)))
    # The run must exercise the planner: drops, whole-conversation drops and recompute rows.
    assert stats.dropped_blocks > 50 and stats.fully_dropped > 5 and stats.recompute_rows > 300
    assert stats.steps == 30
