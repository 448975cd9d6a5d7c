"""Matrix-core items in eight-wave workgroups (256 query vectors, one workgroup per CU), against
the CPU oracle.  The plan uses them in calls whose 128-vector items would not fill one round of
the GPU and that hold a request of more than 128 query vectors per KV head: a long prefill or
recompute request beside decode rows ("Stateful Large Language Model Serving with Pensieve",
Methodology: prefill, recompute and decode rows of one step in one batch).  Each case covers
head groups of 1-32, head_dim 64 and 128, f16 and bf16, recomputed leading rows, a short
matrix-core request in the same launch (its items leave waves idle) and ragged row counts,
through the default plan, the unsplit plan, one stream, the explicit split pair and the call that
allocates nothing.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import poison_, run_attn, run_split, to_f64, upload
from oracle_helpers import oracle_output, oracle_pools
from workloads import custom_batch

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "bf16": 1e-2}


def _say(msg):
    print(f"[wide] {msg}", flush=True)


def _widest(gb, flags=0, P=0):
    plan = pk.pensieve_debug_plan(gb.make_desc(flags), P)
    live = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
    G = gb.batch.num_heads // gb.batch.num_kv_heads
    return int((live[:, 4] * G).max()) if len(live) else 0


def _noalloc(gb):
    import torch
    o = torch.empty_like(gb.q)
    poison_(o, gb.batch.dtype)
    pk.pensieve_attn_fwd_noalloc(gb.make_desc(0), gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                                 gb.cu_q_lens, gb.q_pos, o)
    torch.cuda.synchronize()
    return o


CASES = [(1, 128, "bf16"), (1, 64, "f16"), (2, 128, "f16"), (4, 64, "bf16"), (8, 128, "bf16"),
         (8, 64, "f16"), (16, 128, "f16"), (32, 128, "bf16"), (32, 64, "bf16")]


@pytest.mark.parametrize("G,d,dtype", CASES)
def test_eight_wave_items_match_the_oracle(G, d, dtype):
    # Request 0: 64 recomputed rows + 237 new (ragged against 256 / G tokens per item); request 1:
    # a short matrix-core request; 2: decode; 3: prefill with no history.
    b = custom_batch([2500, 900, 1800, 0], [237, 20, 1, 40], [64, 0, 0, 0], num_heads=2 * G, num_kv_heads=2,
                     head_dim=d, dtype=dtype, seed=400 + G + d)
    ref = oracle_output(b, pools=oracle_pools(b))
    gb = upload(b)
    assert _widest(gb) > 128, "the plan should use eight-wave items"
    outs = {
        "default": lambda: run_attn(gb, 0),
        "no_split": lambda: run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT),
        "single_stream": lambda: run_attn(gb, pk.PENSIEVE_FLAG_SINGLE_STREAM),
        "split3": lambda: run_split(gb, 3)[3],
        "noalloc": lambda: _noalloc(gb),
    }
    for name, fn in outs.items():
        got = to_f64(fn())
        assert np.all(np.isfinite(got)), name
        err = float(np.max(np.abs(got - ref)))
        _say(f"G={G} d={d} {dtype} {name}: max abs err {err:.3e}")
        assert err <= TOL[dtype], (name, err)


@pytest.mark.parametrize("G,dtype", [(1, "f16"), (8, "bf16")])
def test_eight_wave_items_past_the_first_block_window(G, dtype):
    """Unsplit items over 20 000 keys (313 tiles): each wave's block ids come from more than two
    64-tile windows of its register-held block table, refilled as the item streams."""
    b = custom_batch([20000, 3000], [300, 1], num_heads=2 * G, num_kv_heads=2, head_dim=128, dtype=dtype,
                     seed=450 + G)
    ref = oracle_output(b, pools=oracle_pools(b))
    gb = upload(b)
    assert _widest(gb, pk.PENSIEVE_FLAG_NO_SPLIT) > 128
    got = to_f64(run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT))
    err = float(np.max(np.abs(got - ref)))
    # Relative to the output's own scale too: at 20 000 keys |O| is small.
    rel = err / float(np.max(np.abs(ref)))
    _say(f"G={G} {dtype} unsplit 20k keys: max abs err {err:.3e} (relative {rel:.2e})")
    assert err <= TOL[dtype] and rel <= 5e-2


def _random_case(seed: int):
    """Few KV heads, one request above 128 query vectors per KV head, up to four more (decode,
    prefill, recompute), so the call usually takes eight-wave items; histories to 6 000 tokens."""
    rng = np.random.default_rng(123000 + seed)
    G = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hkv = int(rng.choice([1, 2]))
    R = int(rng.integers(1, 6))
    hist = rng.integers(0, 6000, size=R)
    new = np.where(rng.random(R) < 0.5, 1, rng.integers(1, 400, size=R))
    new[0] = int(rng.integers(max(1, 129 // G + 1), 600))
    ev = np.array([16 * int(rng.integers(1, min(16, h // 32) + 1)) if h >= 32 and rng.random() < 0.3 else 0
                   for h in hist])
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    b = custom_batch(hist, new, ev, num_heads=hkv * G, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                     seed=124000 + seed)
    return b, int(rng.integers(2, 9))


@pytest.mark.parametrize("seed", range(16))
def test_random_batches_through_eight_wave_items(seed):
    b, P = _random_case(seed)
    gb = upload(b)
    widest = _widest(gb)
    ref = oracle_output(b, pools=oracle_pools(b))
    for name, fn in (("default", lambda: run_attn(gb, 0)), ("no_split", lambda: run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT)),
                     (f"split{P}", lambda: run_split(gb, P)[3])):
        got = to_f64(fn())
        assert np.all(np.isfinite(got)), name
        err = float(np.max(np.abs(got - ref)))
        _say(f"seed {seed} G={b.num_heads // b.num_kv_heads} d={b.head_dim} {b.dtype} q={b.q_lens.tolist()} "
             f"widest item {widest} vectors, {name}: max abs err {err:.3e}")
        assert err <= TOL[b.dtype], (seed, name, err)


def test_random_batches_mostly_take_eight_wave_items():
    """The seeded draws above exercise the eight-wave path: most of them plan 256-vector items
    (checked on the host, no GPU work)."""
    wide = 0
    for seed in range(16):
        b, _ = _random_case(seed)
        desc = pk.make_desc(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                            num_blocks=b.num_blocks, block_table_stride=b.block_table_stride,
                            dtype={"f16": 1, "bf16": 2}[b.dtype], softmax_scale=b.softmax_scale,
                            context_lens_host=b.context_lens, cu_q_lens_host=b.cu_q_lens,
                            q_pos_host=None if b.has_default_positions else b.q_pos)
        plan = pk.pensieve_debug_plan(desc)
        live = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
        wide += int((live[:, 4] * (b.num_heads // b.num_kv_heads)).max()) > 128
    assert wide >= 10, wide


@pytest.mark.parametrize("G,dtype", [(1, "bf16"), (4, "f16"), (8, "bf16"), (32, "f16")])
def test_eight_wave_items_on_e4m3_pools(G, dtype):
    """E4M3 pools at head_dim 128 (each wave loads one 1 KB half of a 2 KB block): the codes
    widen exactly, so the output matches the oracle over the same E4M3 pools at the gate
    ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3): the KV cache kept in 8-bit floats)."""
    from oracle_helpers import fp8_kw
    scales = (1 / 64, 1 / 48)
    b = custom_batch([2500, 900, 1800, 0], [237, 20, 1, 40], [64, 0, 0, 0], num_heads=2 * G, num_kv_heads=2,
                     head_dim=128, dtype=dtype, seed=470 + G)
    ref = oracle_output(b, pools=oracle_pools(b, kv_fp8=scales), **fp8_kw(scales))
    gb = upload(b, kv_fp8=scales)
    assert _widest(gb) > 128, "the plan should use eight-wave items"
    for name, fn in (("default", lambda: run_attn(gb, 0)), ("no_split", lambda: run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT)),
                     ("split3", lambda: run_split(gb, 3)[3])):
        got = to_f64(fn())
        assert np.all(np.isfinite(got)), name
        err = float(np.max(np.abs(got - ref)))
        _say(f"E4M3 G={G} {dtype} {name}: max abs err {err:.3e}")
        assert err <= TOL[dtype], (name, err)
