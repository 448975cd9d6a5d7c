"""Seeded random unified batches through every attention path, against the CPU oracle.

Each case draws its own shape: 1-10 requests with histories of 0-2500 tokens (some with up to
four dropped leading blocks that come back as recompute rows, some without any query row), 0-150
new rows, head groups of 1-8 over 1-4 KV heads, head_dim 64 or 128, f32 / f16 / bf16, and E4M3
pools for about a third of the 16-bit cases; eight wider cases reach 20 000-token histories, 600
new rows, 32 dropped blocks, head groups of 32 and 64 partitions.  Every case runs through the default plan, the
vector kernel alone, the unsplit plan, one stream, the call that allocates nothing and the
explicit split pair (2-9 partitions, then the merge), each compared with the float64 oracle
element by element at the dtype's gate ("Stateful Large Language Model Serving with Pensieve",
Methodology: one batch mixes prefill, decode and recompute rows over a scattered cache).
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import poison_, run_attn, run_split, to_f64, upload
from oracle_helpers import fp8_kw, oracle_output, oracle_pools
from workloads import custom_batch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}
SCALES = (1 / 64, 1 / 48)
NOALLOC_SCRATCH = 64 << 20   # bytes of the library's scratch array


def _say(msg):
    print(f"[random] {msg}", flush=True)


def _case(seed: int):
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.integers(1, 11))
    hist = np.where(rng.random(R) < 0.2, 0, rng.integers(0, 2501, size=R))
    new = np.where(rng.random(R) < 0.15, 0, rng.integers(1, 151, size=R))
    ev = np.array([16 * int(rng.integers(1, min(4, h // 32) + 1)) if h >= 32 and rng.random() < 0.3 else 0
                   for h in hist], dtype=np.int64)
    if int((ev + new).sum()) == 0:
        new[0] = 1
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    kv_fp8 = SCALES if dtype != "f32" and rng.random() < 0.35 else None
    P = int(rng.integers(2, 10))
    b = custom_batch(hist, new, ev, num_heads=hkv * group, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                     seed=7100 + seed, name=f"random_{seed}")
    return b, kv_fp8, P


def _wide_case(seed: int):
    """Wider draws: histories to 20 000 tokens, up to 600 new rows and 32 dropped blocks, head
    groups to 32, E4M3 pools for half the 16-bit cases, 2-64 partitions."""
    rng = np.random.default_rng(90000 + seed)
    R = int(rng.integers(1, 7))
    hist = np.where(rng.random(R) < 0.15, 0, rng.integers(0, 20001, size=R))
    new = np.where(rng.random(R) < 0.1, 0, rng.integers(1, 601, size=R))
    ev = np.array([16 * int(rng.integers(1, min(32, h // 32) + 1)) if h >= 32 and rng.random() < 0.4 else 0
                   for h in hist], dtype=np.int64)
    if int((ev + new).sum()) == 0:
        new[0] = 1
    group = int(rng.choice([1, 2, 4, 8, 16, 32]))
    hkv = int(rng.choice([1, 2])) if group >= 16 else int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    kv_fp8 = SCALES if dtype != "f32" and rng.random() < 0.5 else None
    P = int(rng.integers(2, 65))
    b = custom_batch(hist, new, ev, num_heads=hkv * group, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                     seed=91000 + seed, name=f"random_wide_{seed}")
    return b, kv_fp8, P


def _noalloc(gb):
    import torch
    o = torch.empty_like(gb.q)
    poison_(o, gb.batch.dtype)
    pk.pensieve_attn_fwd_noalloc(gb.make_desc(0), gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                                 gb.cu_q_lens, gb.q_pos, o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("wide,seed", [(False, s) for s in range(24)] + [(True, s) for s in range(8)])
def test_random_batch_every_path(wide, seed):
    b, kv_fp8, P = (_wide_case if wide else _case)(seed)
    _say(f"seed {seed}: R={b.num_reqs} q={b.q_lens.tolist()} L={b.context_lens.tolist()} Hq={b.num_heads} "
         f"Hkv={b.num_kv_heads} d={b.head_dim} {b.dtype} e4m3={kv_fp8 is not None} P={P}")
    ref = oracle_output(b, pools=oracle_pools(b, kv_fp8=kv_fp8), **fp8_kw(kv_fp8))
    gb = upload(b, kv_fp8=kv_fp8)
    outs = {
        "default": lambda: run_attn(gb, 0),
        "vector": lambda: run_attn(gb, pk.PENSIEVE_FLAG_VECTOR_ONLY),
        "no_split": lambda: run_attn(gb, pk.PENSIEVE_FLAG_NO_SPLIT),
        "single_stream": lambda: run_attn(gb, pk.PENSIEVE_FLAG_SINGLE_STREAM),
        "noalloc": lambda: _noalloc(gb) if pk.pensieve_attn_workspace_size(gb.desc) <= NOALLOC_SCRATCH else None,
        f"split{P}": lambda: run_split(gb, P)[3],
    }
    for name, fn in outs.items():
        out = fn()
        if out is None:   # beyond the allocation-free call's scratch: refused by design, tested elsewhere
            continue
        got = to_f64(out)
        assert np.all(np.isfinite(got)), name
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        _say(f"  {name}: max abs err {err:.3e}")
        assert err <= TOL[b.dtype], (seed, name, err)
