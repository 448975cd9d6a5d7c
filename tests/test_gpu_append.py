"""GPU kv_append against the oracle's append: bit-exact on whole pools (cut-down
batches) and on sampled blocks of the full-size workloads."""

import numpy as np
import pytest

import oracle
from gpu_harness import to_host_storage, upload
from oracle_helpers import oracle_pools, poison_fill
from workloads import config_batch, custom_batch, storage_dtype

pytestmark = pytest.mark.gpu


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def _say(msg):
    print(f"[append] {msg}", flush=True)


CASES = {
    "tiny_f32": lambda: config_batch(0),
    "mixed_f16_cut": lambda: config_batch(1, num_reqs=4, num_heads=8),
    "gqa_recompute_bf16_cut": lambda: config_batch(3, num_reqs=3, max_hist=1500),
    "long_bf16_cut": lambda: config_batch(4, num_reqs=2, num_heads=2, max_hist=3000),
    "d64_f16_ragged": lambda: custom_batch([0, 15, 16, 17, 250], [1, 1, 16, 33, 7], num_heads=6, num_kv_heads=3,
                                           head_dim=64, dtype="f16", seed=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_whole_pool_bit_exact(name):
    b = CASES[name]()
    _say(f"{name}: R={b.num_reqs} NB={b.num_blocks} Hkv={b.num_kv_heads} d={b.head_dim} {b.dtype}")
    gb = upload(b)
    k_ref, v_ref = oracle_pools(b)
    k_gpu = to_host_storage(gb.k_pool, b.dtype)
    v_gpu = to_host_storage(gb.v_pool, b.dtype)
    assert k_gpu.shape == k_ref.shape and v_gpu.shape == v_ref.shape
    assert np.array_equal(_bits(k_gpu), _bits(k_ref)), "K pool differs"
    assert np.array_equal(_bits(v_gpu), _bits(v_ref)), "V pool differs"


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_scattered_order_and_skips(dtype):
    """Tokens in random order with scattered slots, some skipped with slot -1."""
    import torch
    import paged_kv_token_amd as pk
    from gpu_harness import poison_, to_device
    rng = np.random.default_rng(11)
    nb, hkv, d, n = 40, 3, 128 if dtype != "f32" else 64, 300
    sd = storage_dtype(dtype)
    slots = rng.permutation(nb * 16)[:n].astype(np.int32)
    slots[rng.choice(n, 20, replace=False)] = -1
    x = rng.standard_normal((2, n, hkv, d)).astype(np.float32)
    if dtype == "f32":
        k_new, v_new = x[0], x[1]
    elif dtype == "f16":
        k_new, v_new = x[0].astype(np.float16), x[1].astype(np.float16)
    else:
        from workloads import bf16_bits_from_f32
        k_new, v_new = bf16_bits_from_f32(x[0]), bf16_bits_from_f32(x[1])
    fill = poison_fill(dtype)
    k_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    v_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    oracle.append_kv(k_ref, v_ref, k_new, v_new, slots, 16)
    _say(f"scattered {dtype}: n={n} nb={nb}")
    from gpu_harness import torch_dtype
    k_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    v_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    pk.pensieve_kv_append(to_device(k_new, dtype), to_device(v_new, dtype), k_pool, v_pool,
                          torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_host_storage(k_pool, dtype)), _bits(k_ref))
    assert np.array_equal(_bits(to_host_storage(v_pool, dtype)), _bits(v_ref))


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_append_full_size_sampled_blocks(index):
    """Full-size workloads: sampled blocks equal the oracle's append of that block's positions."""
    b = config_batch(index)
    _say(f"full {b.name}: R={b.num_reqs} NB={b.num_blocks}")
    gb = upload(b)
    rng = np.random.default_rng(index)
    reqs = rng.choice(b.num_reqs, size=min(6, b.num_reqs), replace=False)
    sd = storage_dtype(b.dtype)
    fill = poison_fill(b.dtype)
    for r in reqs:
        k, v = b.request_kv(int(r))
        nblk = b.num_logical_blocks(int(r))
        for j in sorted(set([0, nblk - 1, int(rng.integers(0, nblk))])):
            phys = int(b.block_tables[r, j])
            mk = np.full((1, b.num_kv_heads, 16, b.head_dim), fill, dtype=sd)
            mv = np.full((1, b.num_kv_heads, 16, b.head_dim), fill, dtype=sd)
            pos = np.arange(16 * j, min(16 * j + 16, int(b.context_lens[r])))
            oracle.append_kv(mk, mv, k[pos], v[pos], (pos % 16).astype(np.int32), 16)
            gk = to_host_storage(gb.k_pool[phys:phys + 1], b.dtype)
            gv = to_host_storage(gb.v_pool[phys:phys + 1], b.dtype)
            assert np.array_equal(_bits(gk), _bits(mk)), (r, j)
            assert np.array_equal(_bits(gv), _bits(mv)), (r, j)


def _run_slots(rng, nb: int) -> np.ndarray:
    """In-order runs starting at every block offset, of lengths that end inside, at and past the
    16-token windows of the append grid; a block whose two halves arrive far apart in the token
    list; skipped tokens inside runs; a token count that is not a multiple of 16."""
    blocks = iter(rng.permutation(nb).tolist())
    slots = []
    for start in range(16):
        for length in (1, 15 - start if start < 15 else 2, 16, 17, 31, 33):
            s = next(blocks) * 16 + start
            for k in range(max(length, 1)):
                if k > 0 and s % 16 == 0:
                    s = next(blocks) * 16
                slots.append(s)
                s += 1
    split = next(blocks) * 16
    slots[5:5] = list(range(split, split + 8))
    slots.extend(range(split + 8, split + 16))
    slots = np.asarray(slots, dtype=np.int32)
    slots[rng.choice(len(slots), 25, replace=False)] = -1
    return slots[:len(slots) - 3]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_runs_across_windows(dtype):
    """Runs that start anywhere in a block and cross the append grid's 16-token windows are
    written exactly once: whole pools equal the oracle's append bit for bit."""
    import torch
    import paged_kv_token_amd as pk
    from gpu_harness import poison_, to_device, torch_dtype
    rng = np.random.default_rng(23)
    nb, hkv, d = 420, 2, 128 if dtype != "f32" else 64
    slots = _run_slots(rng, nb)
    n = len(slots)
    assert n % 16 != 0
    sd = storage_dtype(dtype)
    x = rng.standard_normal((2, n, hkv, d)).astype(np.float32)
    if dtype == "f32":
        k_new, v_new = x[0], x[1]
    elif dtype == "f16":
        k_new, v_new = x[0].astype(np.float16), x[1].astype(np.float16)
    else:
        from workloads import bf16_bits_from_f32
        k_new, v_new = bf16_bits_from_f32(x[0]), bf16_bits_from_f32(x[1])
    fill = poison_fill(dtype)
    k_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    v_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    oracle.append_kv(k_ref, v_ref, k_new, v_new, slots, 16)
    _say(f"runs {dtype}: n={n} nb={nb}")
    k_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    v_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    pk.pensieve_kv_append(to_device(k_new, dtype), to_device(v_new, dtype), k_pool, v_pool,
                          torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_host_storage(k_pool, dtype)), _bits(k_ref))
    assert np.array_equal(_bits(to_host_storage(v_pool, dtype)), _bits(v_ref))


def _random_run_slots(rng, nb: int) -> np.ndarray:
    """Requests' new tokens as in-order runs from random block offsets; then pieces of that list
    moved elsewhere (a block's tokens then arrive in several places), and some tokens skipped."""
    blocks = iter(rng.permutation(nb).tolist())
    slots = []
    while len(slots) < int(rng.integers(40, 400)):
        s = next(blocks) * 16 + int(rng.integers(0, 16))
        for k in range(int(rng.integers(1, 70))):
            if k > 0 and s % 16 == 0:
                s = next(blocks) * 16
            slots.append(s)
            s += 1
    slots = np.asarray(slots, dtype=np.int32)
    for _ in range(int(rng.integers(0, 4))):
        lo = int(rng.integers(0, len(slots)))
        hi = min(len(slots), lo + int(rng.integers(1, 24)))
        piece, rest = slots[lo:hi], np.concatenate([slots[:lo], slots[hi:]])
        at = int(rng.integers(0, len(rest) + 1))
        slots = np.concatenate([rest[:at], piece, rest[at:]]).astype(np.int32)
    slots[rng.random(len(slots)) < 0.05] = -1
    return slots


@pytest.mark.parametrize("seed", range(12))
def test_append_random_run_layouts(seed):
    """Random run layouts (in order, pieces moved, skips), f16 d = 128 and f32 d = 64 alternately:
    whole pools equal the oracle's append bit for bit."""
    import torch
    import paged_kv_token_amd as pk
    from gpu_harness import poison_, to_device, torch_dtype
    rng = np.random.default_rng(700 + seed)
    dtype, d = ("f16", 128) if seed % 2 == 0 else ("f32", 64)
    nb, hkv = 160, 2
    slots = _random_run_slots(rng, nb)
    n = len(slots)
    sd = storage_dtype(dtype)
    x = rng.standard_normal((2, n, hkv, d)).astype(np.float32)
    k_new, v_new = (x[0].astype(np.float16), x[1].astype(np.float16)) if dtype == "f16" else (x[0], x[1])
    fill = poison_fill(dtype)
    k_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    v_ref = np.full((nb, hkv, 16, d), fill, dtype=sd)
    oracle.append_kv(k_ref, v_ref, k_new, v_new, slots, 16)
    _say(f"random runs seed {seed} {dtype}: n={n}")
    k_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    v_pool = poison_(torch.empty((nb, hkv, 16, d), dtype=torch_dtype(dtype), device="cuda"), dtype)
    pk.pensieve_kv_append(to_device(k_new, dtype), to_device(v_new, dtype), k_pool, v_pool,
                          torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(to_host_storage(k_pool, dtype)), _bits(k_ref))
    assert np.array_equal(_bits(to_host_storage(v_pool, dtype)), _bits(v_ref))
