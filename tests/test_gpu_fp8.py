"""FP8 (E4M3) KV pools on the GPU against the CPU oracle.

* pensieve_kv_append_fp8 is bit-exact: every pool byte equals the oracle's E4M3 code of
  value / scale (float32 division, round to nearest even, saturation at 448), on random rows
  plus spliced-in ties, subnormal-range values, zeros of both signs, saturating values and
  infinities, with scattered and skipped slots.
* Attention over E4M3 pools (both kernels, split partials, the adaptive split inside
  pensieve_attn_fwd) matches the oracle's attention over the decoded codes times the scales
  within 1e-2: the codes are widened exactly, so only fp32 accumulation and the rounding of
  the softmax weights differ from the float64 reference, as for f16 / bf16 pools.
* A swap round trip of E4M3 blocks leaves attention bitwise unchanged.
"""

import numpy as np
import pytest

import oracle
import paged_kv_token_amd as pk
from gpu_harness import run_attn, run_split, to_device, to_f64, upload
from oracle_helpers import fp8_kw, oracle_output, oracle_pools, oracle_split
from workloads import config_batch, custom_batch, draw_rows

pytestmark = pytest.mark.gpu

TOL = 1e-2
SCALES = (1 / 64, 1 / 48)
PATHS = {"default": 0, "vector": pk.PENSIEVE_FLAG_VECTOR_ONLY}


def _say(msg):
    print(f"[fp8] {msg}", flush=True)


def _special_values():
    """Values (in units of the scale) that probe rounding: every tie of the E4M3 grid, the
    subnormal range, zeros, saturation and infinities."""
    grid = oracle.E4M3_VALUES[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2
    extra = np.array([0.0, -0.0, 448.0, 464.0, 470.0, 500.0, 1e4, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12,
                      -2.0 ** -12, np.inf, -np.inf])
    return np.concatenate([mids, -mids, grid, -grid, extra])


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [1 / 64, 1.0, 0.0123])
def test_append_fp8_is_bit_exact(src, d, scale):
    import torch
    hkv, nb, n = 3, 24, 150
    rng = np.random.default_rng(5)
    k = draw_rows((31, d, 1), (n, hkv, d), src)
    v = draw_rows((31, d, 2), (n, hkv, d), src)
    # Splice special values (times the scale, rounded to the source type) into both tensors.
    sp = _special_values() * scale
    sp_store = (torch.from_numpy(sp.astype(np.float32)).to(torch.float16 if src == "f16" else torch.bfloat16))
    sp_store = sp_store.view(torch.int16).numpy().view(np.float16 if src == "f16" else np.uint16)
    for arr in (k, v):
        flat = arr.reshape(-1)
        where = rng.choice(flat.size, size=len(sp_store), replace=False)
        flat[where] = sp_store
    # Scattered slots: runs inside blocks, single tokens, a skipped token every 11th.
    runs = np.concatenate([np.arange(16 * 5, 16 * 5 + 40),     # an aligned run over whole blocks
                           np.arange(16 * 9 + 3, 16 * 9 + 10)])  # an unaligned run
    rest = np.setdiff1d(np.arange(nb * 16), runs)
    slots = np.concatenate([runs, rng.permutation(rest)[:n - len(runs)]]).astype(np.int32)
    slots[::11] = -1                                             # distinct slots, some skipped
    _say(f"append {src} d={d} scale={scale}: {n} tokens, {int((slots >= 0).sum())} written")
    kp = np.full((nb, hkv, 16, d), 0xAA, np.uint8)
    vp = np.full((nb, hkv, 16, d), 0xAA, np.uint8)
    oracle.append_kv(kp, vp, oracle.quantize_e4m3(k, src, scale), oracle.quantize_e4m3(v, src, scale), slots, 16)
    gk = torch.full((nb, hkv, 16, d), 0xAA, dtype=torch.uint8, device="cuda")
    gv = torch.full((nb, hkv, 16, d), 0xAA, dtype=torch.uint8, device="cuda")
    pk.pensieve_kv_append_fp8(to_device(k, src), to_device(v, src), gk, gv, torch.from_numpy(slots).cuda(),
                              scale, scale)
    torch.cuda.synchronize()
    got_k, got_v = gk.cpu().numpy(), gv.cpu().numpy()
    bad = int((got_k != kp).sum() + (got_v != vp).sum())
    if bad:
        i = np.argwhere(got_k != kp)[:4]
        _say(f"mismatches {bad}; first K: {[(tuple(x), hex(got_k[tuple(x)]), hex(kp[tuple(x)])) for x in i]}")
    assert bad == 0


CASES = {
    "mixed_f16_cut": lambda: config_batch(1, num_reqs=6, num_heads=8),
    "decode_f16_cut": lambda: config_batch(2, num_reqs=24, num_heads=8),
    "gqa_recompute_bf16_cut": lambda: config_batch(3, num_reqs=4, max_hist=1200),
    "long_bf16_cut": lambda: config_batch(4, num_reqs=4, num_heads=4, max_hist=3000),
    "gqa4_d64_f16_ragged": lambda: custom_batch([0, 15, 16, 17, 250, 63, 64], [1, 1, 16, 33, 7, 65, 64],
                                                num_heads=8, num_kv_heads=2, head_dim=64, dtype="f16", seed=21),
    "mha_d64_bf16_long_rows": lambda: custom_batch([100, 0], [300, 257], num_heads=2, num_kv_heads=2,
                                                   head_dim=64, dtype="bf16", seed=22),
    "gqa16_f16": lambda: custom_batch([40, 200], [20, 3], num_heads=16, num_kv_heads=1, head_dim=128,
                                      dtype="f16", seed=23),
    "gqa8_decode_bf16": lambda: custom_batch([0, 1, 15, 16, 63, 64, 65, 700, 1999], [1] * 9, num_heads=16,
                                             num_kv_heads=2, head_dim=128, dtype="bf16", seed=25),
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_attention_parity(name, path):
    b = CASES[name]()
    _say(f"attn {name}/{path}: R={b.num_reqs} T={b.total_q} Hq={b.num_heads} Hkv={b.num_kv_heads} "
         f"d={b.head_dim} {b.dtype} maxL={int(b.context_lens.max())}")
    ref = oracle_output(b, pools=oracle_pools(b, kv_fp8=SCALES), **fp8_kw(SCALES))
    gb = upload(b, kv_fp8=SCALES)
    got = to_f64(run_attn(gb, PATHS[path]))
    assert np.all(np.isfinite(got)), "non-finite output"
    err = float(np.max(np.abs(got - ref)))
    _say(f"attn {name}/{path}: max abs err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name,P", [("gqa_recompute_bf16_cut", 4), ("decode_f16_cut", 3)])
def test_fp8_split_partials(name, P):
    b = CASES[name]()
    pools = oracle_pools(b, kv_fp8=SCALES)
    rpo, rpm, rpl = oracle_split(b, P, pools=pools, **fp8_kw(SCALES))
    gb = upload(b, kv_fp8=SCALES)
    po, pm, pl, o = run_split(gb, P)
    po, pm, pl, o = to_f64(po), to_f64(pm), to_f64(pl), to_f64(o)
    live = rpl > 0
    assert np.array_equal(live, pl > 0)
    assert np.max(np.abs(pm[live] - rpm[live])) <= 1e-3
    assert np.max(np.abs(pl[live] / rpl[live] - 1)) <= 1e-2
    assert np.max(np.abs(po[live] - rpo[live])) <= TOL
    ref = oracle_output(b, pools=pools, **fp8_kw(SCALES))
    err = float(np.max(np.abs(o - ref)))
    _say(f"split {name} P={P}: merged max abs err {err:.3e}")
    assert err <= TOL


def test_fp8_adaptive_split_in_attn_fwd():
    b = custom_batch([20000] + [300] * 6, [1] * 7, num_heads=8, num_kv_heads=8, head_dim=128, dtype="f16",
                     seed=61)
    gb = upload(b, kv_fp8=SCALES)
    plan = pk.pensieve_debug_plan(gb.make_desc())
    parts = {int(row[1]): int(row[6]) for row in plan[plan[:, 4] > 0]}
    assert parts[0] > 1
    ref = oracle_output(b, pools=oracle_pools(b, kv_fp8=SCALES), **fp8_kw(SCALES))
    got = to_f64(run_attn(gb))
    err = float(np.max(np.abs(got - ref)))
    _say(f"adaptive split: partitions {parts[0]}, max abs err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL


def test_fp8_swap_round_trip_leaves_attention_bitwise_unchanged():
    import torch
    b = config_batch(3, num_reqs=3, max_hist=900)
    gb = upload(b, kv_fp8=SCALES)
    before = run_attn(gb).clone()
    used = b.used_blocks()
    rng = np.random.default_rng(8)
    nh = len(used) + 3
    k_host = torch.empty((nh,) + tuple(gb.k_pool.shape[1:]), dtype=torch.uint8).pin_memory()
    v_host = torch.empty((nh,) + tuple(gb.v_pool.shape[1:]), dtype=torch.uint8).pin_memory()
    host_ids = rng.permutation(nh)[:len(used)].astype(np.int32)
    pk.pensieve_kv_swap_out(gb.k_pool, gb.v_pool, k_host, v_host, used, host_ids)
    torch.cuda.synchronize()
    gb.k_pool.fill_(0x7F)
    gb.v_pool.fill_(0x7F)
    new_ids = rng.permutation(b.num_blocks)[:len(used)].astype(np.int32)
    pk.pensieve_kv_swap_in(gb.k_pool, gb.v_pool, k_host, v_host, host_ids, new_ids)
    remap = np.full(b.num_blocks, -1, np.int64)
    remap[used] = new_ids
    bt = b.block_tables.copy()
    for r in range(b.num_reqs):
        nl = b.num_logical_blocks(r)
        bt[r, :nl] = remap[bt[r, :nl]]
    gb.block_tables = torch.from_numpy(bt).cuda()
    torch.cuda.synchronize()
    after = run_attn(gb)
    assert torch.equal(before.view(torch.int16), after.view(torch.int16))


def test_fp8_pool_offsets_beyond_4_gib():
    """Blocks placed past byte 2^32 of 4.6 GB E4M3 pools: append and both kernels must address them
    with 64-bit offsets (reference: the oracle over each request's logical K/V, quantised)."""
    import torch
    nb = 300_000                                 # 8 KV heads x 16 x 128 bytes = 16 KiB per block
    b = custom_batch([700, 1500, 33, 90], [1, 40, 5, 1], num_heads=16, num_kv_heads=8, head_dim=128,
                     dtype="bf16", seed=77, num_blocks=nb)
    bt = b.block_tables.copy()
    top = nb - 1
    for r in range(b.num_reqs):
        n = b.num_logical_blocks(r)
        bt[r, :n] = top - np.arange(n) * 7 - r   # descending ids near the end of the pool
    used = np.concatenate([bt[r, :b.num_logical_blocks(r)] for r in range(b.num_reqs)])
    assert len(np.unique(used)) == len(used)
    b.block_tables = bt
    assert (int(bt.max()) + 1) * 8 * 16 * 128 > 2 ** 32
    gb = upload(b, kv_fp8=SCALES)
    for path in sorted(PATHS):
        got = to_f64(run_attn(gb, PATHS[path]))
        q = b.q_all()
        err = 0.0
        for r in range(b.num_reqs):
            k, v = b.request_kv(r)
            lo, hi = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
            for h in range(b.num_heads):
                g = h // 2
                kk = oracle.e4m3_decode(oracle.quantize_e4m3(k[:, g], b.dtype, SCALES[0])) * SCALES[0]
                vv = oracle.e4m3_decode(oracle.quantize_e4m3(v[:, g], b.dtype, SCALES[1])) * SCALES[1]
                ref = oracle.causal_attention(oracle.to_f64(q[lo:hi, h], b.dtype), kk, vv, b.query_positions(r),
                                              b.softmax_scale)
                err = max(err, float(np.max(np.abs(got[lo:hi, h] - ref))))
        _say(f"pool past 4 GiB ({path}): max abs err {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= TOL
    del gb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("index", [1, 2, 3])
def test_full_size_fp8_sampled_parity(index):
    """The workloads the benchmark times with E4M3 pools, at full size: sampled (request, head)
    outputs against the oracle over each request's quantised logical K/V."""
    scales = (1 / 128, 1 / 128)
    b = config_batch(index)
    _say(f"full-size {b.name}: R={b.num_reqs} T={b.total_q}")
    gb = upload(b, kv_fp8=scales)
    got = to_f64(run_attn(gb))
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(300 + index)
    reqs = sorted(set(rng.choice(b.num_reqs, size=3, replace=False).tolist() + [int(np.argmax(b.context_lens))]))
    heads = sorted(set([0, b.num_heads - 1] + rng.choice(b.num_heads, size=2, replace=False).tolist()))
    G = b.num_heads // b.num_kv_heads
    q = b.q_all()
    worst = 0.0
    for r in reqs:
        k, v = b.request_kv(r)
        lo, hi = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
        for h in heads:
            g = h // G
            kk = oracle.e4m3_decode(oracle.quantize_e4m3(k[:, g], b.dtype, scales[0])) * scales[0]
            vv = oracle.e4m3_decode(oracle.quantize_e4m3(v[:, g], b.dtype, scales[1])) * scales[1]
            ref = oracle.causal_attention(oracle.to_f64(q[lo:hi, h], b.dtype), kk, vv, b.query_positions(r),
                                          b.softmax_scale)
            worst = max(worst, float(np.max(np.abs(got[lo:hi, h] - ref))))
    _say(f"full-size {b.name}: requests {reqs} heads {heads}: max abs err {worst:.3e}")
    assert worst <= TOL
    del gb
