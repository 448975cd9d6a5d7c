"""GPU generalized paged attention against the CPU oracle.

Element-wise parity on seeded batches that span several tiles with ragged
tails, for both kernels (matrix-core default routing and vector-only), plus
structured cases that the flat N(0,1)*0.5 workloads cannot see: a zero query
(exact mean of the visible values), one-hot attention (routing), NaN-poisoned
stale slots, request-order shuffles, empty requests and GQA.
"""

import numpy as np
import pytest

import paged_kv_token_amd as pk
from gpu_harness import run_attn, to_f64, upload
from oracle_helpers import oracle_output
from workloads import config_batch, custom_batch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}
PATHS = {"default": 0, "vector": pk.PENSIEVE_FLAG_VECTOR_ONLY}


def _say(msg):
    print(f"[attn] {msg}", flush=True)


def _max_err(got, ref):
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


CASES = {
    "tiny_f32": lambda: config_batch(0),
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
    "gqa32_d64_bf16": lambda: custom_batch([0, 70, 300], [5, 1, 33], num_heads=32, num_kv_heads=1, head_dim=64,
                                           dtype="bf16", seed=26),
    "gqa8_decode_bf16": lambda: custom_batch([0, 1, 15, 16, 63, 64, 65, 700, 1999], [1] * 9, num_heads=16,
                                             num_kv_heads=2, head_dim=128, dtype="bf16", seed=25),
    "f32_d128_gqa2": lambda: custom_batch([30, 0, 77], [3, 40, 1], num_heads=4, num_kv_heads=2, head_dim=128,
                                          dtype="f32", seed=24),
    # Head groups that do not divide 32 run on the vector kernel in items of up to 8 query vectors
    # that hold whole tokens' groups where they fit (G = 3, 5, 6) or part of one group (G = 12, 64).
    "gqa5_f16": lambda: custom_batch([300, 0, 2000, 77], [5, 40, 1, 130], num_heads=10, num_kv_heads=2,
                                     head_dim=128, dtype="f16", seed=27),
    "gqa3_d64_bf16": lambda: custom_batch([40, 900, 16], [33, 1, 17], num_heads=12, num_kv_heads=4, head_dim=64,
                                          dtype="bf16", seed=28),
    "gqa6_f32": lambda: custom_batch([100, 5], [7, 60], num_heads=12, num_kv_heads=2, head_dim=64, dtype="f32",
                                     seed=29),
    "gqa12_bf16": lambda: custom_batch([600, 31], [2, 45], num_heads=24, num_kv_heads=2, head_dim=128,
                                       dtype="bf16", seed=30),
    "gqa64_f16": lambda: custom_batch([1500, 64], [1, 9], num_heads=64, num_kv_heads=1, head_dim=128, dtype="f16",
                                      seed=32),
}


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", sorted(CASES))
def test_parity_with_oracle(name, path):
    b = CASES[name]()
    _say(f"{name}/{path}: R={b.num_reqs} T={b.total_q} Hq={b.num_heads} Hkv={b.num_kv_heads} d={b.head_dim} "
         f"{b.dtype} maxL={int(b.context_lens.max())}")
    ref = oracle_output(b)
    gb = upload(b)
    got = to_f64(run_attn(gb, PATHS[path]))
    err = _max_err(got, ref)
    _say(f"{name}/{path}: max abs err {err:.3e}")
    assert err <= TOL[b.dtype]


def test_paths_agree_closely():
    """Matrix-core and vector kernels agree far inside the gate on the same inputs."""
    b = config_batch(3, num_reqs=3, max_hist=900)
    gb = upload(b)
    a = to_f64(run_attn(gb, 0))
    v = to_f64(run_attn(gb, pk.PENSIEVE_FLAG_VECTOR_ONLY))
    # the matrix path rounds softmax weights to bf16 before P.V: allow two output ulps
    assert np.all(np.isfinite(a)) and np.all(np.abs(a - v) <= 2.0 ** -6 * np.abs(v) + 1e-3)


@pytest.mark.parametrize("dtype,group", [("f16", 1), ("bf16", 8), ("bf16", 1), ("f16", 4)])
def test_zero_query_exact_mean(dtype, group):
    """Q = 0 and V[t] = (-1)^t * 256: O[i] = 256/(p+1) for even p, else 0 (any one-key slip is gross)."""
    A = 256.0
    hkv = 2
    hq = hkv * group
    b = custom_batch([1800, 37, 0, 3000, 500], [1, 90, 130, 1, 64], [0, 0, 0, 0, 480], num_heads=hq,
                     num_kv_heads=hkv, head_dim=128, dtype=dtype, seed=31)
    b.q_fn = lambda r: np.zeros((int(b.q_lens[r]), hq, 128), np.float32)
    b.v_fn = lambda r: (A * (-1.0) ** np.arange(int(b.context_lens[r])))[:, None, None] * np.ones((1, hkv, 128),
                                                                                                   np.float32)
    _say(f"zero-query {dtype} G={group}")
    gb = upload(b)
    for path, flags in PATHS.items():
        got = to_f64(run_attn(gb, flags))
        exp = np.zeros_like(got)
        for r in range(b.num_reqs):
            lo = int(b.cu_q_lens[r])
            for i, p in enumerate(b.query_positions(r)):
                exp[lo + i] = A / (p + 1) if p % 2 == 0 else 0.0
        ulp = 2.0 ** (-7 if dtype == "bf16" else -10)
        bad = np.abs(got - exp) > ulp * np.abs(exp) + 1e-7
        assert not bad.any(), f"{path}: {np.argwhere(bad)[:5]}"


@pytest.mark.parametrize("dtype,group", [("f16", 1), ("bf16", 8)])
def test_one_hot_routing(dtype, group):
    """Q[i] = 4 K[p_i] with random +-1 keys: each row returns (almost exactly) V at its own position."""
    hkv, d = 2, 128
    hq = hkv * group
    b = custom_batch([700, 0, 1500], [33, 70, 1], [0, 0, 0], num_heads=hq, num_kv_heads=hkv, head_dim=d,
                     dtype=dtype, seed=32)
    rng = np.random.default_rng(5)
    ks = {r: rng.choice([-1.0, 1.0], size=(int(b.context_lens[r]), hkv, d)).astype(np.float32)
          for r in range(b.num_reqs)}
    b.k_fn = lambda r: ks[r]
    b.q_fn = lambda r: 4.0 * np.repeat(ks[r][b.query_positions(r)], group, axis=1)
    _say(f"one-hot {dtype} G={group}")
    gb = upload(b)
    for path, flags in PATHS.items():
        got = to_f64(run_attn(gb, flags))
        for r in range(b.num_reqs):
            _, v = b.request_kv(r)
            vv = v.astype(np.float32) if dtype == "f16" else (v.astype(np.uint32) << 16).view(np.float32)
            lo = int(b.cu_q_lens[r])
            pos = b.query_positions(r)
            for h in range(hq):
                exp = vv[pos, h // group, :]
                err = np.max(np.abs(got[lo:lo + len(pos), h, :] - exp))
                assert err <= 1e-2, (path, r, h, err)


def test_nan_poison_and_block_table_tails():
    """Stale slots are NaN; block-table entries past each request's blocks name a NaN block."""
    b = config_batch(1, num_reqs=5, num_heads=4)
    ref = oracle_output(b)
    spare = min(set(range(b.num_blocks)) - set(b.used_blocks().tolist()))
    bt = b.block_tables.copy()
    for r in range(b.num_reqs):
        bt[r, b.num_logical_blocks(r):] = spare
    b.block_tables = np.concatenate([bt, np.full((b.num_reqs, 3), spare, np.int32)], axis=1)
    gb = upload(b)  # pools start as NaN everywhere
    for path, flags in PATHS.items():
        got = to_f64(run_attn(gb, flags))
        assert _max_err(got, ref) <= 1e-2, path


def test_request_order_shuffle_is_bitwise_stable():
    b = config_batch(1, num_reqs=5, num_heads=4)
    gb = upload(b)
    base = to_f64(run_attn(gb, 0))
    perm = np.random.default_rng(3).permutation(b.num_reqs)
    b2 = config_batch(1, num_reqs=5, num_heads=4)
    q_all = {r: b.request_q(r) for r in range(b.num_reqs)}
    kv_all = {r: b.request_kv(r) for r in range(b.num_reqs)}
    for attr in ("hist_lens", "new_lens", "evict_lens"):
        setattr(b2, attr, getattr(b, attr)[perm])
    b2.block_tables = b.block_tables[perm]
    to32 = (lambda a: a.astype(np.float32))
    b2.q_fn = lambda r: to32(q_all[int(perm[r])])
    b2.k_fn = lambda r: to32(kv_all[int(perm[r])][0])
    b2.v_fn = lambda r: to32(kv_all[int(perm[r])][1])
    got = to_f64(run_attn(upload(b2), 0))
    for r2, r in enumerate(perm):
        a = got[int(b2.cu_q_lens[r2]):int(b2.cu_q_lens[r2 + 1])]
        c = base[int(b.cu_q_lens[r]):int(b.cu_q_lens[r + 1])]
        assert np.array_equal(a, c), r


def test_empty_requests_and_minimal_lengths():
    b = custom_batch([0, 40, 5, 0, 16], [1, 0, 0, 16, 0], num_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16",
                     seed=41)
    ref = oracle_output(b)
    gb = upload(b)
    for path, flags in PATHS.items():
        assert _max_err(to_f64(run_attn(gb, flags)), ref) <= 1e-2, path


def test_invalid_arguments_are_rejected_before_launch():
    b = custom_batch([10], [2], num_heads=4, num_kv_heads=4, head_dim=64, dtype="f16", seed=1)
    gb = upload(b)
    bad = pk.make_desc(num_heads=4, num_kv_heads=3, head_dim=64, num_blocks=b.num_blocks,
                       block_table_stride=b.block_table_stride, dtype=1, softmax_scale=0.125,
                       context_lens_host=b.context_lens, cu_q_lens_host=b.cu_q_lens)
    with pytest.raises(pk.PensieveError):
        pk.pensieve_attn_workspace_size(bad)
    import torch
    with pytest.raises(pk.PensieveError) as ei:
        pk.pensieve_attn_fwd(gb.desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                             gb.cu_q_lens, None, torch.empty_like(gb.q),
                             torch.empty(1, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 3


def test_host_positions_change_no_result():
    """The optional host copy of the query positions only orders the work: the outputs with the
    true copy, with none and with arbitrary values are bitwise equal, and match the oracle."""
    import torch
    from gpu_harness import poison_, to_host_storage
    b = config_batch(3, num_reqs=6, max_hist=2500)
    _say(f"host positions: {b.name} R={b.num_reqs} T={b.total_q}")
    gb = upload(b)
    junk = np.random.default_rng(5).integers(-2**31, 2**31 - 1, size=b.total_q, dtype=np.int64).astype(np.int32)
    outs = []
    for qp in (b.q_pos, None, junk, np.zeros(b.total_q, np.int32)):
        desc = pk.make_desc(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                            num_blocks=b.num_blocks, block_table_stride=b.block_table_stride, dtype=2,
                            softmax_scale=b.softmax_scale, context_lens_host=b.context_lens,
                            cu_q_lens_host=b.cu_q_lens, q_pos_host=qp)
        ws = torch.empty(max(pk.pensieve_attn_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        o = torch.empty_like(gb.q)
        poison_(o, b.dtype)
        pk.pensieve_attn_fwd(desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens, gb.cu_q_lens,
                             gb.q_pos, o, ws)
        torch.cuda.synchronize()
        outs.append(o)
    bits = [to_host_storage(o, b.dtype) for o in outs]
    for other in bits[1:]:
        assert np.array_equal(bits[0], other)
    err = _max_err(to_f64(outs[0]), oracle_output(b))
    assert err <= TOL[b.dtype], err
