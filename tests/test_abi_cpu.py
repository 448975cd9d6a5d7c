"""The C ABI without a GPU: the library loads, exports every declared entry point,
rejects bad arguments on the host, and plans every (row, head) exactly once."""

import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_token_amd as pk
from paged_kv_token_amd import binding
from workloads import config_batch, custom_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from paged_kv_token_amd.build import build
        build(verbose=False)
    return pk.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pensieve.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pensieve_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding.EXPORTED)


def test_version_string(lib):
    assert "gfx950" in pk.pensieve_version()


def desc_for(b, **over):
    kw = dict(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim, num_blocks=b.num_blocks,
              block_table_stride=b.block_table_stride, dtype={"f32": 0, "f16": 1, "bf16": 2}[b.dtype],
              softmax_scale=b.softmax_scale, context_lens_host=b.context_lens, cu_q_lens_host=b.cu_q_lens)
    kw.update(over)
    return pk.make_desc(**kw)


@pytest.mark.parametrize("over,status", [
    (dict(num_kv_heads=3), 1), (dict(head_dim=96), 2), (dict(block_size=32), 2), (dict(dtype=7), 2),
    (dict(num_blocks=0), 1), (dict(block_table_stride=1), 1), (dict(softmax_scale=0.0), 1),
    (dict(softmax_scale=-1.0), 1), (dict(flags=8), 1),
    (dict(context_lens_host=[4, 5, 6], cu_q_lens_host=[0, 5, 6, 7]), 1),   # q > L
    (dict(context_lens_host=[4, 5, 6], cu_q_lens_host=[1, 2, 3, 4]), 1),   # cu[0] != 0
    (dict(context_lens_host=[4, 5, 6], cu_q_lens_host=[0, 2, 1, 2]), 1),   # decreasing
    (dict(context_lens_host=[4, -1, 6], cu_q_lens_host=[0, 1, 1, 2]), 1),
    (dict(kv_dtype=0), 2),                                   # f32 pools under f16 queries
    (dict(kv_dtype=9), 2),
    (dict(kv_dtype=3, k_scale=0.0), 1), (dict(kv_dtype=3, v_scale=float("inf")), 1),
    (dict(kv_dtype=3, k_scale=float("nan")), 1), (dict(kv_dtype=3, v_scale=-1.0), 1),
    (dict(dtype=0, kv_dtype=3), 2),                          # E4M3 pools need f16 / bf16 queries
])
def test_bad_descriptors_are_rejected(lib, over, status):
    b = custom_batch([10, 20, 30], [1, 2, 3], num_heads=4, num_kv_heads=2, head_dim=64, dtype="f16", seed=1)
    with pytest.raises(pk.PensieveError) as ei:
        pk.pensieve_attn_workspace_size(desc_for(b, **over))
    assert ei.value.status == status
    assert lib.pensieve_last_error().decode()


def test_null_pointers_rejected_without_gpu(lib):
    b = custom_batch([10], [2], num_heads=4, num_kv_heads=4, head_dim=64, dtype="f16", seed=1)
    d = desc_for(b)
    st = lib.pensieve_attn_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None)
    assert st == 1
    st = lib.pensieve_kv_append(None, None, None, None, None, 5, 4, 64, 16, 10, 1, None)
    assert st == 1
    st = lib.pensieve_kv_append(None, None, None, None, None, 0, 4, 64, 16, 10, 1, None)   # nothing to do
    assert st == 0
    st = lib.pensieve_attn_split_merge(None, None, None, 4, 2, 64, 300, 1, None, None)     # P too large
    assert st == 1
    assert lib.pensieve_attn_workspace_size(None, 0, None) == 1


def _coverage(b, plan, P=None):
    """Every (row, query head) is covered once in each of its request's partitions 0..P_r-1
    (P_r fixed to P when given, else the request's own count, the same on all its items)."""
    parts = {}
    for row in plan[plan[:, 4] > 0]:
        parts.setdefault(int(row[1]), set()).add(int(row[6]))
    Pmax = max([P or 1] + [max(v) for v in parts.values()])
    seen = np.zeros((b.total_q, b.num_heads, Pmax), dtype=np.int32)
    want = np.zeros_like(seen)
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        counts = parts.get(r, {P or 1})
        assert len(counts) == 1, f"request {r} has items with different partition counts"
        pr = counts.pop()
        assert P is None or pr == P
        want[int(b.cu_q_lens[r]):int(b.cu_q_lens[r + 1]), :, :pr] = 1
    for kern, r, g, q0, qc, part, nparts, cost, h0, hc in plan:
        assert 0 <= part < nparts and (P is None or nparts == P)
        lo = int(b.cu_q_lens[r]) + q0
        assert q0 + qc <= int(b.q_lens[r])
        for h in range(g * G + h0, g * G + h0 + hc):
            seen[lo:lo + qc, h, part] += 1
    return seen, want


def _cost_class(cost) -> int:
    """Class of a planned item's cost: its octave in 64-unit steps, three octaves per class."""
    return (int(max(1, int(cost) // 64)).bit_length() - 1) // 3


@pytest.mark.parametrize("index", [0, 1, 2, 3, 4])
def test_plan_covers_each_row_head_once(lib, index):
    b = config_batch(index)
    plan = pk.pensieve_debug_plan(desc_for(b))
    seen, want = _coverage(b, plan)
    assert np.array_equal(seen, want)
    mat = plan[plan[:, 0] == 1]
    if len(mat) >= 16:
        # matrix-core items: interleaved over 8 XCD bins (slot % 8); each bin runs its items by cost
        # class (three octaves of the cost), longest first, and keeps all items of one (request, KV
        # head, partition) on one XCD
        assert len(mat) % 8 == 0
        owner = {}
        for x in range(8):
            live = [row for row in mat[x::8] if row[4] > 0]
            classes = [_cost_class(row[7]) for row in live]
            assert classes == sorted(classes, reverse=True)
            for row in live:
                assert owner.setdefault((row[1], row[2], row[5]), x) == x
        assert np.all(mat[mat[:, 4] == 0][:, 7] == 0)    # fillers carry no work


@pytest.mark.parametrize("P", [1, 7, 32])
def test_split_plan_covers_each_partition(lib, P):
    b = config_batch(4, num_heads=4, max_hist=3000)
    plan = pk.pensieve_debug_plan(desc_for(b), P)
    seen, want = _coverage(b, plan, P)
    assert np.array_equal(seen, want) and want.all()


def _adaptive_parts(b):
    plan = pk.pensieve_debug_plan(desc_for(b))
    out = {}
    for row in plan[plan[:, 4] > 0]:
        out[int(row[1])] = int(row[6])
    return out


@pytest.mark.parametrize("index", [0, 1, 2, 3])
def test_adaptive_split_leaves_ordinary_batches_whole(lib, index):
    assert set(_adaptive_parts(config_batch(index)).values()) == {1}


def test_adaptive_split_cuts_only_the_long_requests(lib):
    """Long-context batch: among the requests of one kernel the longest histories get the most
    partitions, at least 64 blocks each; a batch of short requests beside one long one splits
    only the long one."""
    b = config_batch(4)
    parts = _adaptive_parts(b)
    nblk = -(-b.context_lens // 16)
    assert all(parts[r] > 1 for r in range(b.num_reqs))
    decode = [r for r in np.argsort(nblk, kind="stable") if b.q_lens[r] == 1]   # the vector kernel's
    assert [parts[int(r)] for r in decode] == sorted(parts[int(r)] for r in decode)
    assert all(nblk[r] / parts[r] >= 4 for r in parts)
    mixed = custom_batch([20000] + [300] * 12, [1] * 13, num_heads=8, num_kv_heads=8, head_dim=128, dtype="f16",
                         seed=9)
    mp = _adaptive_parts(mixed)
    assert mp[0] > 1 and all(mp[r] == 1 for r in range(1, 13))


def test_adaptive_split_workspace_holds_the_partials(lib):
    b = config_batch(4)
    d = desc_for(b)
    parts = _adaptive_parts(b)
    n_items = len(pk.pensieve_debug_plan(d))
    rows = sum(int(b.q_lens[r]) for r, p in parts.items() if p > 1)
    partials = rows * b.num_heads * max(parts.values())
    ws = pk.pensieve_attn_workspace_size(d)
    assert ws % 256 == 0
    assert ws >= 32 * n_items + partials * (b.head_dim + 2) * 4
    assert ws < 32 * n_items + partials * (b.head_dim + 2) * 4 + 6 * 256 + 4 * (b.num_reqs + 2 * rows)


def test_routing_rules(lib):
    b = config_batch(1, num_reqs=4, num_heads=8)
    plan = pk.pensieve_debug_plan(desc_for(b))
    for kern, r, g, q0, qc, *_ in plan:
        q = int(b.q_lens[r])
        assert kern == (1 if q > 8 else 0)
    plan_v = pk.pensieve_debug_plan(desc_for(b, flags=pk.PENSIEVE_FLAG_VECTOR_ONLY))
    assert np.all(plan_v[:, 0] == 0) and np.all(plan_v[:, 4] * plan_v[:, 9] <= 8)
    f32 = custom_batch([100], [50], num_heads=4, num_kv_heads=4, head_dim=64, dtype="f32", seed=2)
    assert np.all(pk.pensieve_debug_plan(desc_for(f32))[:, 0] == 0)
    # Head groups of 4 or more go to the matrix cores even for one decode token; pairs stay on
    # the vector kernel up to 8 query vectors.
    for hq, hkv, want in ((16, 2, 1), (8, 2, 1), (4, 2, 0), (4, 4, 0)):
        dec = custom_batch([300, 40, 0], [1, 1, 1], num_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16",
                           seed=3)
        live = pk.pensieve_debug_plan(desc_for(dec))
        live = live[live[:, 4] > 0]
        assert np.all(live[:, 0] == want), (hq, hkv)


def test_workspace_size_matches_plan(lib):
    b = config_batch(3)
    d = desc_for(b)
    n = len(pk.pensieve_debug_plan(d))
    ws = pk.pensieve_attn_workspace_size(d)
    assert ws >= 32 * n and ws % 256 == 0 and ws < 32 * n + 256


def _swap_args(n, src, dst, **over):
    a = dict(k_pool=ctypes.c_void_p(0x1000), v_pool=ctypes.c_void_p(0x2000), num_blocks=64,
             k_host=ctypes.c_void_p(0x3000), v_host=ctypes.c_void_p(0x4000), num_host_blocks=32,
             n=n, num_kv_heads=4, head_dim=64, dtype=1)
    a.update(over)
    s = (ctypes.c_int32 * max(1, n))(*src)
    d = (ctypes.c_int32 * max(1, n))(*dst)
    return a, s, d


@pytest.mark.parametrize("direction", ["out", "in"])
@pytest.mark.parametrize("case,status", [
    ("src_out_of_range", 1), ("dst_out_of_range", 1), ("negative_id", 1), ("duplicate_destination", 1),
    ("bad_head_dim", 2), ("bad_dtype", 2), ("null_pool", 1), ("null_list", 1), ("negative_n", 1),
])
def test_kv_swap_rejects_bad_arguments_before_any_launch(lib, direction, case, status):
    """Block ids are checked against their own pool on the host (device pools have 64 blocks, the
    host tier 32), so a bad list never reaches a kernel; the fake pool pointers are never touched."""
    out = direction == "out"
    n_src, n_dst = (64, 32) if out else (32, 64)
    src, dst = [0, 5, 7], [1, 2, 3]
    over = {}
    if case == "src_out_of_range":
        src = [0, n_src, 1]
    elif case == "dst_out_of_range":
        dst = [0, n_dst, 1]
    elif case == "negative_id":
        src = [0, -1, 2]
    elif case == "duplicate_destination":
        dst = [4, 9, 4]
    elif case == "bad_head_dim":
        over["head_dim"] = 96
    elif case == "bad_dtype":
        over["dtype"] = 7
    elif case == "null_pool":
        over["k_pool"] = None
    a, s, d = _swap_args(3, src, dst, **over)
    if case == "null_list":
        s = None
    if case == "negative_n":
        a["n"] = -1
    fn = lib.pensieve_kv_swap_out if out else lib.pensieve_kv_swap_in
    st = fn(a["k_pool"], a["v_pool"], a["num_blocks"], a["k_host"], a["v_host"], a["num_host_blocks"], s, d, a["n"],
            a["num_kv_heads"], a["head_dim"], a["dtype"], None)
    assert st == status
    assert lib.pensieve_last_error().decode()


def test_kv_swap_of_nothing_is_a_no_op(lib):
    assert lib.pensieve_kv_swap_in(None, None, 1, None, None, 1, None, None, 0, 4, 64, 1, None) == 0


def test_fp8_descriptor_is_accepted(lib):
    b = custom_batch([10, 20, 30], [1, 2, 3], num_heads=4, num_kv_heads=2, head_dim=64, dtype="bf16", seed=1)
    assert pk.pensieve_attn_workspace_size(desc_for(b, kv_dtype=3, k_scale=0.5, v_scale=2.0)) > 0


@pytest.mark.parametrize("args,status", [
    (dict(src=0), 2), (dict(src=3), 2), (dict(ks=0.0), 1), (dict(vs=float("nan")), 1), (dict(d=80), 2),
    (dict(n=-1), 1), (dict(n=4), 1),                         # NULL pointers with work to do
])
def test_fp8_append_rejects_bad_arguments(lib, args, status):
    a = dict(src=1, ks=1.0, vs=1.0, d=64, n=0)
    a.update(args)
    st = lib.pensieve_kv_append_fp8(None, None, None, None, None, a["n"], 2, a["d"], 16, 10, a["src"], a["ks"],
                                    a["vs"], None)
    assert st == status


def test_no_split_flag_keeps_every_request_whole(lib):
    b = custom_batch([20000, 300, 300], [1, 1, 40], num_heads=8, num_kv_heads=8, head_dim=128, dtype="f16", seed=5)
    split = pk.pensieve_debug_plan(desc_for(b))
    whole = pk.pensieve_debug_plan(desc_for(b, flags=pk.PENSIEVE_FLAG_NO_SPLIT))
    assert split[split[:, 4] > 0][:, 6].max() > 1
    assert np.all(whole[:, 6] == 1)
    assert (pk.pensieve_attn_workspace_size(desc_for(b, flags=pk.PENSIEVE_FLAG_NO_SPLIT))
            < pk.pensieve_attn_workspace_size(desc_for(b)))


@pytest.mark.parametrize("seed", range(12))
def test_plan_covers_random_batches(lib, seed):
    """Random ragged batches (empty requests, first turns, long contexts, every head grouping,
    both kernels, head groups that do and do not divide 32, adaptive and fixed splits): every (row,
    head, partition) is planned once."""
    rng = np.random.default_rng(500 + seed)
    R = int(rng.integers(1, 24))
    hist = rng.integers(0, 20000 if seed % 3 == 0 else 2000, size=R)
    new = np.where(rng.random(R) < 0.2, 0, rng.integers(1, 300, size=R))
    hist = np.where((new == 0) & (hist == 0), 1, hist)
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 12]))
    b = custom_batch(hist, new, num_heads=hkv * G, num_kv_heads=hkv, head_dim=int(rng.choice([64, 128])),
                     dtype=str(rng.choice(["f16", "bf16", "f32"])), seed=seed)
    for flags in (0, pk.PENSIEVE_FLAG_VECTOR_ONLY, pk.PENSIEVE_FLAG_NO_SPLIT):
        seen, want = _coverage(b, pk.pensieve_debug_plan(desc_for(b, flags=flags)))
        assert np.array_equal(seen, want), flags
    for P in (3, 32):
        seen, want = _coverage(b, pk.pensieve_debug_plan(desc_for(b), P), P)
        assert np.array_equal(seen, want), P


def _bin_spread(b, plan, pos):
    """max / mean over the 8 XCD bins (slot % 8) of the 64-key tiles the matrix-core items' rows
    can see, from the positions themselves."""
    mat = plan[plan[:, 0] == 1]
    load = np.zeros(8)
    for i, row in enumerate(mat):
        r, q0, qc = int(row[1]), int(row[3]), int(row[4])
        if qc:
            load[i % 8] += -(-(int(pos[int(b.cu_q_lens[r]) + q0 + qc - 1]) + 1) // 64)
    return load.max() / load.mean()


def test_host_positions_balance_the_xcd_bins(lib):
    """GQA recompute workload: with the host copy of the query positions every matrix-core item is
    costed by the keys its rows can see, and the eight XCD bins carry equal causal work within 1 %
    (costed by whole contexts, the recomputed leading rows make them about 6 % apart)."""
    b = config_batch(3)
    with_pos = _bin_spread(b, pk.pensieve_debug_plan(desc_for(b, q_pos_host=b.q_pos)), b.q_pos)
    without = _bin_spread(b, pk.pensieve_debug_plan(desc_for(b)), b.q_pos)
    assert with_pos < 1.01 and with_pos < without


def test_host_positions_never_change_the_work_covered(lib):
    """Host positions only order the work: true, zero or arbitrary values plan every (row, head,
    partition) exactly once, and each XCD bin still runs its longest cost classes first."""
    b = config_batch(3, num_reqs=12, max_hist=3000)
    rng = np.random.default_rng(3)
    junk = rng.integers(-2**31, 2**31 - 1, size=b.total_q, dtype=np.int64).astype(np.int32)
    for qp in (b.q_pos, np.zeros(b.total_q, np.int32), junk):
        plan = pk.pensieve_debug_plan(desc_for(b, q_pos_host=qp))
        seen, want = _coverage(b, plan)
        assert np.array_equal(seen, want)
        mat = plan[plan[:, 0] == 1]
        for x in range(8):
            classes = [_cost_class(row[7]) for row in mat[x::8] if row[4] > 0]
            assert classes == sorted(classes, reverse=True)
    with pytest.raises(ValueError):
        desc_for(b, q_pos_host=b.q_pos[:-1])


def test_vector_requests_beside_matrix_items_split_finer(lib):
    """Long-context workload: the 512-row prefill request alone fills fewer than 512 matrix-core
    items, so the three long decode requests (vector kernel, run beside it) are cut against half
    the usual share, about twice as many partitions as the prefill request's rule gives."""
    b = config_batch(4)
    plan = pk.pensieve_debug_plan(desc_for(b))
    parts = {int(row[1]): int(row[6]) for row in plan if row[4] > 0}
    kern = {int(row[1]): int(row[0]) for row in plan if row[4] > 0}
    nblk = -(-b.context_lens.astype(np.int64) // 16)
    items = np.where(b.q_lens > 1, -(-b.q_lens // 128), 1)
    share = max(64, int((items * b.num_kv_heads * (nblk + 1)).sum()) // 512)
    for r in range(b.num_reqs):
        usual = -(-(int(nblk[r]) + 1) // share)
        if kern[r] == 1:
            assert parts[r] == usual
        else:
            assert parts[r] >= 2 * usual - 1 and parts[r] > usual


def test_xcd_bins_keep_a_requests_items_together_inside_a_cost_class(lib):
    """Inside one XCD bin and one cost class, the items of one (request, KV head, partition) form a
    single contiguous run, so they run close together and share that K/V in the XCD's L2."""
    b = config_batch(3)
    plan = pk.pensieve_debug_plan(desc_for(b, q_pos_host=b.q_pos))
    mat = plan[plan[:, 0] == 1]
    for x in range(8):
        live = [row for row in mat[x::8] if row[4] > 0]
        seen, prev = set(), None
        for row in live:
            key = (_cost_class(row[7]), int(row[1]), int(row[2]), int(row[5]))
            if key != prev:
                assert key not in seen, f"bin {x}: items of {key} split into two runs"
                seen.add(key)
            prev = key


def _max_vectors(b, plan):
    live = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
    G = b.num_heads // b.num_kv_heads
    return int((live[:, 4] * G).max()) if len(live) else 0


def test_eight_wave_items_only_where_four_wave_items_leave_the_gpu_short(lib):
    """Matrix-core items of up to 256 query vectors (eight-wave workgroups) appear only in calls
    whose 128-vector items would number fewer than 512 and that hold a request of more than 128
    query vectors per KV head, with 2-byte pools; every other call keeps 128-vector items.  Rows
    and partitions stay covered exactly once either way."""
    lc = config_batch(4)                      # 512-row prefill: 320 four-wave items
    plan = pk.pensieve_debug_plan(desc_for(lc))
    assert _max_vectors(lc, plan) == 256
    seen, want = _coverage(lc, plan)
    assert np.array_equal(seen, want)
    mat = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
    assert len(mat) == 160                    # 2 row blocks x 40 heads x 2 partitions
    # The explicit split pair: one partition leaves 160 four-wave items (eight-wave), 32 partitions
    # 5120 (four-wave).
    for P, widest in ((1, 256), (32, 128)):
        plan_p = pk.pensieve_debug_plan(desc_for(lc), P)
        assert _max_vectors(lc, plan_p) == widest
        seen, want = _coverage(lc, plan_p, P)
        assert np.array_equal(seen, want)
    # The GQA recompute workload fills the GPU with four-wave items; the 13B batch has no request
    # above 128 query vectors; E4M3 pools have an eight-wave kernel at head_dim 128 only.
    for b, over in ((config_batch(3), {}), (config_batch(1), {})):
        assert 0 < _max_vectors(b, pk.pensieve_debug_plan(desc_for(b, **over))) <= 128
    f8 = dict(kv_dtype=3, k_scale=1.0, v_scale=1.0)
    assert _max_vectors(lc, pk.pensieve_debug_plan(desc_for(lc, **f8))) == 256
    lc64 = custom_batch([4000, 3000], [300, 1], num_heads=8, num_kv_heads=8, head_dim=64, dtype="bf16", seed=6)
    assert _max_vectors(lc64, pk.pensieve_debug_plan(desc_for(lc64))) == 256
    assert 0 < _max_vectors(lc64, pk.pensieve_debug_plan(desc_for(lc64, **f8))) <= 128
    # Groups of G query heads: rows of 256 / G tokens, the short request of the call too.
    for hq, hkv in ((4, 4), (8, 4), (16, 4), (32, 4), (32, 1)):
        b = custom_batch([3000, 700, 900], [300, 20, 1], num_heads=hq, num_kv_heads=hkv, head_dim=128,
                         dtype="f16", seed=5)
        plan = pk.pensieve_debug_plan(desc_for(b))
        G = hq // hkv
        live = plan[(plan[:, 0] == 1) & (plan[:, 4] > 0)]
        assert live[:, 4].max() == min(256 // G, 300)
        seen, want = _coverage(b, plan)
        assert np.array_equal(seen, want)
