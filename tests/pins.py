"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes an implementation namespace (the real ``oracle`` module,
or a copy with a planted mistake) and raises AssertionError when the
implementation disagrees with:

* a hand-derived worked example (tests/golden/worked_example.json);
* a library routine (torch's scaled_dot_product_attention in float64 over
  contiguous K/V, scipy's logsumexp for split partials);
* a pure-Python brute force on tiny inputs;
* closed forms (zero query -> mean of visible values; one-hot attention);
* invariants (block placement, history split, GQA replication, split/merge,
  NaN in stale slots).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle_helpers import oracle_output, oracle_pools, oracle_split, poison_fill
from workloads import custom_batch, storage_dtype

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), what
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def _sym(x: str) -> float:
    x = x.strip()
    if x.startswith("ln"):
        return math.log(float(x[2:]))
    return float(x)


def _frac(x: str) -> float:
    return float(Fraction(x))


# ---------------------------------------------------------------------------
def pin_worked_example(impl):
    spec = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    B, d, hq, hkv = spec["block_size"], spec["head_dim"], spec["num_heads"], spec["num_kv_heads"]
    nb = spec["num_blocks"]
    k_pool = np.full((nb, hkv, B, d), np.nan, dtype=np.float32)
    v_pool = np.full((nb, hkv, B, d), np.nan, dtype=np.float32)
    reqs = spec["requests"]
    stride = max(len(r["block_table"]) for r in reqs)
    bt = np.zeros((len(reqs), stride), dtype=np.int32)
    qs, expected, ctx, cu, qpos = [], [], [], [0], []
    for i, r in enumerate(reqs):
        bt[i, :len(r["block_table"])] = r["block_table"]
        L = r["context_len"]
        slots = np.array([r["block_table"][t // B] * B + t % B for t in range(L)], dtype=np.int32)
        k = np.array(r["k"], dtype=np.float32).reshape(L, hkv, d)
        v = np.array(r["v"], dtype=np.float32).reshape(L, hkv, d)
        impl.append_kv(k_pool, v_pool, k, v, slots, B)
        n = len(r["positions"])
        q = np.zeros((n, hq, d))
        exp_o = np.zeros((n, hq, d))
        for h in range(hq):
            q[:, h, :] = [[_sym(x) for x in row] for row in r[f"q_head{h}"]]
            exp_o[:, h, :] = [[_frac(x) for x in row] for row in r[f"expected_head{h}"]]
        qs.append(q); expected.append(exp_o); ctx.append(L); cu.append(cu[-1] + n)
        qpos.extend(r["positions"])
    q = np.concatenate(qs)
    out = impl.paged_attention(q, k_pool, v_pool, bt, np.array(ctx), np.array(cu), np.array(qpos),
                               spec["softmax_scale"], "f32")
    _close(out, np.concatenate(expected), 1e-12, "worked example")


# ---------------------------------------------------------------------------
def _sharp_batch(seed, hist, new, ev, hq, hkv, d, dtype="f32", sharp=4.0):
    b = custom_batch(hist, new, ev, num_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed)
    rng_q = np.random.default_rng(seed + 1)
    rng_kv = np.random.default_rng(seed + 2)
    qs = [rng_q.standard_normal((int(b.q_lens[r]), hq, d)).astype(np.float32) * sharp for r in range(b.num_reqs)]
    ks = [rng_kv.standard_normal((int(b.context_lens[r]), hkv, d)).astype(np.float32) * sharp for r in range(b.num_reqs)]
    vs = [rng_kv.standard_normal((int(b.context_lens[r]), hkv, d)).astype(np.float32) for r in range(b.num_reqs)]
    b.q_fn = lambda r: qs[r]
    b.k_fn = lambda r: ks[r]
    b.v_fn = lambda r: vs[r]
    return b


def pin_library_sdpa(impl):
    """Oracle (paged) == torch SDPA (float64, contiguous K/V, explicit boolean mask)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(7)
    for case in range(18):
        d = [1, 2, 8, 64][case % 4]
        group = [1, 2, 4][case % 3]
        hkv = 1 + case % 2
        hq = hkv * group
        R = 1 + case % 3
        L = rng.integers(1, 49, size=R)
        q_lens = np.array([rng.integers(1, l + 1) for l in L])
        b = _sharp_batch(100 + case, L - q_lens, q_lens, None, hq, hkv, d)
        out = oracle_output(b, impl)
        for r in range(b.num_reqs):
            lo, hi = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
            q = torch.from_numpy(b.request_q(r).astype(np.float64)).permute(1, 0, 2)[None]
            k, v = b.request_kv(r)
            kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
            vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
            pos = torch.from_numpy(b.query_positions(r))
            mask = torch.arange(int(b.context_lens[r]))[None, :] <= pos[:, None]
            ref = F.scaled_dot_product_attention(q, kt, vt, attn_mask=mask, scale=b.softmax_scale)
            _close(out[lo:hi], ref[0].permute(1, 0, 2).numpy(), 1e-12, f"sdpa case {case} req {r}")


def pin_python_loops(impl):
    """Oracle == scalar pure-Python attention (math.exp, explicit loops) on tiny inputs."""
    for case in range(6):
        d = 1 + case % 3
        b = _sharp_batch(300 + case, [3 + case, 0, 5], [2, 4, 1], [0, 0, 0] if case % 2 else None,
                         2, 1 + case % 2, d)
        out = oracle_output(b, impl)
        for r in range(b.num_reqs):
            q = b.request_q(r).astype(float); k, v = b.request_kv(r)
            group = b.num_heads // b.num_kv_heads
            for i, p in enumerate(b.query_positions(r)):
                for h in range(b.num_heads):
                    g = h // group
                    s = [sum(q[i, h, c] * float(k[t, g, c]) for c in range(d)) * b.softmax_scale
                         for t in range(int(p) + 1)]
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = sum(w)
                    for c in range(d):
                        ref = sum(w[t] * float(v[t, g, c]) for t in range(len(w))) / tot
                        got = out[int(b.cu_q_lens[r]) + i, h, c]
                        assert abs(got - ref) <= 1e-12, (case, r, i, h, c, got, ref)


# ---------------------------------------------------------------------------
def pin_shuffle_invariance(impl):
    """Re-drawing the physical placement leaves the output bit-identical."""
    base = _sharp_batch(11, [40, 17, 0, 64], [3, 1, 9, 16], None, 4, 2, 8)
    ref = oracle_output(base, impl)
    for seed in (5, 6, 7):
        other = _sharp_batch(11, [40, 17, 0, 64], [3, 1, 9, 16], None, 4, 2, 8)
        rng = np.random.default_rng(seed)
        nb = other.num_blocks * 2
        perm = rng.permutation(nb).astype(np.int32)
        need = [other.num_logical_blocks(r) for r in range(other.num_reqs)]
        bt = np.full_like(other.block_tables, 0)
        off = 0
        for r, n in enumerate(need):
            bt[r, :n] = perm[off:off + n]; off += n
        other.block_tables = bt
        other.num_blocks = nb
        out = oracle_output(other, impl)
        assert np.array_equal(out, ref), f"placement seed {seed} changed the output"


def pin_aliased_blocks(impl):
    """Two requests mapping the same physical blocks for a shared prefix (copy-on-write sharing)."""
    b = _sharp_batch(21, [32, 32], [5, 2], None, 2, 2, 8)
    ks, vs = {}, {}
    rk = np.random.default_rng(99)
    shared_k = rk.standard_normal((32, 2, 8)).astype(np.float32) * 4
    shared_v = rk.standard_normal((32, 2, 8)).astype(np.float32)
    orig_k, orig_v = b.k_fn, b.v_fn
    for r in range(2):
        k = np.array(orig_k(r)); v = np.array(orig_v(r))
        k[:32] = shared_k; v[:32] = shared_v
        ks[r], vs[r] = k, v
    b.k_fn = lambda r: ks[r]
    b.v_fn = lambda r: vs[r]
    ref = oracle_output(b, impl)
    aliased = _sharp_batch(21, [32, 32], [5, 2], None, 2, 2, 8)
    aliased.k_fn, aliased.v_fn = b.k_fn, b.v_fn
    bt = aliased.block_tables.copy()
    bt[1, :2] = bt[0, :2]            # request 1's prefix blocks are request 0's
    aliased.block_tables = bt
    out = oracle_output(aliased, impl)
    assert np.array_equal(out, ref)


def pin_history_split(impl):
    """Cached history + n new rows == the same rows of one-shot causal attention over [0, L)."""
    for seed, (H, n, d, hq, hkv) in enumerate([(37, 5, 8, 4, 2), (80, 1, 64, 2, 2), (16, 16, 2, 8, 1)]):
        full = _sharp_batch(40 + seed, [0], [H + n], None, hq, hkv, d)
        split = _sharp_batch(40 + seed, [H], [n], None, hq, hkv, d)
        qf = full.q_fn(0)
        split.q_fn = lambda r, qf=qf: qf[H:]
        split.k_fn, split.v_fn = full.k_fn, full.v_fn
        _close(oracle_output(split, impl), oracle_output(full, impl)[H:], 1e-12, f"history split {seed}")


def pin_recompute_rows(impl):
    """Rows [0,E) + [H,H+n) with explicit positions == those rows of one-shot attention."""
    H, E, n = 70, 32, 6
    full = _sharp_batch(61, [0], [H + n], None, 4, 1, 8)
    rec = _sharp_batch(61, [H], [n], [E], 4, 1, 8)
    qf = full.q_fn(0)
    rows = np.r_[0:E, H:H + n]
    rec.q_fn = lambda r: qf[rows]
    rec.k_fn, rec.v_fn = full.k_fn, full.v_fn
    _close(oracle_output(rec, impl), oracle_output(full, impl)[rows], 1e-12, "recompute rows")


def pin_default_positions(impl):
    """Passing the default positions explicitly changes nothing."""
    b = _sharp_batch(71, [9, 0, 30], [4, 7, 1], None, 2, 2, 8)
    k_pool, v_pool = oracle_pools(b, impl)
    args = (b.q_all(), k_pool, v_pool, b.block_tables, b.context_lens, b.cu_q_lens)
    a = impl.paged_attention(*args, None, b.softmax_scale, b.dtype)
    c = impl.paged_attention(*args, b.q_pos, b.softmax_scale, b.dtype)
    assert np.array_equal(a, c)


# ---------------------------------------------------------------------------
def pin_zero_query_closed_form(impl):
    """Q = 0: every visible key weighs 1, so O[i] = mean_{t<=p} V[t]; V[t] = (-1)^t A gives A/(p+1) or 0."""
    A = 256.0
    for dtype in ("f32", "f16", "bf16"):
        b = custom_batch([50, 0, 17, 96], [3, 20, 1, 5], [0, 0, 0, 32], num_heads=4, num_kv_heads=2,
                         head_dim=8, dtype=dtype, seed=5)
        b.q_fn = lambda r, b=b: np.zeros((int(b.q_lens[r]), 4, 8), np.float32)
        b.v_fn = lambda r, b=b: (A * (-1.0) ** np.arange(int(b.context_lens[r])))[:, None, None] * np.ones((1, 2, 8), np.float32)
        out = oracle_output(b, impl)
        exp = np.zeros_like(out)
        for r in range(b.num_reqs):
            lo = int(b.cu_q_lens[r])
            for i, p in enumerate(b.query_positions(r)):
                exp[lo + i] = A / (p + 1) if p % 2 == 0 else 0.0
        _close(out, exp, 1e-9, f"zero query {dtype}")


def pin_one_hot(impl):
    """Q[i] = c * K[p_i] with orthonormal K: each row returns V at its own position."""
    d = 64
    b = custom_batch([20, 33], [4, 2], [0, 16], num_heads=2, num_kv_heads=1, head_dim=d, dtype="f32", seed=8)
    eye = np.eye(d, dtype=np.float32)
    ks = {r: eye[np.arange(int(b.context_lens[r])) % d][:, None, :] for r in range(b.num_reqs)}
    b.k_fn = lambda r: ks[r]
    c = 30.0 / b.softmax_scale
    b.q_fn = lambda r: np.repeat((c * eye[b.query_positions(r) % d])[:, None, :], 2, axis=1)
    out = oracle_output(b, impl)
    for r in range(b.num_reqs):
        _, v = b.request_kv(r)
        lo = int(b.cu_q_lens[r])
        for i, p in enumerate(b.query_positions(r)):
            for h in range(2):
                _close(out[lo + i, h], v[p, 0], 1e-9 * (p + 1), f"one-hot r{r} i{i}")


def pin_gqa_replication(impl):
    """GQA (Hq=8, Hkv=2) == MHA with each KV head replicated Hq/Hkv times."""
    g = _sharp_batch(81, [25, 3], [6, 1], None, 8, 2, 8)
    m = _sharp_batch(81, [25, 3], [6, 1], None, 8, 8, 8)
    m.q_fn = g.q_fn
    m.k_fn = lambda r: np.repeat(g.k_fn(r), 4, axis=1)
    m.v_fn = lambda r: np.repeat(g.v_fn(r), 4, axis=1)
    assert np.array_equal(oracle_output(g, impl), oracle_output(m, impl))


# ---------------------------------------------------------------------------
def _merge_check(b, P, impl, tol=1e-12):
    pools = oracle_pools(b, impl)
    po, pm, pl = oracle_split(b, P, impl, pools=pools)
    _close(impl.split_merge(po, pm, pl), oracle_output(b, impl, pools=pools), tol, f"merge P={P}")
    return po, pm, pl


def pin_split_equals_unsplit(impl):
    b = _sharp_batch(91, [200, 33, 0, 700], [1, 40, 5, 1], None, 4, 2, 8)
    for P in (1, 3, 32):
        _merge_check(b, P, impl)


def pin_split_single_partition(impl):
    """P = 1: the one partial is the whole attention with l = sum of weights, O_p = O."""
    b = _sharp_batch(92, [50, 3], [4, 2], None, 2, 2, 8)
    po, pm, pl = oracle_split(b, 1, impl)
    _close(po[:, :, 0, :], oracle_output(b, impl), 1e-12, "P=1 partial")


def pin_split_partials_logsumexp(impl):
    """m + log(l) of each partition == logsumexp of its visible scaled scores (scipy)."""
    from scipy.special import logsumexp
    b = _sharp_batch(93, [70, 5], [9, 30], [32, 0], 2, 1, 8)
    P = 4
    po, pm, pl = oracle_split(b, P, impl)
    for r in range(b.num_reqs):
        lo = int(b.cu_q_lens[r]); L = int(b.context_lens[r])
        q = b.request_q(r).astype(np.float64); k, v = b.request_kv(r)
        nblk = -(-L // 16); per = -(-nblk // P)
        for i, p in enumerate(b.query_positions(r)):
            for h in range(b.num_heads):
                s = (k[:, 0, :].astype(np.float64) @ q[i, h]) * b.softmax_scale
                for part in range(P):
                    a, e = part * per * 16, min((part + 1) * per * 16, L)
                    keys = np.arange(a, max(a, e))
                    keys = keys[keys <= p]
                    m, l = pm[lo + i, h, part], pl[lo + i, h, part]
                    if len(keys) == 0:
                        assert m == -np.inf and l == 0 and np.all(po[lo + i, h, part] == 0), (r, i, h, part)
                    else:
                        assert abs((m + math.log(l)) - logsumexp(s[keys])) <= 1e-12
                        assert abs(m - s[keys].max()) <= 1e-12
                        w = np.exp(s[keys] - logsumexp(s[keys]))
                        _close(po[lo + i, h, part], w @ v[keys, 0, :].astype(np.float64), 1e-12, "O_p")


def pin_split_empty_and_masked(impl):
    """Fewer blocks than partitions, and recompute rows whose positions end before later partitions."""
    b = _sharp_batch(94, [48, 5], [3, 1], [16, 0], 2, 2, 8)
    po, pm, pl = _merge_check(b, 8, impl)
    assert np.any(pl == 0) and np.all(pm[pl == 0] == -np.inf)


# ---------------------------------------------------------------------------
def pin_nan_poison(impl):
    """NaN in unused blocks, stale tail slots and block-table tails leaves the output unchanged."""
    b = _sharp_batch(101, [21, 0, 40], [2, 3, 1], None, 2, 2, 8)
    b.num_blocks += 4
    ref = oracle_output(b, impl)
    k_pool, v_pool = oracle_pools(b, impl)       # untouched slots are NaN already
    bt = b.block_tables.copy()
    spare = b.num_blocks - 1                     # never written: all NaN
    for r in range(b.num_reqs):
        bt[r, b.num_logical_blocks(r):] = spare
    b2 = _sharp_batch(101, [21, 0, 40], [2, 3, 1], None, 2, 2, 8)
    b2.num_blocks = b.num_blocks
    b2.block_tables = np.concatenate([bt, np.full((b.num_reqs, 2), spare, np.int32)], axis=1)
    out = oracle_output(b2, impl, pools=(k_pool, v_pool))
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, ref)


def pin_append_slots(impl):
    """Append writes exactly the named slots of both pools and skips negative slots."""
    for dtype in ("f32", "f16", "bf16"):
        sd = storage_dtype(dtype)
        nb, hkv, B, d = 6, 3, 16, 8
        fill = poison_fill(dtype)
        k_pool = np.full((nb, hkv, B, d), fill, dtype=sd)
        v_pool = np.full((nb, hkv, B, d), fill, dtype=sd)
        rng = np.random.default_rng(3)
        slots = rng.permutation(nb * B)[:40].astype(np.int32)
        slots[[3, 17]] = -1
        k_new = rng.integers(0, 30000, size=(40, hkv, d)).astype(np.uint16).view(sd) if dtype != "f32" else \
            rng.standard_normal((40, hkv, d)).astype(np.float32)
        v_new = rng.integers(0, 30000, size=(40, hkv, d)).astype(np.uint16).view(sd) if dtype != "f32" else \
            rng.standard_normal((40, hkv, d)).astype(np.float32)
        impl.append_kv(k_pool, v_pool, k_new, v_new, slots, B)
        written = np.zeros((nb, B), dtype=bool)
        for t, s in enumerate(slots):
            if s < 0:
                continue
            blk, off = int(s) // B, int(s) % B
            written[blk, off] = True
            for g in range(hkv):
                for c in range(d):
                    assert k_pool[blk, g, off, c].tobytes() == k_new[t, g, c].tobytes()
                    assert v_pool[blk, g, off, c].tobytes() == v_new[t, g, c].tobytes()
        for blk in range(nb):
            for off in range(B):
                if not written[blk, off]:
                    assert np.all(np.isnan(k_pool[blk, :, off, :].astype(np.float32))) if dtype != "bf16" else \
                        np.all(k_pool[blk, :, off, :] == fill)
                    assert np.all(np.isnan(v_pool[blk, :, off, :].astype(np.float32))) if dtype != "bf16" else \
                        np.all(v_pool[blk, :, off, :] == fill)


ALL_PINS = [
    pin_worked_example, pin_library_sdpa, pin_python_loops, pin_shuffle_invariance, pin_aliased_blocks,
    pin_history_split, pin_recompute_rows, pin_default_positions, pin_zero_query_closed_form, pin_one_hot,
    pin_gqa_replication, pin_split_equals_unsplit, pin_split_single_partition, pin_split_partials_logsumexp,
    pin_split_empty_and_masked, pin_nan_poison, pin_append_slots,
]
