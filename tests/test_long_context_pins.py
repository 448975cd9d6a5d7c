"""CPU pins of the long-context structured cases (no GPU).

The GPU tests at the long-context workload's real lengths compare against closed forms
(tests/long_cases.py).  These pins show, on the CPU and from the definitions alone, that the
closed forms are right and that the gates can see the mistakes they are meant to catch:

* every expected value differs from what a slip of the causal boundary by one key, one block or
  one 64-key tile would give by at least 10x its tolerance (some output dim of every row);
* reading one wrong block (another block of the request, or the same logical block of another
  request or KV head) moves some dim by at least 10x the tolerance, for all but the pairs whose
  marks coincide (counted here: under 1 %);
* the one-hot expected value (V at the row's own position) agrees with the oracle's exact
  attention to 1e-4 on sampled rows of every request, far inside the 1e-2 gate, while any other
  V row differs from it by 2 in some dim (no two V rows of a request are equal).
"""

import numpy as np
import pytest

import oracle
from long_cases import (A, MAX_HIST, MAX_NEW, ONEHOT_TOL, onehot_batch, onehot_expected, signature_batch,
                        signature_expected, signature_tol, signature_v)
from workloads.batches import _to_storage

SLIPS = (-64, -16, -1, 1, 16, 64)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_signature_values_are_exact_in_storage(dtype):
    v = signature_v(4097, 2, 128, 3)
    back = oracle.to_f64(_to_storage(v, dtype), dtype)
    assert np.array_equal(back, v.astype(np.float64))
    assert set(np.unique(v).tolist()) == {-A, 0.0, A}


def test_structured_values_are_exact_in_e4m3_at_scale_one():
    """The GPU runs the structured cases on E4M3 pools too, with both scales 1: every V value of the
    signature pattern (0, +-A) and every K and V value of the one-hot pattern (+-1) is an E4M3 code,
    so the pools hold the same values as the 16-bit pools and the closed forms and margins carry
    over unchanged; the signature's random K may round, but its queries are zero."""
    v = signature_v(4097, 2, 128, 3).astype(np.float64)
    assert np.array_equal(oracle.e4m3_decode(oracle.e4m3_encode(v)), v)
    pm = np.array([-1.0, 1.0])
    assert np.array_equal(oracle.e4m3_decode(oracle.e4m3_encode(pm)), pm)
    assert A <= oracle.E4M3_MAX


@pytest.mark.parametrize("dtype,group,lengths", [("bf16", 1, "long"), ("bf16", 8, "long"), ("f16", 1, "long"),
                                                  ("bf16", 1, "max")])
def test_signature_expected_is_the_mean_and_every_slip_is_far(dtype, group, lengths):
    b = (signature_batch(dtype, group) if lengths == "long"
         else signature_batch(dtype, group, hist=MAX_HIST, new=MAX_NEW, seed=303))
    exp = signature_expected(b)
    tol = signature_tol(exp, dtype)
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        L = int(b.context_lens[r])
        v = signature_v(L, b.num_kv_heads, b.head_dim, r).astype(np.float64)
        cs = np.cumsum(v, axis=0)
        pos = b.query_positions(r)
        lo = int(b.cu_q_lens[r])
        # the closed form against a direct mean on a few rows
        for i in (0, len(pos) // 2, len(pos) - 1):
            p = int(pos[i])
            assert np.allclose(exp[lo + i, 0], v[:p + 1, 0].mean(axis=0), rtol=0, atol=1e-12)
        # partial sums per dim stay in {0, +-A}: |O| <= A/(p+1)
        assert np.all(np.abs(cs[:, :, :-1]) <= A)
        for h in range(b.num_heads):
            g = h // G
            e = exp[lo:lo + len(pos), h]
            t = tol[lo:lo + len(pos), h]
            for k in SLIPS:
                ok = (pos + k >= 0) & (pos + k < L)
                alt = cs[pos[ok] + k, g] / (pos[ok] + k + 1)[:, None]
                margin = np.max(np.abs(alt - e[ok]) / t[ok], axis=1)
                assert np.all(margin >= 10.0), (r, h, k, float(margin.min()))


@pytest.mark.parametrize("group", [1, 8])
def test_a_wrong_block_moves_some_dim_far(group):
    b = signature_batch("bf16", group)
    rng = np.random.default_rng(11)
    G = b.num_heads // b.num_kv_heads
    sig = {}
    for r in range(b.num_reqs):
        v = signature_v(int(b.context_lens[r]), b.num_kv_heads, b.head_dim, r).astype(np.float64)
        nblk = b.num_logical_blocks(r)
        full = nblk - 1                       # blocks wholly inside the context
        sig[r] = v[:16 * full].reshape(full, 16, b.num_kv_heads, b.head_dim).sum(axis=1)   # [blk][g][d]
    exp = signature_expected(b)
    tol = signature_tol(exp, "bf16")
    tried = coincide = 0
    for r in range(b.num_reqs):
        pos = b.query_positions(r)
        lo = int(b.cu_q_lens[r])
        row = len(pos) - 1                    # the last row sees every full block
        p = int(pos[row])
        for _ in range(400):
            j = int(rng.integers(0, len(sig[r])))
            r2 = int(rng.integers(0, b.num_reqs))
            j2 = int(rng.integers(0, len(sig[r2])))
            h = int(rng.integers(0, b.num_heads))
            g = h // G
            g2 = int(rng.integers(0, b.num_kv_heads))
            if (r2, j2, g2) == (r, j, g):
                continue
            tried += 1
            alt = exp[lo + row, h] + (sig[r2][j2, g2] - sig[r][j, g]) / (p + 1)
            if np.max(np.abs(alt - exp[lo + row, h]) / tol[lo + row, h]) < 10.0:
                coincide += 1
    assert coincide <= 0.01 * tried, (coincide, tried)


@pytest.mark.parametrize("group", [1, 8])
def test_onehot_expected_matches_the_exact_attention(group):
    b = onehot_batch("bf16", group)
    exp = onehot_expected(b)
    rng = np.random.default_rng(12)
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        k, v = b.request_kv(r)
        q = b.request_q(r)
        pos = b.query_positions(r)
        lo = int(b.cu_q_lens[r])
        assert len(np.unique(v.reshape(len(v), -1), axis=0)) == len(v), "two V rows coincide"
        rows = sorted({0, len(pos) - 1} | set(rng.choice(len(pos), size=6, replace=False).tolist()))
        for h in (0, b.num_heads - 1):
            g = h // G
            kk = oracle.to_f64(k[:, g, :], "bf16")
            vv = oracle.to_f64(v[:, g, :], "bf16")
            qq = oracle.to_f64(q[rows, h, :], "bf16")
            ref = oracle.causal_attention(qq, kk, vv, pos[rows], b.softmax_scale)
            err = np.max(np.abs(ref - exp[lo + np.asarray(rows), h]))
            assert err <= 1e-4, (r, h, err)
    assert ONEHOT_TOL * 10 <= 2.0
