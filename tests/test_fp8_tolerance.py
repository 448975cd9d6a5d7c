"""Tolerance analysis for the arithmetic of E4M3 KV pools (CPU only).

E4M3 pools store K and V as 8-bit codes ("LLM上下文缓存与状态复用机制的分析和探索", section 4(3):
the KV cache kept in FP8 to halve its memory).  The kernels widen every code exactly to f16 /
bf16 (every E4M3 value is one of theirs) and run the same f16 / bf16 matrix-core and vector
arithmetic as for f16 / bf16 pools, so against the attention over the decoded codes they carry
exactly the error budget of the f16 / bf16 path, and the 1e-2 gate keeps its meaning.

gfx950's FP8 matrix-core instructions would also need the query rows (QK^T) and the softmax
weights (PV) as 8-bit floats.  These tests measure what that extra rounding costs, with the
float64 oracle as the reference, on the workloads' value distribution and at sharper score
scales: quantising Q to E4M3 (one scale per tensor, largest magnitude at 448) moves the output
by a few 1e-3 at the workloads' scale and past the 1e-2 gate once scores are a few times larger
(large logits are common in trained models); quantising the weights adds error of the same
kind.  Both would be a precision change of the method's arithmetic, not a storage format, which
is why the E4M3 path widens codes instead.
"""

import numpy as np
import pytest

import oracle
from oracle_helpers import oracle_pools
from workloads import custom_batch

KS = VS = 1 / 128


def _e4m3_round(x):
    """x rounded to E4M3 with one scale for the whole array (largest magnitude maps to 448)."""
    s = float(np.max(np.abs(x))) / oracle.E4M3_MAX
    return oracle.e4m3_decode(oracle.e4m3_encode(x / s)) * s


def _attention(b, kc, vc, q_scale=1.0, quant_q=False, quant_p=False):
    """Attention over decoded E4M3 pools with optional E4M3 rounding of Q and of the weights."""
    q = oracle.to_f64(b.q_all(), b.dtype) * q_scale
    out = np.zeros(q.shape)
    G = b.num_heads // b.num_kv_heads
    for r in range(b.num_reqs):
        lo, hi, L = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1]), int(b.context_lens[r])
        pos = b.query_positions(r)
        for h in range(b.num_heads):
            k, v = oracle.gather_kv(kc, vc, b.block_tables[r], L, h // G, 16, "e4m3", KS, VS)
            qr = q[lo:hi, h]
            if quant_q:
                qr = _e4m3_round(qr)
            s = qr @ k.T * b.softmax_scale
            vis = oracle.causal_visible(np.arange(L), pos)
            s = np.where(vis, s, -np.inf)
            p = np.where(vis, np.exp(s - s.max(axis=1, keepdims=True)), 0.0)
            if quant_p:
                p = oracle.e4m3_decode(oracle.e4m3_encode(p))     # weights in [0, 1]: no scale needed
            out[lo:hi, h] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


@pytest.fixture(scope="module")
def batch():
    b = custom_batch([300, 900, 1500, 64], [40, 1, 24, 1], num_heads=4, num_kv_heads=4, head_dim=128,
                     dtype="bf16", seed=51)
    kc, vc = oracle_pools(b, poison=False)
    return b, oracle.quantize_e4m3(kc, b.dtype, KS), oracle.quantize_e4m3(vc, b.dtype, VS)


def test_exact_widening_is_the_decoded_attention(batch):
    b, kc, vc = batch
    ref = oracle.paged_attention(b.q_all(), kc, vc, b.block_tables, b.context_lens, b.cu_q_lens, None,
                                 b.softmax_scale, b.dtype, kv_dtype="e4m3", k_scale=KS, v_scale=VS)
    assert np.max(np.abs(_attention(b, kc, vc) - ref)) <= 1e-12


@pytest.mark.parametrize("q_scale,lo,hi", [(1.0, 1e-4, 1e-2), (8.0, 1e-2, 1.0)])
def test_fp8_query_rounding_error(batch, q_scale, lo, hi):
    """Q in E4M3: a few 1e-3 at the workloads' value scale (under the gate), past the gate when the
    scores are 8x sharper."""
    b, kc, vc = batch
    ref = _attention(b, kc, vc, q_scale)
    err = float(np.max(np.abs(_attention(b, kc, vc, q_scale, quant_q=True) - ref)))
    print(f"Q scale {q_scale}: max |dO| with E4M3 queries {err:.3e}")
    assert lo <= err <= hi


def test_fp8_weight_rounding_error(batch):
    """Softmax weights in E4M3 on top of E4M3 queries: more error of the same kind."""
    b, kc, vc = batch
    ref = _attention(b, kc, vc, 8.0)
    e_q = float(np.max(np.abs(_attention(b, kc, vc, 8.0, quant_q=True) - ref)))
    e_qp = float(np.max(np.abs(_attention(b, kc, vc, 8.0, quant_q=True, quant_p=True) - ref)))
    print(f"Q scale 8: E4M3 queries {e_q:.3e}, queries and weights {e_qp:.3e}")
    assert e_qp >= 1e-2
