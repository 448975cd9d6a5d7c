"""Pins of the oracle's FP8 (E4M3) KV storage: format, rounding, scales.

The E4M3 decode table is checked against torch's float8_e4m3fn conversion and
against values fixed by the format's bit layout; the encoder against torch's
round-to-nearest-even cast over in-range values (exact midpoints included) and
against its own decode (every finite code round-trips); the scales against the
closed form of a zero query and against torch's scaled_dot_product_attention
over K/V decoded by torch.  Mutants of each step must fail a pin.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import custom_batch

from oracle_helpers import oracle_pools


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---- pins of the format -----------------------------------------------------------
def _pin_decode_table(decode):
    codes = np.arange(256, dtype=np.uint8)
    got, ref = decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # Values fixed by the bit layout (bias 7, 3 mantissa bits, subnormals, 448 max).
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0xC0: -2.0, 0xFE: -448.0}
    for c, v in fixed.items():
        assert decode(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(decode(np.array([0x7F, 0xFF], np.uint8))).all()


def _midpoints():
    vals = oracle.E4M3_VALUES[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2          # exact in float32: 5 significant bits at most
    return np.concatenate([vals, mids, -vals, -mids])


def _pin_encode_vs_torch(encode):
    rng = np.random.default_rng(3)
    x = np.concatenate([
        _midpoints(),
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.05,     # subnormal range and below
        np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-14, 9, 4000)) * rng.choice([-1, 1], 4000),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448.0]               # torch's cast does not saturate; compare in range only
    assert np.array_equal(encode(x.astype(np.float64)), _torch_encode(x))


def _pin_round_trip(encode, decode):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode(decode(codes)), codes)


def _pin_saturation(encode):
    assert list(encode(np.array([1e30, -1e30, 449.0, 470.0, -500.0]))) == [0x7E, 0xFE, 0x7E, 0x7E, 0xFE]


def test_e4m3_decode_table():
    _pin_decode_table(oracle.e4m3_decode)


def test_e4m3_encode_matches_round_to_nearest_even():
    _pin_encode_vs_torch(oracle.e4m3_encode)


def test_e4m3_every_finite_code_round_trips():
    _pin_round_trip(oracle.e4m3_encode, oracle.e4m3_decode)


def test_e4m3_saturates_beyond_the_largest_finite_value():
    _pin_saturation(oracle.e4m3_encode)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 1 / 128, 0.0123, 3.0])
def test_quantize_divides_in_float32(dtype, scale):
    b = custom_batch([40], [8], dtype=dtype, seed=9)
    k, _ = b.request_kv(0)
    got = oracle.quantize_e4m3(k, dtype, scale)
    xf = torch.from_numpy(oracle.to_f64(k, dtype).astype(np.float32))
    t = xf / torch.tensor(scale, dtype=torch.float32)
    t = torch.clamp(t, -448.0, 448.0)
    ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


# ---- pins of the scaled attention -----------------------------------------------------
def _fp8_pools(b, k_scale, v_scale):
    """Pools of E4M3 codes of the batch's K/V (every position resident)."""
    kp, vp = oracle_pools(b, poison=False)
    return (oracle.quantize_e4m3(kp, b.dtype, k_scale), oracle.quantize_e4m3(vp, b.dtype, v_scale))


def test_fp8_attention_matches_sdpa_over_torch_decoded_kv():
    b = custom_batch([50, 20], [6, 17], num_heads=4, num_kv_heads=2, dtype="bf16", seed=21)
    ks, vs = 1 / 96, 1 / 80
    kc, vc = _fp8_pools(b, ks, vs)
    got = oracle.paged_attention(b.q_all(), kc, vc, b.block_tables, b.context_lens, b.cu_q_lens, None,
                                 b.softmax_scale, b.dtype, kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    q = oracle.to_f64(b.q_all(), b.dtype)
    for r in range(b.num_reqs):
        lo, hi, L = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1]), int(b.context_lens[r])
        blocks = b.block_tables[r][: -(-L // 16)]
        for h in range(4):
            g = h // 2
            kk = np.concatenate([_torch_decode(kc[p, g]) for p in blocks])[:L] * ks
            vv = np.concatenate([_torch_decode(vc[p, g]) for p in blocks])[:L] * vs
            qq = q[lo:hi, h]
            mask = np.arange(L)[None, :] <= np.arange(L - (hi - lo), L)[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qq)[None], torch.from_numpy(kk)[None], torch.from_numpy(vv)[None],
                attn_mask=torch.from_numpy(mask)[None], scale=b.softmax_scale)[0].numpy()
            np.testing.assert_allclose(got[lo:hi, h], ref, rtol=0, atol=1e-12)


def test_fp8_zero_query_is_the_scaled_mean_of_the_codes():
    b = custom_batch([33], [3], num_heads=2, num_kv_heads=2, dtype="f16", seed=4)
    b.q_fn = lambda r: np.zeros((int(b.q_lens[r]), 2, b.head_dim), np.float32)
    vs = 0.02
    kc, vc = _fp8_pools(b, 0.05, vs)
    got = oracle.paged_attention(b.q_all(), kc, vc, b.block_tables, b.context_lens, b.cu_q_lens, None,
                                 b.softmax_scale, b.dtype, kv_dtype="e4m3", k_scale=0.05, v_scale=vs)
    blocks = b.block_tables[0][:3]
    for h in range(2):
        codes = np.concatenate([vc[p, h] for p in blocks])[:36]
        vals = np.array([[oracle.e4m3_value(int(c)) for c in row] for row in codes]) * vs
        for i, p in enumerate(range(33, 36)):
            np.testing.assert_allclose(got[i, h], vals[: p + 1].mean(axis=0), rtol=0, atol=1e-14)


# ---- mutants: each must fail a pin ------------------------------------------------------
def _encode_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), oracle.E4M3_MAX)
    grid = oracle.E4M3_VALUES[:0x7F]
    code = (np.searchsorted(grid, mag, side="right") - 1).astype(np.uint8)
    return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), oracle.E4M3_MAX)
    grid = oracle.E4M3_VALUES[:0x7F]
    hi = np.clip(np.searchsorted(grid, mag), 0, 126)
    lo = np.maximum(hi - 1, 0)
    code = np.where(grid[hi] - mag <= mag - grid[lo], hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))


def _encode_no_subnormals(x):
    code = oracle.e4m3_encode(x)
    small = (code & 0x78) == 0
    return np.where(small, code & 0x80, code).astype(np.uint8)


def _decode_bias8(codes):
    return oracle.e4m3_decode(codes) / 2.0


def _encode_wraps(x):
    x = np.asarray(x, dtype=np.float64)
    return oracle.e4m3_encode(np.where(np.abs(x) > 448, np.nan, x))


@pytest.mark.parametrize("mutant,pin", [
    (_encode_truncating, "encode"), (_encode_ties_away, "encode"), (_encode_no_subnormals, "encode"),
    (_decode_bias8, "decode"), (_encode_wraps, "saturation"),
])
def test_fp8_pins_catch_mutants(mutant, pin):
    with pytest.raises(AssertionError):
        if pin == "encode":
            _pin_encode_vs_torch(mutant)
        elif pin == "decode":
            _pin_decode_table(mutant)
        else:
            _pin_saturation(mutant)
