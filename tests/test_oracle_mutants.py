"""Plant plausible mistakes in the CPU oracle and check that the pins catch each one.

Every mutant changes one step of the oracle (a mask bound, an index, an
operand, a weight); the test passes only if at least one pin in
``pins.ALL_PINS`` fails for it.  The planted mistakes live here, on the CPU,
and only for the duration of one test.
"""

import sys

import numpy as np
import pytest

import oracle
from pins import ALL_PINS

defs = sys.modules["oracle.definitions"]
_orig = {name: getattr(defs, name) for name in dir(defs) if not name.startswith("_")}


def _gather_shifted(k_pool, v_pool, row, L, g, B, dtype):
    n = -(-L // B)
    return _orig["gather_kv"](k_pool, v_pool, np.roll(np.asarray(row[:n]), 1), L, g, B, dtype)


def _gather_swapped(k_pool, v_pool, row, L, g, B, dtype):
    k, v = _orig["gather_kv"](k_pool, v_pool, row, L, g, B, dtype)
    return v, k


def _gather_v_dim_major(k_pool, v_pool, row, L, g, B, dtype):
    """Reads each V block as if it were stored [d][B] (dim rows) instead of [B][d]."""
    n = -(-L // B)
    k, _ = _orig["gather_kv"](k_pool, v_pool, row, L, g, B, dtype)
    d = k_pool.shape[-1]
    vs = [defs.to_f64(v_pool[int(row[j]), g], dtype).reshape(d, B).T for j in range(n)]
    return k, np.concatenate(vs)[:L] if vs else np.zeros((0, d))


def _attn_no_scale(q, k, v, pos, scale):
    return _orig["causal_attention"](q, k, v, pos, 1.0)


def _attn_scale_squared(q, k, v, pos, scale):
    return _orig["causal_attention"](q, k, v, pos, scale * scale)


def _attn_denominator_all_keys(q, k, v, pos, scale):
    s = (q @ k.T) * scale
    vis = defs.causal_visible(np.arange(k.shape[0]), pos)
    mx = np.where(vis, s, -np.inf).max(axis=1, keepdims=True)
    w = np.where(vis, np.exp(s - mx), 0.0)
    return (w @ v) / np.exp(s - mx).sum(axis=1, keepdims=True)


def _attn_base2(q, k, v, pos, scale):
    s = (q @ k.T) * scale
    vis = defs.causal_visible(np.arange(k.shape[0]), pos)
    m = np.where(vis, s, -np.inf)
    w = np.where(vis, np.exp2(m - m.max(axis=1, keepdims=True)), 0.0)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def _merge_no_rescale(po, pm, pl):
    live = pl > 0
    w = np.where(live, pl, 0.0)
    return (w[..., None] * np.where(live[..., None], po, 0.0)).sum(-2) / w.sum(-1)[..., None]


def _merge_plain_mean(po, pm, pl):
    live = (pl > 0).astype(float)
    return (live[..., None] * np.where(live[..., None] > 0, po, 0.0)).sum(-2) / live.sum(-1)[..., None]


def _ranges_floor(L, P, B):
    n = -(-L // B)
    per = max(n // P, 1)
    return [(min(k * per * B, L), min((k + 1) * per * B, L)) for k in range(P)]


def _append_v_offset(k_pool, v_pool, k_new, v_new, slots, B):
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), B)
        k_pool[b, :, o, :] = k_new[t]
        v_pool[b, :, :, (o + 1) % B] = v_new[t]


def _append_no_skip(k_pool, v_pool, k_new, v_new, slots, B):
    for t, s in enumerate(slots):
        b, o = divmod(int(s), B)
        k_pool[b, :, o, :] = k_new[t]
        v_pool[b, :, :, o] = v_new[t]


def _to_f64_bad_bf16(a, dtype):
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return _orig["to_f64"](a, dtype)


MUTANTS = {
    "mask_strict": {"causal_visible": lambda kp, rp: np.asarray(kp)[None, :] < np.asarray(rp)[:, None]},
    "mask_plus_one": {"causal_visible": lambda kp, rp: np.asarray(kp)[None, :] <= np.asarray(rp)[:, None] + 1},
    "gqa_modulo": {"kv_head_of": lambda h, hq, hkv: h % hkv},
    "gqa_first_head": {"kv_head_of": lambda h, hq, hkv: 0},
    "gather_shifted_blocks": {"gather_kv": _gather_shifted},
    "gather_k_v_swapped": {"gather_kv": _gather_swapped},
    "gather_v_untransposed": {"gather_kv": _gather_v_dim_major},
    "default_positions_shift": {"default_positions": lambda L, q: np.arange(L - q - 1, L - 1)},
    "q_pos_ignored": {"row_positions": lambda qp, lo, hi, L: np.arange(L - (hi - lo), L)},
    "no_scale": {"causal_attention": _attn_no_scale},
    "scale_squared": {"causal_attention": _attn_scale_squared},
    "denominator_all_keys": {"causal_attention": _attn_denominator_all_keys},
    "exp_base2": {"causal_attention": _attn_base2},
    "merge_no_rescale": {"split_merge": _merge_no_rescale},
    "merge_plain_mean": {"split_merge": _merge_plain_mean},
    "partition_floor": {"partition_token_ranges": _ranges_floor},
    "append_v_offset": {"append_kv": _append_v_offset},
    "append_no_skip": {"append_kv": _append_no_skip},
    "bf16_decode": {"to_f64": _to_f64_bad_bf16},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        monkeypatch.setattr(defs, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oracle)
        except Exception as exc:  # any failure (assertion, shape error, NaN) counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutant {name}"
