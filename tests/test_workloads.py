"""Seeded input generator: determinism and the structure each workload promises. CPU only."""

import numpy as np
import pytest

from workloads import bf16_bits_from_f32, config_batch, custom_batch


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.0, 3.0e-3, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 3*2^-8 rounds up to 1 + 2^-6
    assert back[5] == 1.0 and back[6] == np.float32(1.0 + 2 ** -6)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)


@pytest.mark.parametrize("index", [0, 1, 3, 4])
def test_config_structure(index):
    b = config_batch(index)
    L, q = b.context_lens, b.q_lens
    assert np.all(q <= L) and np.all(q >= 1)
    # blocks of all requests are distinct and inside the pool
    used = np.concatenate([b.block_tables[r][:b.num_logical_blocks(r)] for r in range(b.num_reqs)])
    assert len(np.unique(used)) == len(used)
    assert used.min() >= 0 and used.max() < b.num_blocks
    # every query row's slot is unique; positions strictly increase and stay below L
    assert len(np.unique(b.new_slots)) == b.total_q
    for r in range(b.num_reqs):
        p = b.query_positions(r)
        assert np.all(np.diff(p) > 0) and p[-1] == L[r] - 1 and p.min() >= 0
    if index == 0:
        assert list(b.hist_lens) == [37, 80, 0] and list(b.new_lens) == [5, 1, 12] and b.num_blocks == 32
        assert b.dtype == "f32" and b.head_dim == 64 and b.num_heads == b.num_kv_heads == 4
    if index == 1:
        assert b.num_reqs == 64 and np.all(b.new_lens[32:] == 1)
        assert np.all((b.hist_lens >= 256) & (b.hist_lens <= 2048))
        assert np.all((b.new_lens[:32] >= 16) & (b.new_lens[:32] <= 128))
        assert b.num_blocks == int(np.ceil(1.25 * sum(b.num_logical_blocks(r) for r in range(64))))
    if index == 3:
        assert b.num_heads == 16 and b.num_kv_heads == 2 and b.dtype == "bf16"
        assert np.all(b.evict_lens % 16 == 0)
        assert np.all(b.evict_lens // 16 <= (b.hist_lens // 16) // 2)
        assert np.all((b.new_lens >= 1) & (b.new_lens <= 256))
        assert not b.has_default_positions
    if index == 4:
        assert list(b.hist_lens) == [32768, 40960, 49152, 65536] and list(b.new_lens) == [1, 1, 512, 1]


def test_decode_heavy_lengths():
    b = config_batch(2)
    assert b.num_reqs == 256 and np.all(b.new_lens == 1)
    assert b.hist_lens.min() >= 64 and b.hist_lens.max() <= 4096
    assert 600 < np.median(b.hist_lens) < 1600


def test_values_deterministic_and_per_request():
    a = config_batch(1, num_reqs=3, num_heads=4)
    b = config_batch(1, num_reqs=3, num_heads=4)
    for r in range(a.num_reqs):
        assert np.array_equal(a.request_q(r), b.request_q(r))
        ka, va = a.request_kv(r)
        kb, vb = b.request_kv(r)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)
        assert ka.dtype == np.float16 and ka.shape == (a.context_lens[r], a.num_kv_heads, a.head_dim)
    q = a.q_all().astype(np.float32)
    assert abs(q.std() - 0.5) < 0.05 and abs(q.mean()) < 0.05


def test_custom_batch_slots_follow_block_table():
    b = custom_batch([20, 0], [5, 17], num_heads=2, num_kv_heads=1, head_dim=8, seed=3)
    for r in range(2):
        pos = b.query_positions(r)
        slots = b.slots_for(r, pos)
        assert np.array_equal(slots // 16, b.block_tables[r][pos // 16])
        assert np.array_equal(slots % 16, pos % 16)


def test_conversation_script_turns():
    """Each conversation alternates idle spells and turns: a prompt step (16-96 tokens) followed by
    2-6 decode steps of one token (cut at the end of the run); the draws are seeded."""
    from workloads import conversation_script
    s = conversation_script(7, 9, 60)
    assert s.shape == (60, 9) and s.dtype == np.int32
    assert np.array_equal(s, conversation_script(7, 9, 60))
    assert not np.array_equal(s, conversation_script(8, 9, 60))
    for c in range(9):
        col = s[:, c]
        t = 0
        while t < 60:
            if col[t] == 0:
                t += 1
                continue
            assert 16 <= col[t] <= 96, (c, t, col[t])      # a turn opens with its prompt
            t += 1
            n = 0
            while t < 60 and col[t] == 1:
                n += 1
                t += 1
            assert n <= 6 and (n >= 2 or t == 60), (c, t, n)


def test_draw_rows_is_seeded_and_rounded():
    from workloads import draw_rows
    a = draw_rows((1, 2, 3), (5, 4), "bf16")
    assert a.dtype == np.uint16 and a.shape == (5, 4)
    assert np.array_equal(a, draw_rows((1, 2, 3), (5, 4), "bf16"))
    f = draw_rows((1, 2, 3), (5, 4), "f32")
    assert np.array_equal(bf16_bits_from_f32(f), a)     # same normals, rounded to bf16
