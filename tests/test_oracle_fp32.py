"""The oracle carried out in float32 (the precision the CPU baseline is timed in) computes the same
attention as the float64 oracle, to float32 rounding, unsplit and split."""

import numpy as np

import oracle
from oracle_helpers import batch_q_pos, oracle_pools
from workloads import config_batch, custom_batch


def test_float32_oracle_matches_float64():
    for b in (config_batch(1, num_reqs=3, num_heads=4), config_batch(3, num_reqs=2, max_hist=700),
              custom_batch([40, 0, 300], [5, 12, 1], num_heads=4, num_kv_heads=2, head_dim=64, dtype="f32", seed=3)):
        k_pool, v_pool = oracle_pools(b)
        args = (b.q_all(), k_pool, v_pool, b.block_tables, b.context_lens, b.cu_q_lens, batch_q_pos(b),
                b.softmax_scale, b.dtype)
        o64 = oracle.paged_attention(*args)
        o32 = oracle.paged_attention(*args, compute=np.float32)
        assert np.max(np.abs(o32 - o64)) <= 2e-6, b.name
        p64 = oracle.split_partial(*args, 5)
        p32 = oracle.split_partial(*args, 5, compute=np.float32)
        m32 = oracle.split_merge(*p32, compute=np.float32)
        assert np.max(np.abs(m32 - oracle.split_merge(*p64))) <= 2e-6, b.name
        assert np.max(np.abs(m32 - o64)) <= 2e-6, b.name
