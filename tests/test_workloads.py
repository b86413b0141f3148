"""Structure of the seeded inputs (CPU only)."""

import math

import numpy as np
import torch

import workloads as wl


def test_config_shapes_and_poison():
    for cfg, ctx, m in [(1, 256, 1), (2, 300, 2), (3, 2048, 4), (4, 1024, 3), (5, 2000, 4)]:
        c = wl.config_case(cfg, ctx, m)
        spec = wl.CONFIGS[cfg]
        S = c.num_seqs
        assert c.q.shape == (S, m, spec.num_q_heads, spec.head_size)
        assert c.q.dtype == spec.torch_dtype
        assert torch.isnan(c.kv_cache[c.poison_block]).all()
        lens = c.seq_lens.tolist()
        bt = c.block_tables[0]
        for s, L in enumerate(lens):
            need = -(-L // spec.page_size)
            live = bt[s, :need]
            if spec.window_table_only and L:
                first = wl.window_first_page(L, m, spec.window, spec.page_size)
                assert (bt[s, :first] == c.poison_block).all()
                live = bt[s, first:need]
            assert (live != c.poison_block).all()
            assert (bt[s, need:] == c.poison_block).all()
        if cfg == 5:
            assert S == 65 and lens[-1] == 0 and min(lens[:-1]) >= 512
        assert abs(c.scale - 1 / math.sqrt(spec.head_size)) < 1e-12


def test_instances_are_disjoint_and_seeded():
    a = wl.config_case(2, 512, 1, instances=3)
    b = wl.config_case(2, 512, 1, instances=3)
    assert torch.equal(a.q, b.q) and torch.equal(a.kv_cache.nan_to_num(), b.kv_cache.nan_to_num())
    used = [set(t[0, :32].tolist()) for t in a.block_tables]
    assert not (used[0] & used[1]) and not (used[1] & used[2])


def test_compact_is_a_renumbering():
    c = wl.config_case(2, 200, 2)
    kv64, table, lens = wl.compact(c)
    bt = c.block_tables[0].numpy()
    full = wl.as_f64(c.kv_cache)
    for j in range(-(-200 // 16)):
        np.testing.assert_array_equal(kv64[table[0, j]], full[bt[0, j]])
