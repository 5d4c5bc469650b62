"""Synthetic workload generator: shapes, determinism and the stated recipe."""
import numpy as np
import pytest

import workloads as wl
from oracle import lychee_oracle as orc


def test_presets_match_recipe():
    t = wl.get_workload("tiny")
    assert (t.batch, t.layers, t.num_q_heads, t.num_kv_heads, t.head_dim) == (1, 2, 4, 4, 64)
    assert t.seq_lens == (1024,) and t.k_per_seq == (307,)
    assert t.retrieval_masks == (0b1111, 0b0001)
    l = wl.get_workload("llama3_8b_32k")
    assert l.k_per_seq == (9830,) and l.group_size == 4
    assert l.retrieval_masks[0] == (1 << 32) - 1
    assert sum(bin(m).count("1") for m in l.retrieval_masks[1:]) == 32
    q = wl.get_workload("qwen3_8b_128k")
    assert q.k_per_seq == (39321,) and q.layers == 36
    r = wl.get_workload("ragged_b8")
    assert r.batch == 8 and all(16384 <= n <= 65536 for n in r.seq_lens)
    assert r.k_per_seq == tuple((3 * n) // 10 for n in r.seq_lens)
    assert r.retrieval_masks == l.retrieval_masks
    h = wl.get_workload("hysparse_7layer")
    assert h.kv_layers() == 1 and h.k_per_seq == (4096,)
    assert h.retrieval_masks[1:] == (0,) * 6


def test_layer_inputs_deterministic_and_shaped():
    t = wl.get_workload("tiny")
    a = wl.make_layer_inputs(t, 0)
    b = wl.make_layer_inputs(t, 0)
    assert tuple(a.q.shape) == (1, 4, 64) and tuple(a.k.shape) == (4, 1024, 64)
    assert np.array_equal(wl.bf16_bits(a.k), wl.bf16_bits(b.k))
    c = wl.make_layer_inputs(t, 1)
    assert not np.array_equal(wl.bf16_bits(a.q), wl.bf16_bits(c.q))


def test_planted_heavy_hitters_enter_layer0_selection():
    # Seeded sanity check of the data recipe (not parity): with MHA the planted
    # rows score about 4 sigma above the rest, so layer 0 selects all of them.
    t = wl.get_workload("tiny")
    x = wl.make_layer_inputs(t, 0)
    O, S, _ = orc.hybrid_layer_bf16(wl.bf16_bits(x.q), wl.bf16_bits(x.k), wl.bf16_bits(x.v),
                                    t.kv_offsets(), [True] * 4, t.k_per_seq, None)
    for g in range(4):
        pos = wl.heavy_hitter_positions(t, 0, g)
        assert pos.size == 20
        assert set(pos.tolist()) <= set(S[(0, g)].tolist())


def test_random_sorted_sets():
    s = wl.random_sorted_sets(5, 100, 30, 4)
    assert s.shape == (4, 30) and s.dtype == np.int32
    for row in s:
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < 100
