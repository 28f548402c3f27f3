"""The seeded generators: deterministic, right shapes and structure."""

import math

import numpy as np
import pytest
import torch

from paged_kv_cache_186_amd import workloads as W


def _used_blocks(w):
    t = w.block_tables_np()
    lens = w.context_lens_np()
    ids = []
    for s in range(w.num_seqs):
        ids += t[s, : -(-int(lens[s]) // w.block_size)].tolist()
    return ids


def test_tiny_structure_and_poison():
    w = W.tiny(0)
    assert list(w.context_lens_np()) == [1, 7, 16, 33]
    ids = _used_blocks(w)
    assert len(ids) == 6 and len(set(ids)) == 6
    assert w.k_pool.shape == (16, 4, 16, 64) and w.dtype == torch.float32
    assert w.scale == 1 / 8
    unused = sorted(set(range(16)) - set(ids))
    assert torch.isnan(w.k_pool[unused]).all()
    # rows past the length of the last block are poisoned too
    last = int(w.block_tables_np()[1, 0])
    assert torch.isnan(w.k_pool[last, :, 7:]).all() and not torch.isnan(w.k_pool[last, :, :7]).any()


def test_layer_shape_determinism_and_ranges():
    a = W.layer_shape(1)
    b = W.layer_shape(1)
    c = W.layer_shape(2)
    assert np.array_equal(a.context_lens_np(), b.context_lens_np())
    assert np.array_equal(a.block_tables_np(), b.block_tables_np())
    assert torch.equal(a.q, b.q) and torch.equal(a.k_pool[:4], b.k_pool[:4])
    assert not np.array_equal(a.context_lens_np(), c.context_lens_np())
    lens = a.context_lens_np()
    assert lens.min() >= 1 and lens.max() <= 2048 and len(lens) == 8
    ids = _used_blocks(a)
    assert len(ids) == len(set(ids)) and max(ids) < 1024
    assert a.block_tables_np().shape == (8, 128)


def test_continuous_batching_lengths_and_pool():
    w = W.continuous_batching(0, values=False)
    lens = w.context_lens_np()
    assert len(lens) == 64 and lens.min() >= 32 and lens.max() <= 4096
    assert 200 < np.median(lens) < 1200
    assert w.num_blocks >= sum(-(-(int(L) + 48) // 32) for L in lens)
    # 48 steps of one token each fit the pool
    for _ in range(48):
        for s in w.seq_ids:
            w.manager.append_slot(s)
    assert w.block_tables_np().shape[1] >= max(-(-int(L) // 32) for L in w.context_lens_np())


def test_shared_prefix_layout():
    w = W.shared_prefix(0, values=False)
    t = w.block_tables_np()
    lens = w.context_lens_np()
    suffix = w.extra["suffix_lens"]
    assert (lens == 1024 + suffix).all()
    # blocks 0..62 shared by every sequence; block 63 private where a suffix exists
    assert (t[:, :63] == t[0, :63]).all()
    assert len(w.cow_pairs) == int((suffix > 0).sum()) - 1
    srcs = {p[0] for p in w.cow_pairs}
    dsts = [p[1] for p in w.cow_pairs]
    assert len(srcs) == 1 and len(set(dsts)) == len(dsts) and not (srcs & set(dsts))
    assert all(len(sl) == n for sl, n in zip(w.extra["suffix_slots"], suffix))


@pytest.mark.slow
def test_long_context_tables_are_a_permutation():
    w = W.long_context(0, batch=2, values=False, context=16 * 1024)
    t = w.block_tables_np()
    assert t.shape == (2, 1024)
    assert sorted(t.ravel().tolist()) == list(range(2048))


def test_new_token_values_are_seeded():
    w = W.tiny(3)
    a = W.new_token_values(w, 5)
    b = W.new_token_values(w, 5)
    c = W.new_token_values(w, 6)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    assert not torch.equal(a[1], c[1])
