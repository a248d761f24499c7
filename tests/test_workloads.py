"""Seeded input generator: the block pool, tables and slots it builds are well formed."""
import math

import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("cfg_id", sorted(W.CONFIGS))
def test_metadata_well_formed(cfg_id):
    m = W.make_metadata(cfg_id)
    cfg = m.cfg
    bs = cfg.block_size
    L = m.context_lens.astype(np.int64)
    assert len(L) == cfg.num_seqs and L.min() >= 1 and L.max() <= cfg.max_context
    nblk = (L + bs - 1) // bs
    used = []
    for i in range(cfg.num_seqs):
        row = m.block_tables[i]
        assert (row[:nblk[i]] >= 0).all() and (row[nblk[i]:] == -1).all()
        used.extend(row[:nblk[i]].tolist())
        assert (m.owner[row[:nblk[i]]] == i).all()
    assert len(set(used)) == len(used)                     # no block in two tables
    assert max(used) < m.num_blocks
    b, o = m.slot_mapping // bs, m.slot_mapping % bs
    assert np.array_equal(b, m.block_tables[np.arange(cfg.num_seqs), (L - 1) // bs])
    assert np.array_equal(o, (L - 1) % bs)
    assert len(np.unique(m.slot_mapping)) == cfg.num_seqs


def test_tiny_config_matches_the_pages_example():
    m = W.make_metadata(1)
    assert m.context_lens.tolist() == [6, 50, 8, 100]
    assert [int((r >= 0).sum()) for r in m.block_tables] == [1, 4, 1, 7]
    assert m.num_blocks == 64 and m.blocks_in_tables == 13


def test_pool_sizes_follow_each_recipe():
    for cfg_id, factor in ((2, 1.25), (3, 1.0), (5, 1.1)):
        m = W.make_metadata(cfg_id)
        assert m.num_blocks == math.ceil(factor * m.blocks_in_tables - 1e-9)
    m = W.make_metadata(4)
    foreign = (m.owner == W.FOREIGN).sum()
    assert foreign == round(0.3 * m.num_blocks)
    assert m.num_blocks - foreign - m.blocks_in_tables >= 0.2 * m.blocks_in_tables
    m3 = W.make_metadata(3)
    assert sorted(m3.block_tables.ravel().tolist()) == list(range(m3.num_blocks))   # a permutation


def test_lengths_follow_each_distribution():
    L2 = W.make_metadata(2).context_lens
    assert L2.min() >= 128 and L2.max() <= 2048
    L4 = W.make_metadata(4).context_lens
    assert L4.min() >= 8 and L4.max() <= 8192 and 300 < np.median(L4) < 800
    L5 = W.make_metadata(5).context_lens
    assert L5.min() >= 16 and L5.max() <= 4096


@pytest.mark.parametrize("cfg_id", [2, 4])
def test_consecutive_placement_changes_only_block_ids(cfg_id):
    a, b = W.make_metadata(cfg_id), W.make_metadata(cfg_id, placement="consecutive")
    assert np.array_equal(a.context_lens, b.context_lens) and a.num_blocks == b.num_blocks
    assert (a.block_tables >= 0).sum() == (b.block_tables >= 0).sum()
    assert np.array_equal(a.block_tables >= 0, b.block_tables >= 0)
    assert np.array_equal(a.owner == W.FOREIGN, b.owner == W.FOREIGN)
    ids = np.concatenate([row[row >= 0] for row in b.block_tables])
    assert (np.diff(ids) > 0).all()                          # ascending through the batch
    if cfg_id == 2:                                          # no foreign blocks: one run from block 0
        assert np.array_equal(ids, np.arange(len(ids)))
    with pytest.raises(ValueError):
        W.make_metadata(cfg_id, placement="interleaved")


def test_seeded_and_reproducible():
    a, b = W.make_metadata(2), W.make_metadata(2)
    assert np.array_equal(a.block_tables, b.block_tables) and np.array_equal(a.context_lens, b.context_lens)
    c = W.make_metadata(2, seed=5)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_poisoned_workload_on_cpu():
    import torch
    m = W.make_metadata(1)
    w = W.make_workload(m, "cpu")
    k = w.k_cache
    bs = m.cfg.block_size
    for i, L in enumerate(m.context_lens.tolist()):
        row = m.block_tables[i]
        for t in range(L - 1):
            assert torch.isfinite(k[row[t // bs], :, t % bs]).all()
        last = row[(L - 1) // bs]
        assert torch.isnan(k[last, :, (L - 1) % bs:]).all()
    free = np.nonzero(m.owner == W.FREE)[0]
    assert torch.isnan(k[torch.from_numpy(free)]).all()
    assert torch.isfinite(w.q).all() and torch.isfinite(w.k_new).all()


def test_secondary_workloads_are_seeded_and_well_formed():
    sc = W.SamplingConfig()
    lens, nb, order = W.sampling_prompts(sc)
    assert len(lens) == sc.prompts and lens.min() >= sc.min_len and lens.max() <= sc.max_len
    assert sorted(order.tolist()) == list(range(nb))
    assert nb >= -(-(lens.astype(np.int64) + 15) // 16).sum()
    l2, _, o2 = W.sampling_prompts(sc)
    assert np.array_equal(lens, l2) and np.array_equal(order, o2)
    bc = W.BatchingConfig()
    p, g = W.batching_requests(bc, 1000)
    assert p.min() >= bc.prompt_min and p.max() <= bc.prompt_max and 300 < np.median(p) < 800
    assert g.min() >= bc.gen_min and g.max() <= bc.gen_max
    assert bc.width * bc.block_size >= bc.prompt_max + bc.gen_max
    pc = W.PrefillConfig()
    lens, nb, order = W.prefill_prompts(pc)
    assert len(lens) == pc.prompts and nb == -(-5 * int(((lens + 15) // 16).sum()) // 4)


def test_kv_pool_is_one_allocation_with_v_after_k():
    """The generators hold a layer's K and V caches as the two halves of one tensor (V directly after K), the
    placement the decode measured fastest; each half is a contiguous [NB, H, bs, D] cache."""
    torch = pytest.importorskip("torch")
    for zero in (False, True):
        k, v = W.kv_pool(7, 3, 16, 64, torch.bfloat16, "cpu", zero=zero)
        assert k.shape == v.shape == (7, 3, 16, 64) and k.is_contiguous() and v.is_contiguous()
        assert k.untyped_storage().data_ptr() == v.untyped_storage().data_ptr()
        assert v.data_ptr() - k.data_ptr() == k.numel() * k.element_size()
        if zero:
            assert not k.any() and not v.any()
    meta = W.make_metadata(1)
    w = W.make_workload(meta, "cpu")
    assert w.v_cache.data_ptr() - w.k_cache.data_ptr() == w.k_cache.numel() * w.k_cache.element_size()

