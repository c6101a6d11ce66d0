"""Invariants of the seeded workload generator.

* Block-table invariant: every physical block is free, owned by one logical block, or
  shared with a reference count equal to its number of users ("vllm-project-vllm -- L2",
  section 8).
* Waste bound: a sequence of n tokens uses ceil(n / BS) blocks, so fewer than BS slots are
  wasted (same page, section 11 step 2).
* The step writes the new token at logical position n - 1 (blocks are extended every decode
  step, same page, section 6 "KV Cache Block Tables").
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_224_amd import inputs as I


@pytest.mark.parametrize("name", I.CONFIG_ORDER)
def test_table_invariants_full_size(name):
    cfg = I.CONFIGS[name]
    w = I.make_workload(cfg, tensors=False)
    BS, MB = cfg.block_size, cfg.max_blocks
    n = w.context_lens.astype(np.int64)
    assert w.block_tables.shape == (cfg.B, MB)
    assert np.all(n >= 1) and np.all(n <= cfg.max_len)
    used = -(-n // BS)
    assert np.all(used * BS - n < BS) and np.all(used * BS >= n)        # waste < one block
    ref = np.zeros(w.num_blocks, dtype=np.int64)
    for b in range(cfg.B):
        row = w.block_tables[b, :used[b]]
        assert np.all((row >= 0) & (row < w.num_blocks))
        assert len(set(row.tolist())) == row.size                     # no block twice in a row
        np.add.at(ref, row, 1)
        assert np.all(w.block_tables[b, used[b]:] == w.trap_block)
    assert np.array_equal(ref, w.refcount)
    assert w.refcount[w.trap_block] == 0
    shared = np.flatnonzero(w.refcount > 1)
    assert set(shared.tolist()) == set(w.prefix_blocks.tolist())
    assert np.all(w.refcount[w.prefix_blocks] == cfg.B) if w.prefix_blocks.size else True
    # new token of sequence b goes to logical position n_b - 1
    pos = n - 1
    assert np.array_equal(w.slot_mapping, w.block_tables[np.arange(cfg.B), pos // BS].astype(np.int64) * BS + pos % BS)
    assert len(set(w.slot_mapping.tolist())) == cfg.B                  # no duplicate slots


def test_pool_sizes_follow_recipe():
    w = I.make_workload(I.CONFIGS["tiny"], tensors=False)
    assert w.num_blocks == 80
    for name in ("llama3_8b", "long_ctx", "llama3_70b_fp8", "shared_prefix"):
        cfg = I.CONFIGS[name]
        w = I.make_workload(cfg, tensors=False)
        unique = int(np.count_nonzero(w.refcount))
        assert w.num_blocks == int(np.ceil(1.25 * unique))


def test_length_distributions():
    w = I.make_workload(I.CONFIGS["llama3_70b_fp8"], tensors=False)
    n = w.context_lens
    assert n.min() >= 16 and n.max() <= 32768
    assert 1500 < np.median(n) < 3000          # exp(7.5) ~ 1808
    w = I.make_workload(I.CONFIGS["shared_prefix"], tensors=False)
    assert np.all((w.context_lens >= 2048 + 64) & (w.context_lens <= 2048 + 512))
    assert w.prefix_blocks.size == 2048 // 16


def test_same_seed_same_tensors():
    a = I.make_workload(I.CONFIGS["tiny"])
    b = I.make_workload(I.CONFIGS["tiny"])
    for x, y in ((a.q, b.q), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool), (a.k_new, b.k_new)):
        assert torch.equal(x, y)
    assert np.array_equal(a.block_tables, b.block_tables)
    c = I.make_workload(I.shrink(I.CONFIGS["tiny"], seed=1))
    assert not torch.equal(a.q, c.q)


def test_values_are_standard_normal_rounded():
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=4, len_div=8))
    x = w.k_pool.float()
    assert w.k_pool.dtype == torch.bfloat16 and w.q.dtype == torch.bfloat16
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_fp8_scales_are_amax_over_448():
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_70b_fp8"], B=4, len_div=16))
    amax = max(float(w.k_pool.abs().max()), float(w.k_new.abs().max()))
    assert w.k_scale == float(np.float32(amax) / np.float32(448.0))
    assert w.k_pool.dtype == torch.bfloat16


def test_permute_and_unshare_preserve_logical_content():
    w = I.make_workload(I.shrink(I.CONFIGS["shared_prefix"], B=4, len_div=8))
    for w2 in (I.permute_blocks(w, 5), I.unshare_prefix(w)):
        BS = w.cfg.block_size
        for b in range(w.cfg.B):
            for t in range(0, int(w.context_lens[b]), 7):
                s1 = int(w.block_tables[b, t // BS]) * BS + t % BS
                s2 = int(w2.block_tables[b, t // BS]) * BS + t % BS
                assert torch.equal(w.k_pool.view(-1, 8, 128)[s1], w2.k_pool.view(-1, 8, 128)[s2])
                assert torch.equal(w.v_pool.view(-1, 8, 128)[s1], w2.v_pool.view(-1, 8, 128)[s2])


def test_algorithmic_bytes_llama3_8b():
    w = I.make_workload(I.CONFIGS["llama3_8b"], tensors=False)
    nb = I.algorithmic_bytes(w)
    assert nb["kv_logical"] == int(w.context_lens.sum()) * 8 * 128 * 2 * 2
    assert nb["kv_unique"] == nb["kv_logical"]
    w = I.make_workload(I.CONFIGS["shared_prefix"], tensors=False)
    nb = I.algorithmic_bytes(w)
    assert nb["kv_logical"] - nb["kv_unique"] == 255 * 2048 * 8 * 128 * 4
