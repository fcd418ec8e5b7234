"""Seeded input generators: reproducible, tables valid, shapes as named (CPU)."""
import math

import numpy as np
import pytest
import torch

from workloads import make_config, make_small, permute_pool, poison_unused, raw_numpy


def _owned_counts(w):
    B = w.block_size
    if "prompts" in w.meta:
        return w.meta["prompt_blocks"] + -(-(w.meta["tails"].astype(np.int64) + 1) // B)
    return -(-(w.context_lens.astype(np.int64) + 1) // B)


def _check_tables(w):
    owned = _owned_counts(w)
    assert owned.max() <= w.max_blocks_per_seq
    T = w.block_tables
    assert T.min() >= 0 and T.max() < w.num_blocks
    ids = np.concatenate([T[s, :owned[s]] for s in range(w.num_seqs)])
    if "prompts" in w.meta:
        n_prompts, n_sib, _ = w.meta["prompts"]
        pb = w.meta["prompt_blocks"]
        for j in range(n_prompts):
            rows = T[j * n_sib:(j + 1) * n_sib, :pb]
            assert (rows == rows[0]).all()          # siblings alias the prompt
        private = np.concatenate([T[s, pb:owned[s]] for s in range(w.num_seqs)])
        shared = T[::n_sib, :pb].ravel()
        assert len(np.unique(private)) == len(private)
        assert len(np.unique(shared)) == len(shared)
        assert not set(private.tolist()) & set(shared.tolist())
    else:
        assert len(np.unique(ids)) == len(ids)       # no block owned twice


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_named_config_tables(k):
    w = make_config(k, values=False)
    _check_tables(w)
    need = w.meta["total_need"]
    if k == 1:
        assert w.num_blocks == 32 and w.context_lens.tolist() == [5, 16, 17, 40]
        assert (w.q_heads, w.kv_heads, w.head_dim, w.block_size, w.dtype) == (4, 4, 64, 16, "f32")
        assert w.scale == 0.125
    else:
        assert w.num_blocks == math.ceil(1.25 * need)
    if k == 2:
        assert w.num_seqs == 64 and 128 <= w.context_lens.min() and w.context_lens.max() <= 2048
        assert (w.q_heads, w.kv_heads, w.head_dim, w.block_size) == (32, 32, 128, 16)
    if k == 3:
        assert w.num_seqs == 256 and 1 <= w.context_lens.min() and w.context_lens.max() <= 4096
        assert (w.q_heads, w.kv_heads, w.block_size) == (32, 8, 32)
        assert 300 < np.median(w.context_lens) < 800
    if k == 4:
        assert w.num_seqs == 512 and (w.context_lens >= 1024).all() and (w.context_lens <= 1087).all()
        assert (w.q_heads, w.kv_heads, w.block_size) == (40, 40, 16)
    if k == 5:
        assert w.num_seqs == 8 and (w.context_lens == 32768).all()
        assert (w.q_heads, w.kv_heads) == (64, 8) and w.num_blocks == 20490


def test_seeded_and_reproducible():
    a, b = make_config(1), make_config(1)
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.k_new, b.k_new)]:
        assert torch.equal(x, y)
    assert np.array_equal(a.block_tables, b.block_tables)
    c = make_small(2, seed_offset=1)
    assert not np.array_equal(c.context_lens, make_small(2).context_lens)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_small_configs(k):
    w = make_small(k)
    _check_tables(w)
    assert w.q.shape == (w.num_seqs, w.q_heads, w.head_dim)
    assert w.k_cache.shape == (w.num_blocks, w.block_size, w.kv_heads, w.head_dim)
    assert w.k_new.shape == (w.num_seqs, w.kv_heads, w.head_dim)
    assert w.q.dtype == (torch.float32 if w.dtype == "f32" else torch.bfloat16)


def test_bf16_is_round_to_nearest_even():
    w = make_small(2)
    bits = raw_numpy(w.q)
    assert bits.dtype == np.uint16
    # regenerate the fp32 draw and round it by hand (RNE on the top 16 bits)
    rng = np.random.default_rng(w.seed)
    rng.integers(1, 700, size=6)
    rng.permutation(w.num_blocks)
    f = rng.standard_normal(w.q.shape, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rne = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(bits, rne)


def test_permute_and_poison():
    w = make_small(3)
    perm = np.random.default_rng(3).permutation(w.num_blocks)
    p = permute_pool(w, perm)
    for b in range(w.num_blocks):
        assert torch.equal(p.k_cache[perm[b]], w.k_cache[b])
    z = poison_unused(w)
    free = z.meta["free_blocks"]
    assert torch.isnan(z.k_cache[torch.from_numpy(free)].float()).all()
    _check_tables(z)
