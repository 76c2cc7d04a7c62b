"""Pins of the oracle's tree-masked prefill (T1) -- checks of the oracle against things it was not
written from.

Lecture 34 "vLLM 生产级系统架构全景剖析" §5.3: a tree of drafted tokens (EAGLE) is verified by the
target model in one pass; each drafted token sees the context and the drafted tokens on its own path
from the root. The oracle takes that as one 64-bit mask per row. These tests build trees from parent
arrays, walk each node's path explicitly, and compare with torch's float64 attention over exactly
those rows; the special trees reduce to operations pinned elsewhere (causal prefill, decode).
"""
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from pa_testutil import random_parents, tree_masks as masks, tree_path as path


def sdpa64(q, K, V, scale):
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None, None]
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, 0, 0].numpy()


def rows_of(w, cache, s, kvh, positions):
    """float64 rows of the given positions of sequence s, kv head kvh (numpy view of the pool)."""
    pos = np.asarray(positions, dtype=np.int64)
    pool = np.asarray(cache).reshape(w.num_blocks, w.H_kv, W.BLOCK, w.D)
    blk = w.block_tables[s][pos // W.BLOCK]
    return oracle.to_double(pool[blk, kvh, pos % W.BLOCK, :], w.dtype)


def run_tree(w, tree_masks):
    return oracle.prefill_tree(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                               w.cu_q_lens, tree_masks, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype,
                               w.scale)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tree_rows_equal_attention_over_context_and_path(dtype):
    rng = np.random.default_rng(60)
    sizes = [1, 7, 23, 64]
    ctx = [0, 40, 17, 100]
    w = W.build([c + n for c, n in zip(ctx, sizes)], 4, 2, 64, dtype, seed=61, n_decode=0,
                q_lens=sizes)
    trees = [random_parents(n, rng) for n in sizes]
    out = run_tree(w, np.concatenate([masks(t) for t in trees]))
    for s, (parents, c) in enumerate(zip(trees, ctx)):
        a = int(w.cu_q_lens[s])
        for i in range(len(parents)):
            visible = list(range(c)) + [c + j for j in path(parents, i)]
            for h in range(w.H_q):
                K = rows_of(w, w.k_cache, s, h // 2, visible)
                V = rows_of(w, w.v_cache, s, h // 2, visible)
                q = oracle.to_double(w.query_prefill[a + i, h], dtype)
                np.testing.assert_allclose(out[a + i, h], sdpa64(q, K, V, w.scale), rtol=1e-12,
                                           atol=1e-13)


def test_chain_tree_equals_causal_prefill_bit_for_bit():
    """A chain (each node the child of the one before) is ordinary causal attention."""
    q_lens = [5, 64, 30]
    w = W.build([12, 64, 600], 8, 2, 128, "bf16", seed=62, n_decode=0, q_lens=q_lens)
    chain = np.array([(1 << (i + 1)) - 1 for n in q_lens for i in range(n)], dtype=np.uint64)
    want = oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                          w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(run_tree(w, chain), want)


def test_star_tree_rows_are_decodes_of_context_plus_own_token():
    """Children of the root only: row i sees the context and itself -- the decode of a sequence
    whose table lists the context blocks and then a block holding only row i's K/V."""
    n, c = 9, 37
    w = W.build([c + n], 4, 4, 64, "f16", seed=63, n_decode=0, q_lens=[n])
    out = run_tree(w, np.array([1 << i for i in range(n)], dtype=np.uint64))
    for i in range(n):
        for h in range(4):
            visible = list(range(c)) + [c + i]
            K = rows_of(w, w.k_cache, 0, h, visible)
            V = rows_of(w, w.v_cache, 0, h, visible)
            q = oracle.to_double(w.query_prefill[i, h], "f16")
            np.testing.assert_allclose(out[i, h], sdpa64(q, K, V, w.scale), rtol=1e-12, atol=1e-13)


def test_mask_bits_above_the_row_are_ignored():
    rng = np.random.default_rng(64)
    n = 20
    w = W.build([50 + n], 4, 2, 64, "bf16", seed=64, n_decode=0, q_lens=[n])
    base = masks(random_parents(n, rng))
    noisy = base.copy()
    for i in range(n):
        noisy[i] |= np.uint64(int(rng.integers(0, 1 << 62)) << (i + 1) & ((1 << 64) - 1))
    assert np.array_equal(run_tree(w, noisy), run_tree(w, base))


def test_row_with_no_visible_key_is_zero():
    """A whole prompt drafted as a tree (no context) and a row whose mask is empty: an empty key
    set gives a zero row, as a zero-length decode does; the other rows are unaffected."""
    n = 6
    w = W.build([n], 2, 2, 64, "f16", seed=65, n_decode=0, q_lens=[n])
    m = masks([-1, 0, 1, -1, 3, 4])
    m[2] = 0
    out = run_tree(w, m)
    assert not out[2].any()
    ref = run_tree(w, masks([-1, 0, 1, -1, 3, 4]))
    assert np.array_equal(np.delete(out, 2, axis=0), np.delete(ref, 2, axis=0))


def test_more_than_64_rows_is_rejected():
    w = W.build([65], 2, 2, 64, "f16", seed=66, n_decode=0, q_lens=[65])
    with pytest.raises(ValueError):
        run_tree(w, np.full(65, (1 << 64) - 1, dtype=np.uint64))
