"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one oracle function to something the oracle cannot have produced: values the pages
print for a worked example (tests/golden), closed forms of softmax attention, a library routine the
special case reduces to (numpy/torch number decoding, torch's scaled_dot_product_attention in
float64), brute force at 50 digits with mpmath, or an invariant the definition forces (key order,
block relabelling, GQA as replicated MHA). A plausible slip in the oracle -- a dropped term, a wrong
sign or index, a transposed operand -- breaks at least one of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def sdpa64(q, K, V, scale, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU: q [n, D], K, V [L, D]."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None]
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))[None, None]
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m,
                                                            scale=scale)[0, 0].numpy()


def pool4(w, cache):
    """View a flat pool as [block][kv_head][16][D] (the interface layout) with numpy."""
    return np.asarray(cache).reshape(w.num_blocks, w.H_kv, W.BLOCK, w.D)


def contiguous(w, cache, s, kvh, L):
    """Rows 0..L-1 of one sequence and kv head, by numpy fancy indexing of the 4-d pool view."""
    pos = np.arange(L)
    blk = w.block_tables[s][pos // W.BLOCK]
    return oracle.to_double(pool4(w, cache)[blk, kvh, pos % W.BLOCK, :], w.dtype)


# ----------------------------------------------------------------------------- O1: decoding
def test_f16_words_match_numpy_for_all_65536_codes():
    words = np.arange(65536, dtype=np.uint16)
    got = oracle.to_double(words, "f16")
    want = words.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_bf16_words_match_torch_for_all_65536_codes():
    words = np.arange(65536, dtype=np.uint16)
    got = oracle.to_double(words, "bf16")
    want = torch.from_numpy(words.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------------------ O2/O3: scatter, copy
def test_scatter_matches_hand_enumerated_fixture():
    g = golden("scatter_tiny.json")
    n = g["pool_words"]
    kc, vc = oracle.reshape_and_cache(np.array(g["key"]), np.array(g["value"]),
                                      np.zeros(n, np.uint16), np.zeros(n, np.uint16),
                                      g["slot_mapping"], g["num_blocks"], g["H_kv"], g["D"])
    wk, wv = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    for i, x in g["expected_k"].items():
        wk[int(i)] = x
    for i, x in g["expected_v"].items():
        wv[int(i)] = x
    assert np.array_equal(kc, wk) and np.array_equal(vc, wv)


def test_scatter_rejects_duplicate_and_out_of_range_slots():
    key = np.ones((2, 1, 2), np.uint16)
    pool = np.zeros(2 * 16 * 2, np.uint16)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(key, key, pool, pool, [5, 5], 2, 1, 2)
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(key, key, pool, pool, [5, 32], 2, 1, 2)


def test_copy_blocks_matches_hand_enumerated_fixture():
    g = golden("copy_tiny.json")
    k0 = np.arange(48, dtype=np.uint16)
    v0 = (100 + np.arange(48)).astype(np.uint16)
    kc, vc = oracle.copy_blocks(k0, v0, g["mapping"], g["num_blocks"], g["H_kv"], g["D"])
    assert kc.tolist() == g["expected_k"] and vc.tolist() == g["expected_v"]


def test_copy_blocks_rejects_chained_or_duplicate_destinations():
    pool = np.zeros(3 * 16, np.uint16)
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 1], [1, 2]], 3, 1, 1)   # dst 1 is also a src
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 2], [1, 2]], 3, 1, 1)   # dst 2 twice


def test_scatter_then_gather_round_trip_is_bit_exact():
    """I1: every token written through slot_mapping comes back through the block table."""
    w = W.build([37, 16, 1, 50], 4, 2, 64, "f16", seed=11, n_decode=2, q_lens=[1, 50])
    kc, vc = oracle.reshape_and_cache(w.new_key, w.new_value, w.k_cache, w.v_cache,
                                      w.slot_mapping, w.num_blocks, w.H_kv, w.D)
    # the last positions of every sequence are the new tokens, in order
    t = 0
    for s in range(len(w.seq_lens)):
        L = int(w.seq_lens[s])
        n_new = 1 if s < w.n_decode else int(w.cu_q_lens[s - w.n_decode + 1] - w.cu_q_lens[s - w.n_decode])
        for kvh in range(w.H_kv):
            rows = oracle.gather(kc, w.block_tables[s], L, kvh, w.num_blocks, w.H_kv, w.D, w.dtype)
            want = oracle.to_double(w.new_key[t:t + n_new, kvh, :], w.dtype)
            assert np.array_equal(rows[L - n_new:], want)
        t += n_new
    assert t == len(w.slot_mapping)
    # words of slots not written are unchanged
    changed = np.flatnonzero(kc != w.k_cache)
    touched = set()
    for slot in w.slot_mapping:
        for kvh in range(w.H_kv):
            base = ((slot // 16 * w.H_kv + kvh) * 16 + slot % 16) * w.D
            touched.update(range(base, base + w.D))
    assert set(changed.tolist()) <= touched


def test_gather_matches_numpy_view_of_layout():
    w = W.build([45, 3], 2, 2, 64, "bf16", seed=12)
    for s in range(2):
        for kvh in range(2):
            L = int(w.seq_lens[s])
            a = oracle.gather(w.v_cache, w.block_tables[s], L, kvh, w.num_blocks, w.H_kv, w.D, w.dtype)
            assert np.array_equal(a, contiguous(w, w.v_cache, s, kvh, L))


# --------------------------------------------------------------------------- O5: closed forms
rng = np.random.default_rng(2024)


def test_single_key_returns_its_value_exactly():
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(oracle.attention(q, K, V, 0.3), V[0])


def test_equal_values_return_that_value():
    c = rng.standard_normal(16)
    out = oracle.attention(rng.standard_normal(16), rng.standard_normal((9, 16)), np.tile(c, (9, 1)), 0.25)
    assert np.allclose(out, c, rtol=0, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    V = rng.standard_normal((7, 4))
    out = oracle.attention(np.zeros(4), rng.standard_normal((7, 4)), V, 1.0)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-15)


def test_two_keys_give_logistic_weights():
    q, K, V = rng.standard_normal(5), rng.standard_normal((2, 5)), rng.standard_normal((2, 5))
    scale = 0.7
    d = scale * (q @ K[0] - q @ K[1])
    w0 = 1.0 / (1.0 + math.exp(-d))
    assert np.allclose(oracle.attention(q, K, V, scale), w0 * V[0] + (1 - w0) * V[1], atol=1e-15)


def test_hardmax_limit_picks_best_key():
    q = rng.standard_normal(6)
    K = rng.standard_normal((5, 6))
    V = rng.standard_normal((5, 6))
    out = oracle.attention(q, K, V, 1e4)
    assert np.allclose(out, V[np.argmax(K @ q)], atol=1e-12)


def test_common_key_shift_and_value_affine_map():
    q, K, V = rng.standard_normal(8), rng.standard_normal((11, 8)), rng.standard_normal((11, 8))
    base = oracle.attention(q, K, V, 0.5)
    shifted = oracle.attention(q, K + rng.standard_normal(8), V, 0.5)
    assert np.allclose(base, shifted, atol=1e-13)
    c = rng.standard_normal(8)
    assert np.allclose(oracle.attention(q, K, 3.0 * V + c, 0.5), 3.0 * base + c, atol=1e-13)


def test_key_order_does_not_matter():
    q, K, V = rng.standard_normal(8), rng.standard_normal((13, 8)), rng.standard_normal((13, 8))
    p = rng.permutation(13)
    assert np.allclose(oracle.attention(q, K, V, 0.4), oracle.attention(q, K[p], V[p], 0.4), atol=1e-14)


def test_empty_context_gives_zeros():
    assert np.array_equal(oracle.attention(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0), np.zeros(4))


@pytest.mark.parametrize("L,D", [(1, 1), (2, 3), (3, 2), (5, 4)])
def test_attention_matches_50_digit_brute_force(L, D):
    mpmath.mp.dps = 50
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    scale = 1 / math.sqrt(D)
    s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[d]) * mpmath.mpf(K[j, d]) for d in range(D))
         for j in range(L)]
    e = [mpmath.exp(x) for x in s]
    Z = mpmath.fsum(e)
    want = [float(mpmath.fsum(e[j] * mpmath.mpf(V[j, d]) for j in range(L)) / Z) for d in range(D)]
    got = oracle.attention(q, K, V, scale)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("L", [1, 17, 300])
def test_attention_matches_torch_sdpa_float64(L):
    D = 64
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    got = oracle.attention(q, K, V, 0.125)
    assert np.allclose(got, sdpa64(q[None], K, V, 0.125)[0], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------ O8: split and merge
@pytest.mark.parametrize("part", [1, 3, 16, 48, 512, 1000, 1037])
def test_split_merge_equals_unsplit(part):
    L, D = 1000, 32
    q, K, V = rng.standard_normal(D), 2 * rng.standard_normal((L, D)), rng.standard_normal((L, D))
    a = oracle.attention(q, K, V, 0.3)
    b = oracle.split_merge(q, K, V, 0.3, part)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_split_merge_two_parts_by_hand():
    """Two single-key parts: the merge must weight part p by exp(m_p - M) * Z_p with Z_p = 1."""
    q = np.array([1.0, 0.0])
    K = np.array([[2.0, 0.0], [0.0, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    e2 = math.exp(2.0)
    assert np.allclose(oracle.split_merge(q, K, V, 1.0, 1), [e2 / (e2 + 1), 1 / (e2 + 1)], atol=1e-15)


# ------------------------------------------------------------------------------ O6: paged decode
def test_decode_matches_sdpa_on_layout_gathered_rows():
    w = W.build([1, 7, 16, 33, 100], 4, 4, 64, "f16", seed=21)
    out = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                        w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    for s, L in enumerate(w.seq_lens):
        for h in range(w.H_q):
            K = contiguous(w, w.k_cache, s, h, int(L))
            V = contiguous(w, w.v_cache, s, h, int(L))
            q = oracle.to_double(w.query_decode[s, h], w.dtype)
            assert np.allclose(out[s, h], sdpa64(q[None], K, V, w.scale)[0], rtol=1e-12, atol=1e-13)


def test_decode_single_token_returns_its_value():
    w = W.tiny_decode()
    out = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                        w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    assert w.seq_lens[0] == 1
    for h in range(w.H_q):
        assert np.array_equal(out[0, h], contiguous(w, w.v_cache, 0, h, 1)[0])


def relabel(w, perm):
    """The same logical content under a different physical block assignment: block b -> perm[b]."""
    kc = np.empty_like(pool4(w, w.k_cache))
    vc = np.empty_like(kc)
    kc[perm] = pool4(w, w.k_cache)
    vc[perm] = pool4(w, w.v_cache)
    bt = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    return kc.ravel(), vc.ravel(), bt


def test_decode_is_invariant_under_block_relabelling():
    """I2: paged results do not depend on which physical blocks hold the logical ones."""
    w = W.build([5, 64, 129], 8, 2, 64, "bf16", seed=22)
    a = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                      w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    kc, vc, bt = relabel(w, np.random.default_rng(5).permutation(w.num_blocks))
    b = oracle.decode(w.query_decode, kc, vc, bt, w.seq_lens, w.H_q, w.H_kv, w.D, w.num_blocks,
                      w.dtype, w.scale)
    assert np.array_equal(a, b)


def test_gqa_equals_mha_with_replicated_kv_heads():
    """I9: a group of query heads over one kv head is MHA over copies of that kv head."""
    w = W.build([20, 77], 8, 2, 64, "f16", seed=23)
    gqa = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                        8, 2, 64, w.num_blocks, w.dtype, w.scale)
    kc = np.repeat(pool4(w, w.k_cache), 4, axis=1).ravel()
    vc = np.repeat(pool4(w, w.v_cache), 4, axis=1).ravel()
    mha = oracle.decode(w.query_decode, kc, vc, w.block_tables, w.seq_lens, 8, 8, 64,
                        w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(gqa, mha)


def test_gqa_head_map_follows_page_figure():
    g = golden("page_worked_examples.json")["gqa_figure"]
    w = W.build([33], g["H_q"], g["H_kv"], 8, "f16", seed=24)
    v = pool4(w, w.v_cache).copy()
    for kvh in range(g["H_kv"]):
        v[:, kvh] = W.f32_to_words(np.full(v[:, kvh].shape, float(kvh + 1), np.float32), "f16")
    out = oracle.decode(w.query_decode, w.k_cache, v.ravel(), w.block_tables, w.seq_lens,
                        g["H_q"], g["H_kv"], 8, w.num_blocks, w.dtype, w.scale)
    got = [int(round(out[0, h, 0])) - 1 for h in range(g["H_q"])]
    assert got == g["kv_head_of_q_head"]


def test_decode_zero_length_gives_zeros_and_pair_selection_matches_full():
    w = W.build([0, 40], 2, 2, 64, "f16", seed=25)
    full = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                         2, 2, 64, w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(full[0], np.zeros((2, 64)))
    sel = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                        2, 2, 64, w.num_blocks, w.dtype, w.scale, pairs=[[1, 1], [1, 0]])
    assert np.array_equal(sel, full[1, ::-1])


# ----------------------------------------------------------------------------- O7: prefill
def test_prefill_rows_equal_full_causal_attention_rows():
    """I8: chunk rows are the matching rows of causal attention over the whole sequence, computed
    by torch's sdpa with an explicit mask (row at position p sees keys 0..p)."""
    w = W.build([50, 37], 4, 2, 64, "bf16", seed=31, n_decode=0, q_lens=[20, 37])
    out = oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                         w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    for s in range(2):
        L = int(w.seq_lens[s])
        a, b = int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])
        qlen = b - a
        for h in range(w.H_q):
            K = contiguous(w, w.k_cache, s, h // 2, L)
            V = contiguous(w, w.v_cache, s, h // 2, L)
            q = oracle.to_double(w.query_prefill[a:b, h], w.dtype)
            pos = np.arange(L - qlen, L)
            mask = np.arange(L)[None, :] <= pos[:, None]
            want = sdpa64(q, K, V, w.scale, mask)
            assert np.allclose(out[a:b, h], want, rtol=1e-12, atol=1e-13)


def test_prefill_first_row_of_full_prompt_sees_only_itself():
    w = W.build([21], 2, 2, 64, "f16", seed=32, n_decode=0, q_lens=[21])
    out = oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                         w.cu_q_lens, 2, 2, 64, w.num_blocks, w.dtype, w.scale)
    for h in range(2):
        assert np.array_equal(out[0, h], contiguous(w, w.v_cache, 0, h, 1)[0])


def test_prefill_last_row_equals_decode_at_same_length():
    w = W.build([70], 4, 2, 64, "f16", seed=33, n_decode=0, q_lens=[9])
    pre = oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                         w.cu_q_lens, 4, 2, 64, w.num_blocks, w.dtype, w.scale)
    dec = oracle.decode(w.query_prefill[-1:], w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                        4, 2, 64, w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(pre[-1], dec[0])


def test_multi_token_rows_equal_decode_at_each_cut_length():
    """I8 for k-token steps (speculative verification): row i of a k-row chunk of a length-L
    sequence is the decode of the sequence cut to L - k + 1 + i tokens, bit for bit."""
    k = [2, 5, 8]
    w = W.build([40, 17, 8], 4, 2, 64, "bf16", seed=34, n_decode=0, q_lens=k)
    pre = oracle.prefill(w.query_prefill, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                         w.cu_q_lens, 4, 2, 64, w.num_blocks, w.dtype, w.scale)
    tables, cut = [], []
    for s, ks in enumerate(k):
        for i in range(ks):
            tables.append(w.block_tables[s])
            cut.append(int(w.seq_lens[s]) - ks + 1 + i)
    dec = oracle.decode(w.query_prefill, w.k_cache, w.v_cache, np.asarray(tables, np.int32),
                        np.asarray(cut, np.int32), 4, 2, 64, w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(pre, dec)


# ---------------------------------------------------------------------- poison helper
def test_poison_touches_only_free_slots():
    w = W.build([17, 3], 2, 2, 64, "f16", seed=41)
    kc, vc = oracle.poison_free_slots(w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                                      w.num_blocks, w.H_kv, w.D, w.dtype)
    a = oracle.decode(w.query_decode, w.k_cache, w.v_cache, w.block_tables, w.seq_lens,
                      2, 2, 64, w.num_blocks, w.dtype, w.scale)
    b = oracle.decode(w.query_decode, kc, vc, w.block_tables, w.seq_lens,
                      2, 2, 64, w.num_blocks, w.dtype, w.scale)
    assert np.array_equal(a, b)
    n_used = 17 + 3
    assert (pool4(w, kc)[..., 0] == oracle.NAN_WORD["f16"]).sum() == (w.num_blocks * 16 - n_used) * 2
