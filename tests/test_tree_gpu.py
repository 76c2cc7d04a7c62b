"""Drafted-token trees on the GPU: pa_prefill_chunk_tree against the oracle's tree-masked prefill.

Lecture 34 "vLLM 生产级系统架构全景剖析" §5.3: a tree of drafted tokens (EAGLE) is verified in one
pass of the target model, each drafted token seeing the context and its own path from the root.
Each sequence appends its drafted tokens (1..64) as one chunk; row i's mask holds row i and its
ancestors. Gates: every row within the attention gate of the float64 oracle on the pool after the
step's scatter; chain trees equal pa_prefill_chunk bit for bit (same kernel arithmetic, the mask
only removes keys); repeated calls are bitwise identical; more than 64 rows is refused on the host.
"""
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import GpuStep, words_from_device
from pa_testutil import assert_attention_close, oracle_pool_after_step, random_parents, tree_masks

pytestmark = pytest.mark.gpu


def tree_workload(H_q, H_kv, D, dtype, seed, n_seqs=24, long_ctx=True):
    rng = np.random.default_rng(seed)
    sizes = rng.integers(1, 65, size=n_seqs)
    sizes[:3] = [64, 1, 33]
    ctx = rng.integers(0, 500, size=n_seqs)
    if long_ctx:
        ctx[n_seqs // 2:] = rng.integers(512, 3000, size=n_seqs - n_seqs // 2)  # pipelined loop
    ctx[1] = 0                                      # a whole prompt drafted as a tree
    ctx[2] = 16 * 7                                 # the tree starts on a block edge
    w = W.build((ctx + sizes).tolist(), H_q, H_kv, D, dtype, seed=seed + 1, n_decode=0,
                q_lens=sizes.tolist())
    trees = [random_parents(int(n), rng) for n in sizes]
    return w, np.concatenate([tree_masks(t) for t in trees])


def run_tree(w, masks):
    g = GpuStep(w)
    g.scatter()
    tm = torch.from_numpy(np.ascontiguousarray(masks).view(np.int64)).to(g.device)
    binding.prefill_chunk(g.pre_out, g.pre_query, g.k_cache, g.v_cache, g.pre_tables, g.pre_lens,
                          g.pre_cu, g.max_q_len, w.scale, tree_mask=tm)
    torch.cuda.synchronize()
    return g, tm


@pytest.mark.parametrize("H_q,H_kv,D,dtype", [(32, 32, 128, "f16"), (32, 8, 128, "bf16"),
                                               (64, 8, 128, "bf16"), (8, 8, 64, "f16"),
                                               (16, 4, 64, "bf16"), (12, 4, 128, "f16")])
def test_tree_rows_match_oracle(H_q, H_kv, D, dtype):
    w, masks = tree_workload(H_q, H_kv, D, dtype, seed=700 + H_q + D)
    print(f"[tree] {len(w.seq_lens)} trees, {len(masks)} rows, H_q={H_q} H_kv={H_kv} D={D} "
          f"{dtype}", flush=True)
    g, _ = run_tree(w, masks)
    kc, vc = oracle_pool_after_step(w)
    ref = oracle.prefill_tree(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                              masks, H_q, H_kv, D, w.num_blocks, dtype, w.scale)
    assert_attention_close(words_from_device(g.pre_out), ref, dtype,
                           f"tree rows H_q={H_q} H_kv={H_kv} D={D} {dtype}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_chain_tree_equals_causal_chunk_bit_for_bit(dtype):
    w, _ = tree_workload(32, 8, 128, dtype, seed=720)
    cu = np.asarray(w.cu_q_lens)
    chain = np.array([(1 << (i + 1)) - 1 for s in range(len(cu) - 1) for i in range(cu[s + 1] - cu[s])],
                     dtype=np.uint64)
    print(f"[tree] chain trees vs causal chunk, {dtype}", flush=True)
    g, _ = run_tree(w, chain)
    c = GpuStep(w)
    c.scatter()
    c.prefill()
    torch.cuda.synchronize()
    assert np.array_equal(words_from_device(g.pre_out), words_from_device(c.pre_out))


def test_tree_is_deterministic():
    w, masks = tree_workload(64, 8, 128, "bf16", seed=730)
    print("[tree] determinism", flush=True)
    g, tm = run_tree(w, masks)
    first = words_from_device(g.pre_out)
    binding.prefill_chunk(g.pre_out, g.pre_query, g.k_cache, g.v_cache, g.pre_tables, g.pre_lens,
                          g.pre_cu, g.max_q_len, w.scale, tree_mask=tm)
    torch.cuda.synchronize()
    assert np.array_equal(first, words_from_device(g.pre_out))


def test_more_than_64_rows_is_refused_without_launch():
    w, masks = tree_workload(8, 8, 64, "f16", seed=740, n_seqs=4, long_ctx=False)
    g = GpuStep(w)
    tm = torch.from_numpy(masks.view(np.int64)).to(g.device)
    before = g.pre_out.clone()
    with pytest.raises(binding.PAError):
        binding.prefill_chunk(g.pre_out, g.pre_query, g.k_cache, g.v_cache, g.pre_tables,
                              g.pre_lens, g.pre_cu, 65, w.scale, tree_mask=tm)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), g.pre_out.view(torch.int16))
