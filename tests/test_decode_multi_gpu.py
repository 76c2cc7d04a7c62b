"""Multi-token decode (pa_decode_multi, pa_decode_multi_fp8) on the GPU against the oracle.

Lecture 32 "LLM 在线推理两阶段" §5.4 (speculative decoding): the target model checks the k drafted
tokens of a sequence in one pass, each seeing the context and the drafts before it; lecture 34
"vLLM 生产级系统架构全景剖析" §5.3: a draft tree is checked the same way, each token seeing its own
path from the root. Each sequence appends k = 1..16 tokens in one step; the rows are read like a
decode (the MFMA decode kernel over (row, query head) columns, split-K with a log-sum-exp merge).

Gates: every row within the attention gate of the float64 oracle's chunked prefill (O7) or its
tree-masked prefill (T1) on the pool after the step's scatter; over E4M3 caches, the oracle's E4M3
prefill (F7), and for trees T1 over the dequantized pool (scales are powers of two, so every
code times its scale is an exact 16-bit word). Chain-shaped trees give the causal rows' bits;
repeated calls are bitwise identical; split and unsplit calls both meet the gate.
"""
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import GpuStep, words_from_device
from pa_testutil import (assert_attention_close, oracle_fp8_after_step, oracle_fp8_pool,
                         oracle_pool_after_step, random_parents, tree_masks)

pytestmark = pytest.mark.gpu

SHAPES = [(32, 32, 128, "f16"), (32, 8, 128, "bf16"), (64, 8, 128, "bf16"), (8, 8, 64, "f16"),
          (16, 4, 64, "bf16"), (12, 4, 128, "f16"), (6, 2, 128, "bf16")]


def multi_workload(H_q, H_kv, D, dtype, seed, n=40, k_max=16):
    rng = np.random.default_rng(seed)
    k = rng.integers(1, k_max + 1, size=n)
    k[:3] = [k_max, 1, 2]
    lens = np.maximum(rng.integers(1, 9000, size=n), k)
    lens[:4] = k[:4]                                  # whole prompts: the first row sees one key
    lens[4:8] = 16 * rng.integers(1, 40, size=4) + k[4:8] - 1   # rows straddle a block edge
    lens[8] = 2048 * 3 + k[8]                          # rows start on a slot edge
    w = W.build(lens.tolist(), H_q, H_kv, D, dtype, seed=seed + 1, n_decode=0, q_lens=k.tolist())
    return w, k


def run_multi(g, w, part=None, tree=None, fp8=None):
    binding.decode_multi(g.pre_out, g.pre_query, g.k_cache, g.v_cache, g.pre_tables, g.pre_lens,
                         g.pre_cu, g.max_q_len, int(np.max(w.seq_lens)), w.scale,
                         partition_size=part, tree_mask=tree,
                         k_scale=None if fp8 is None else fp8[0],
                         v_scale=None if fp8 is None else fp8[1])
    torch.cuda.synchronize()
    return words_from_device(g.pre_out)


def step(w, **kw):
    g = GpuStep(w, **kw)
    g.scatter()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("H_q,H_kv,D,dtype", SHAPES)
@pytest.mark.parametrize("part", [None, 0, 128])
def test_rows_match_oracle(H_q, H_kv, D, dtype, part):
    w, k = multi_workload(H_q, H_kv, D, dtype, seed=1100 + H_q + D)
    print(f"[multi] {len(k)} sequences, {int(k.sum())} rows, H_q={H_q} H_kv={H_kv} D={D} {dtype} "
          f"part={part}", flush=True)
    got = run_multi(step(w), w, part)
    kc, vc = oracle_pool_after_step(w)
    ref = oracle.prefill(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens, H_q,
                         H_kv, D, w.num_blocks, dtype, w.scale)
    assert_attention_close(got, ref, dtype, f"multi-token rows H_q={H_q} H_kv={H_kv} D={D} "
                                            f"part={part}")


@pytest.mark.parametrize("H_q,H_kv,D,dtype", SHAPES)
def test_tree_rows_match_oracle(H_q, H_kv, D, dtype):
    w, k = multi_workload(H_q, H_kv, D, dtype, seed=1200 + H_q + D)
    rng = np.random.default_rng(1300 + H_q)
    masks = np.concatenate([tree_masks(random_parents(int(n), rng)) for n in k])
    print(f"[multi] trees, {int(k.sum())} rows, H_q={H_q} H_kv={H_kv} D={D} {dtype}", flush=True)
    g = step(w)
    tm = torch.from_numpy(masks.view(np.int64)).to(g.device)
    got = run_multi(g, w, tree=tm)
    kc, vc = oracle_pool_after_step(w)
    ref = oracle.prefill_tree(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                              masks, H_q, H_kv, D, w.num_blocks, dtype, w.scale)
    assert_attention_close(got, ref, dtype, f"multi-token tree rows H_q={H_q} H_kv={H_kv} D={D}")


def test_chain_trees_equal_causal_rows_bit_for_bit():
    w, k = multi_workload(32, 8, 128, "bf16", seed=1400)
    chain = np.concatenate([np.array([(1 << (i + 1)) - 1 for i in range(n)], np.uint64)
                            for n in k])
    print("[multi] chain trees vs causal rows", flush=True)
    g = step(w)
    causal = run_multi(g, w)
    tm = torch.from_numpy(chain.view(np.int64)).to(g.device)
    assert np.array_equal(run_multi(g, w, tree=tm), causal)
    assert np.array_equal(run_multi(g, w), causal)   # repeated calls: the same bits


@pytest.mark.parametrize("H_q,H_kv,D,dtype", [(32, 8, 128, "bf16"), (16, 16, 64, "f16"),
                                               (64, 8, 128, "f16")])
def test_e4m3_rows_match_oracle(H_q, H_kv, D, dtype):
    ks, vs = 2.0 ** -5, 2.0 ** -6
    w, k = multi_workload(H_q, H_kv, D, dtype, seed=1500 + H_q + D)
    kc, vc = oracle_fp8_pool(w, ks, vs, poison=True)
    g = step(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc))
    kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
    print(f"[multi] E4M3 caches, {int(k.sum())} rows, H_q={H_q} H_kv={H_kv} D={D} {dtype}",
          flush=True)
    got = run_multi(g, w, fp8=(ks, vs))
    ref = oracle.prefill_fp8(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                             H_q, H_kv, D, w.num_blocks, dtype, w.scale, ks, vs)
    assert_attention_close(got, ref, dtype, f"multi-token E4M3 rows H_q={H_q} D={D}")

    # trees over the same E4M3 caches, against T1 over the dequantized (exact) 16-bit pool
    rng = np.random.default_rng(1600 + H_q)
    masks = np.concatenate([tree_masks(random_parents(int(n), rng)) for n in k])
    tm = torch.from_numpy(masks.view(np.int64)).to(g.device)
    got = run_multi(g, w, tree=tm, fp8=(ks, vs))

    def dequantized(codes, scale):
        x = oracle.e4m3_to_double(np.arange(256, dtype=np.uint8)) * scale
        fin = np.isfinite(x)
        words = np.full(256, oracle.NAN_WORD[dtype], np.uint16)  # the two NaN codes
        words[fin] = W.f32_to_words(x[fin].astype(np.float32), dtype)
        assert (oracle.to_double(words[fin], dtype) == x[fin]).all(), \
            "a scaled E4M3 value is not an exact 16-bit word"
        return words[np.asarray(codes, np.uint8)]

    ref = oracle.prefill_tree(w.query_prefill, dequantized(kc, ks), dequantized(vc, vs),
                              w.block_tables, w.seq_lens, w.cu_q_lens, masks, H_q, H_kv, D,
                              w.num_blocks, dtype, w.scale)
    assert_attention_close(got, ref, dtype, f"multi-token E4M3 tree rows H_q={H_q} D={D}")


def test_bad_arguments_are_refused_without_launch():
    w, k = multi_workload(8, 8, 64, "f16", seed=1700, n=10, k_max=4)
    g = step(w)
    before = g.pre_out.clone()
    with pytest.raises(binding.PAError):   # more than 16 rows per sequence
        binding.decode_multi(g.pre_out, g.pre_query, g.k_cache, g.v_cache, g.pre_tables,
                             g.pre_lens, g.pre_cu, 17, int(np.max(w.seq_lens)), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), g.pre_out.view(torch.int16))


@pytest.mark.parametrize("part", [0, 16, 512])
def test_rows_that_see_no_position_are_zero(part):
    """Drafted trees with no context whose masks leave some rows nothing to see (their own bit
    cleared): those rows are zeros, split or not, like T1's empty rows; the rest meet the gate."""
    k = [6, 16, 5, 9]
    lens = [6, 16, 3000, 700]             # the first two trees are whole prompts
    w = W.build(lens, 16, 4, 128, "bf16", seed=1800, n_decode=0, q_lens=k)
    rng = np.random.default_rng(1801)
    masks = [tree_masks(random_parents(n, rng)) for n in k]
    masks[0][[0, 3]] = 0                   # rows 0 and 3 of the first tree see nothing
    masks[1][5] &= ~np.uint64(1 << 5)      # row 5 of the second keeps only its ancestors
    masks[1][0] = 0
    masks = np.concatenate(masks)
    print(f"[multi] empty rows, part={part}", flush=True)
    g = step(w)
    tm = torch.from_numpy(masks.view(np.int64)).to(g.device)
    got = run_multi(g, w, part=part, tree=tm)
    kc, vc = oracle_pool_after_step(w)
    ref = oracle.prefill_tree(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                              masks, 16, 4, 128, w.num_blocks, "bf16", w.scale)
    empty = [0, 3, 6]                      # rows of the first two sequences (cu_q = 0, 6, ...)
    assert not np.any(ref[empty]), "the oracle's empty rows are zeros"
    assert not np.any(got.reshape(ref.shape)[empty]), "empty rows must be written as zeros"
    assert_attention_close(got, ref, "bf16", f"multi-token rows with empty views, part={part}")


# ------------------------------------------------------------- the speculative benchmark workloads
@pytest.mark.parametrize("name,kv", [("llama2_7b_spec4", "auto"), ("llama2_7b_spec4", "fp8"),
                                     ("llama70b_gqa_spec4", "auto"), ("llama70b_gqa_spec4", "fp8")])
def test_speculative_workload_full(name, kv):
    """The benchmark's speculative steps at full size, in the launch configuration bench.py times
    (GpuStep picks pa_decode_multi and its partition itself): every drafted row, every head,
    against the oracle's prefill rows on the pool after the step's scatter."""
    w = W.named(name)
    print(f"[multi] {name} {kv}: {len(w.seq_lens)} sequences, {int(w.cu_q_lens[-1])} rows",
          flush=True)
    if kv == "fp8":
        ks, vs = 0.03, 0.02
        kc, vc = oracle_fp8_pool(w, ks, vs, poison=False)
        g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc))
    else:
        g = GpuStep(w)
    assert g.multi_token and g.n_decode == 0
    g.run()
    torch.cuda.synchronize()
    got = words_from_device(g.pre_out)
    if kv == "fp8":
        kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
        ref = oracle.prefill_fp8(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                                 w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, ks, vs)
    else:
        kc, vc = oracle_pool_after_step(w)
        ref = oracle.prefill(w.query_prefill, kc, vc, w.block_tables, w.seq_lens, w.cu_q_lens,
                             w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale)
    assert_attention_close(got, ref, w.dtype, f"speculative step {name} {kv}", absolute=True)
