"""Multi-token decode on the GPU: each sequence appends k = 2..8 tokens in one step (the draft
tokens a speculative step verifies) and every new token attends its causal prefix. The step runs
through pa_prefill_chunk with one k-row chunk per sequence (lecture 32 "LLM 在线推理两阶段" §5.4,
speculative decoding: the target model checks the k drafted tokens in one parallel pass; the causal
rule of §2 gives row i the keys up to its own position).

Gate: every row equals a one-token decode of its sequence cut at that row's position, computed by
the oracle; the same cut sequences also go through the GPU decode kernel, so both GPU paths are held
to the same expected values.
"""
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import GpuStep, words_from_device
from pa_testutil import assert_attention_close, oracle_pool_after_step

pytestmark = pytest.mark.gpu


def per_row_decode_view(w):
    """The chunk rows as independent decodes: row i of a k-row chunk of a length-L sequence is a
    decode of length L - k + 1 + i over the same block table."""
    nd = w.n_decode
    tables, lens = [], []
    for s in range(len(w.seq_lens) - nd):
        L = int(w.seq_lens[nd + s])
        a, b = int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1])
        for i in range(b - a):
            tables.append(w.block_tables[nd + s])
            lens.append(L - (b - a) + 1 + i)
    return np.asarray(tables, np.int32), np.asarray(lens, np.int32)


@pytest.mark.parametrize("H_q,H_kv,D,dtype", [(32, 32, 128, "f16"), (32, 8, 128, "bf16"),
                                               (64, 8, 128, "bf16"), (8, 8, 64, "f16"),
                                               (16, 4, 64, "bf16")])
def test_multi_token_rows_equal_per_row_decode(H_q, H_kv, D, dtype):
    rng = np.random.default_rng(400 + H_q + D)
    n = 40
    k = rng.integers(2, 9, size=n)
    lens = np.maximum(rng.integers(1, 3000, size=n), k)
    lens[:4] = k[:4]                      # whole prompts of k tokens: first row sees one key
    lens[4:8] = 16 * rng.integers(1, 20, size=4) + k[4:8] - 1   # rows straddle a block edge
    w = W.build(lens.tolist(), H_q, H_kv, D, dtype, seed=410 + H_q + D, n_decode=0,
                q_lens=k.tolist())
    print(f"[multi-token] {n} sequences, k in [{k.min()}, {k.max()}], {int(k.sum())} rows, "
          f"H_q={H_q} H_kv={H_kv} D={D} {dtype}", flush=True)
    g = GpuStep(w, multi_token=False)   # the chunk kernel (pa_decode_multi has its own tests)
    assert not g.multi_token
    g.scatter()
    g.prefill()
    torch.cuda.synchronize()
    got = words_from_device(g.pre_out)

    kc, vc = oracle_pool_after_step(w)
    tables, cut = per_row_decode_view(w)
    ref = oracle.decode(w.query_prefill, kc, vc, tables, cut, H_q, H_kv, D, w.num_blocks, dtype,
                        w.scale)
    assert_attention_close(got, ref, dtype, f"multi-token rows H_q={H_q} H_kv={H_kv} D={D}")

    # the same rows as one-token decodes on the GPU (pool after this step's scatter)
    dec = GpuStep(w)
    dec.scatter()
    tables_d = torch.from_numpy(tables).to(dec.device)
    lens_d = torch.from_numpy(cut).to(dec.device)
    max_len = int(cut.max())
    part = binding.default_partition_size(max_len)
    ws = binding.alloc_decode_workspace(len(cut), H_q, D, max_len, part, dec.device)
    out = torch.empty_like(dec.pre_query)
    binding.decode(out, dec.pre_query, dec.k_cache, dec.v_cache, tables_d, lens_d, max_len,
                   w.scale, part, ws)
    torch.cuda.synchronize()
    assert_attention_close(words_from_device(out), ref, dtype, "per-row GPU decode")
