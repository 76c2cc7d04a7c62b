"""pa_decode_noalloc (no workspace, partial results in the library's static scratch) against
pa_decode with a caller's workspace, through the C ABI: calls in a row on one GPU, the later ones
with smaller inputs than the first (so the scratch still holds the first call's partials beyond
what they write). The two entry points run the same kernels on the same layout: outputs are compared bit
for bit, and both against the float64 oracle."""
import numpy as np
import pytest
import torch

import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import GpuStep, words_from_device
from pa_testutil import assert_attention_close, oracle_decode, oracle_pool_after_step

pytestmark = pytest.mark.gpu


def decode_both(w, partition_size):
    g = GpuStep(w, partition_size=partition_size)
    g.scatter()
    print(f"[no-alloc] {w.name}: B={w.n_decode} H_q={w.H_q} H_kv={w.H_kv} D={w.D} {w.dtype} "
          f"max_seq_len={g.max_seq_len} partition={partition_size}", flush=True)
    g.decode()  # pa_decode, workspace from the caller
    ref_out = torch.empty_like(g.dec_out)
    binding.decode_noalloc(ref_out, g.dec_query, g.k_cache, g.v_cache, g.dec_tables, g.dec_lens,
                           g.max_seq_len, w.scale, partition_size)
    torch.cuda.synchronize()
    return g, words_from_device(g.dec_out), words_from_device(ref_out)


def test_noalloc_decode_equals_decode_on_two_calls():
    calls = [
        # 70B-like head groups (MFMA kernel, four parts per scratch slot): 2.2 MB of partials
        W.build([3000, 17, 2500, 900, 1999, 4000, 1, 2048], 32, 4, 128, "bf16", seed=901),
        # then smaller inputs: head groups of 32 (two MFMA column groups per wave, four parts per
        # slot): 0.27 MB of partials
        W.build([2000, 37, 1500, 800], 64, 2, 128, "bf16", seed=904),
        # the vector-ALU kernel (one part per slot): 0.4 MB of partials
        W.build([600, 1100, 5, 700], 16, 16, 64, "f16", seed=902),
    ]
    for i, w in enumerate(calls):
        g, with_ws, no_alloc = decode_both(w, 256)
        assert np.array_equal(with_ws, no_alloc), f"call {i}: pa_decode_noalloc differs from pa_decode"
        kc, vc = oracle_pool_after_step(w)
        assert_attention_close(no_alloc, oracle_decode(w, kc, vc), w.dtype,
                               f"pa_decode_noalloc call {i}")


def test_noalloc_decode_unsplit_and_oversized():
    """Unsplit decodes need no scratch; shapes whose partials exceed the scratch are refused on the
    host before anything is enqueued."""
    w = W.build([40, 300, 1], 8, 8, 128, "f16", seed=903)
    g, with_ws, no_alloc = decode_both(w, 0)
    assert np.array_equal(with_ws, no_alloc)
    # 512 sequences x 8 heads (head groups of 1: one part per slot) x 64 parts of 512 tokens x
    # 130 floats = 136 MB of partials
    B, H = 512, 8
    used = B * H * 64 * (128 + 2) * 4
    assert used > binding.DECODE_SCRATCH_BYTES
    q = torch.empty((B, H, 128), dtype=torch.float16, device="cuda")
    tables = torch.zeros((B, 2048), dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.PAError) as e:
        binding.decode_noalloc(q, q, g.k_cache, g.v_cache, tables, lens, 32768, w.scale, 512)
    assert e.value.status == binding.PA_ERR_WORKSPACE
