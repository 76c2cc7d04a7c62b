"""Block pools larger than 4 GiB per cache: every kernel addresses blocks past the 32-bit range.

The workload's physical blocks are relabelled to the top of a pool of more than 4 GiB per cache
(block b becomes b + offset; tables, slots and copy pairs move with it; the blocks below are
never touched). The library then runs the step -- copy_blocks, reshape_and_cache, decode (the
vector-ALU kernel for MHA, the MFMA kernel for GQA), prefill (16-bit and E4M3 caches) -- and its
results must equal the oracle's on the original, small pool: pools word for word at the
relabelled blocks, attention within the gate. Relabelling blocks changes no result (the oracle pins block-relabelling
invariance on the CPU).
"""
import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import ints_to_device, words_from_device, words_to_device
from pa_testutil import assert_attention_close, oracle_pool_after_step

pytestmark = pytest.mark.gpu

GIB = 1 << 30


def shifted(table, off):
    t = np.asarray(table, np.int64)
    return np.where(t >= 0, t + off, t).astype(np.int32)


@pytest.mark.parametrize("H_q,H_kv,dtype", [(8, 8, "f16"), (32, 8, "bf16")])
def test_step_on_blocks_past_4gib(H_q, H_kv, dtype):
    D = 128
    rng = np.random.default_rng(800 + H_q)
    lens = rng.integers(200, 3000, size=12).tolist()
    w = W.build(lens + [1500, 700], H_q, H_kv, D, dtype, seed=801 + H_q, n_decode=12,
                q_lens=[300, 64])
    block_bytes = H_kv * W.BLOCK * D * 2
    off = (4 * GIB + 64 * 1024 * 1024) // block_bytes + 1      # every used block starts past 4 GiB
    nb = w.num_blocks + off
    print(f"[large pool] {nb} blocks = {nb * block_bytes / GIB:.2f} GiB per cache, H_q={H_q} "
          f"H_kv={H_kv} {dtype}", flush=True)
    dev = torch.device("cuda")
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    kc = torch.empty((nb, H_kv, W.BLOCK, D), dtype=tdt, device=dev)
    vc = torch.empty_like(kc)
    kc[off:] = words_to_device(w.k_cache, dtype, dev).view(w.num_blocks, H_kv, W.BLOCK, D)
    vc[off:] = words_to_device(w.v_cache, dtype, dev).view(w.num_blocks, H_kv, W.BLOCK, D)

    pairs = np.asarray(w.copy_pairs, np.int64).reshape(-1, 2) + off
    binding.copy_blocks(kc, vc, ints_to_device(pairs, dev))
    slots = np.asarray(w.slot_mapping, np.int64)
    slots = np.where(slots >= 0, slots + off * W.BLOCK, slots)
    binding.reshape_and_cache(words_to_device(w.new_key, dtype, dev),
                              words_to_device(w.new_value, dtype, dev), kc, vc,
                              ints_to_device(slots, dev))
    nd = w.n_decode
    tables = shifted(w.block_tables, off)
    dec_lens = np.asarray(w.seq_lens[:nd], np.int32)
    max_len = int(dec_lens.max())
    part = binding.default_partition_size(max_len)
    ws = binding.alloc_decode_workspace(nd, H_q, D, max_len, part, dev)
    dq = words_to_device(w.query_decode, dtype, dev)
    dout = torch.empty_like(dq)
    binding.decode(dout, dq, kc, vc, ints_to_device(tables[:nd], dev), ints_to_device(dec_lens, dev),
                   max_len, w.scale, part, ws)
    pq = words_to_device(w.query_prefill, dtype, dev)
    pout = torch.empty_like(pq)
    cu = np.asarray(w.cu_q_lens, np.int32)
    binding.prefill_chunk(pout, pq, kc, vc, ints_to_device(tables[nd:], dev),
                          ints_to_device(w.seq_lens[nd:], dev), ints_to_device(cu, dev),
                          int(np.diff(cu).max()), w.scale)
    torch.cuda.synchronize()

    kr, vr = oracle_pool_after_step(w)
    for got, ref in ((kc, kr), (vc, vr)):
        assert np.array_equal(words_from_device(got[off:]).ravel(), np.asarray(ref).ravel()), \
            "pool past 4 GiB differs from the oracle's"
    ref_d = oracle.decode(w.query_decode, kr, vr, w.block_tables[:nd], w.seq_lens[:nd], H_q, H_kv,
                          D, w.num_blocks, dtype, w.scale)
    assert_attention_close(words_from_device(dout), ref_d, dtype, "decode past 4 GiB", absolute=True)
    ref_p = oracle.prefill(w.query_prefill, kr, vr, w.block_tables[nd:], w.seq_lens[nd:],
                           w.cu_q_lens, H_q, H_kv, D, w.num_blocks, dtype, w.scale)
    assert_attention_close(words_from_device(pout), ref_p, dtype, "prefill past 4 GiB")

    # copy-on-write copies between blocks past 4 GiB: used blocks into free ones
    used = set(int(b) for b in np.asarray(w.block_tables).ravel() if b >= 0)
    free = [b for b in range(w.num_blocks) if b not in used][:4]
    src = sorted(used)[:len(free)]
    cp = np.array(list(zip(src, free)), np.int32).reshape(-1, 2)
    assert len(cp) > 0
    binding.copy_blocks(kc, vc, ints_to_device(cp.astype(np.int64) + off, dev))
    torch.cuda.synchronize()
    kr, vr = oracle.copy_blocks(kr, vr, cp, w.num_blocks, H_kv, D)
    for got, ref in ((kc, kr), (vc, vr)):
        assert np.array_equal(words_from_device(got[off:]).ravel(), np.asarray(ref).ravel()), \
            "copies past 4 GiB differ from the oracle's"


@pytest.mark.parametrize("H_q,H_kv,dtype", [(8, 8, "f16"), (32, 8, "bf16")])
def test_e4m3_step_on_blocks_past_4gib(H_q, H_kv, dtype):
    D, ks, vs = 128, 0.03, 0.02
    w = W.build(np.random.default_rng(810 + H_q).integers(200, 3000, size=12).tolist() + [1500, 700],
                H_q, H_kv, D, dtype, seed=811 + H_q, n_decode=12, q_lens=[300, 64])
    block_bytes = H_kv * W.BLOCK * D
    off = (4 * GIB + 64 * 1024 * 1024) // block_bytes + 1
    nb = w.num_blocks + off
    print(f"[large pool] E4M3 {nb} blocks = {nb * block_bytes / GIB:.2f} GiB per cache, "
          f"H_q={H_q} H_kv={H_kv} {dtype}", flush=True)
    dev = torch.device("cuda")
    k8 = oracle.quantize_e4m3(w.k_cache, dtype, ks)
    v8 = oracle.quantize_e4m3(w.v_cache, dtype, vs)
    kc = torch.empty((nb, H_kv, W.BLOCK, D), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    kc[off:] = torch.from_numpy(k8).to(dev).view(w.num_blocks, H_kv, W.BLOCK, D)
    vc[off:] = torch.from_numpy(v8).to(dev).view(w.num_blocks, H_kv, W.BLOCK, D)
    slots = np.asarray(w.slot_mapping, np.int64)
    slots = np.where(slots >= 0, slots + off * W.BLOCK, slots)
    binding.reshape_and_cache_fp8(words_to_device(w.new_key, dtype, dev),
                                  words_to_device(w.new_value, dtype, dev), kc, vc,
                                  ints_to_device(slots, dev), ks, vs)
    tables = shifted(w.block_tables, off)
    nd = w.n_decode
    lens = np.asarray(w.seq_lens[:nd], np.int32)
    max_len = int(lens.max())
    part = binding.default_partition_size(max_len)
    ws = binding.alloc_decode_workspace(nd, H_q, D, max_len, part, dev)
    dq = words_to_device(w.query_decode, dtype, dev)
    dout = torch.empty_like(dq)
    binding.decode_fp8(dout, dq, kc, vc, ints_to_device(tables[:nd], dev),
                       ints_to_device(lens, dev), max_len, w.scale, ks, vs, part, ws)
    pq = words_to_device(w.query_prefill, dtype, dev)
    pout = torch.empty_like(pq)
    cu = np.asarray(w.cu_q_lens, np.int32)
    binding.prefill_chunk_fp8(pout, pq, kc, vc, ints_to_device(tables[nd:], dev),
                              ints_to_device(w.seq_lens[nd:], dev), ints_to_device(cu, dev),
                              int(np.diff(cu).max()), w.scale, ks, vs)
    torch.cuda.synchronize()
    kr, vr = oracle.reshape_and_cache_fp8(w.new_key, w.new_value, k8, v8, w.slot_mapping,
                                          w.num_blocks, H_kv, D, dtype, ks, vs)
    for got, ref in ((kc, kr), (vc, vr)):
        assert np.array_equal(got[off:].cpu().numpy().ravel(), np.asarray(ref).ravel())
    ref_d = oracle.decode_fp8(w.query_decode, kr, vr, w.block_tables[:nd], w.seq_lens[:nd], H_q,
                              H_kv, D, w.num_blocks, dtype, w.scale, ks, vs)
    assert_attention_close(words_from_device(dout), ref_d, dtype, "E4M3 decode past 4 GiB", absolute=True)
    ref_p = oracle.prefill_fp8(w.query_prefill, kr, vr, w.block_tables[nd:], w.seq_lens[nd:],
                               w.cu_q_lens, H_q, H_kv, D, w.num_blocks, dtype, w.scale, ks, vs)
    assert_attention_close(words_from_device(pout), ref_p, dtype, "E4M3 prefill past 4 GiB")
