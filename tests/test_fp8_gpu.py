"""FP8 (E4M3) KV cache on the GPU against the oracle (lecture 34 "vLLM 生产级系统架构全景剖析"
§4.4: kv_cache_dtype="fp8", one byte per key and value element).

Gates: after the quantizing scatter and copy_blocks every byte of both caches equals the oracle's
(all 65536 16-bit codes of each type go through the scatter at several scales, NaN, infinity,
subnormal and saturating inputs included); the E4M3 decode is within the attention gate (2e-3
absolute, 1e-2 row-normwise) of the oracle's decode of the same codes, bitwise reproducible, and
never reads a slot outside a sequence's context (such slots hold the NaN code).
"""
import time

import numpy as np
import pytest
import torch

import oracle
import pa_workloads as W
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.step import GpuStep, words_from_device, words_to_device
from pa_testutil import assert_attention_close, oracle_fp8_after_step, oracle_fp8_pool

pytestmark = pytest.mark.gpu

TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def bytes_of(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().ravel()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -6, 1000.0, 3e-5])
def test_scatter_every_16bit_code_bit_exact(dtype, scale):
    """Keys and values are permutations of all 65536 words; 16 extra tokens go to slot -1 or past
    the pool and must be skipped."""
    H, D, nb = 2, 128, 24
    rng = np.random.default_rng(600)
    T = 65536 // (H * D)
    key = rng.permutation(65536).astype(np.uint16).reshape(T, H, D)
    value = rng.permutation(65536).astype(np.uint16).reshape(T, H, D)
    slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    extra_k = rng.integers(0, 65536, size=(16, H, D), dtype=np.uint16)
    extra_v = rng.integers(0, 65536, size=(16, H, D), dtype=np.uint16)
    extra_s = np.array([-1, -7, nb * 16, nb * 16 + 5] * 4, np.int32)
    pool_k = rng.integers(0, 256, size=nb * H * 16 * D, dtype=np.uint8)
    pool_v = rng.integers(0, 256, size=nb * H * 16 * D, dtype=np.uint8)
    want_k, want_v = oracle.reshape_and_cache_fp8(key, value, pool_k, pool_v, slots, nb, H, D,
                                                  dtype, scale, scale * 0.5)
    print(f"[fp8] scatter of all {dtype} codes, k_scale {scale}", flush=True)
    dev = torch.device("cuda")
    kc = torch.from_numpy(pool_k).to(dev).view(nb, H, 16, D)
    vc = torch.from_numpy(pool_v).to(dev).view(nb, H, 16, D)
    keys = words_to_device(np.concatenate([key, extra_k]), dtype, dev)
    values = words_to_device(np.concatenate([value, extra_v]), dtype, dev)
    sm = torch.from_numpy(np.concatenate([slots, extra_s])).to(dev)
    binding.reshape_and_cache_fp8(keys, values, kc, vc, sm, scale, scale * 0.5)
    torch.cuda.synchronize()
    got_k, got_v = bytes_of(kc), bytes_of(vc)
    bad = np.flatnonzero(got_k != want_k)
    assert bad.size == 0, f"{bad.size} key bytes differ, first at {bad[:5]}: " \
                          f"{got_k[bad[:5]]} vs {want_k[bad[:5]]}"
    assert np.array_equal(got_v, want_v)


@pytest.mark.parametrize("name", ["llama2_7b_decode", "prefix_sharing_2040"])
def test_copy_and_scatter_full_pool_bit_exact(name):
    w = W.named(name)
    ks, vs = 0.03, 0.02
    kc, vc = oracle_fp8_pool(w, ks, vs, poison=False)
    print(f"[fp8] copy + scatter {name}: {len(w.copy_pairs)} pairs, {len(w.slot_mapping)} tokens",
          flush=True)
    g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc))
    g.copy()
    g.scatter()
    torch.cuda.synchronize()
    want_k, want_v = oracle_fp8_after_step(w, kc, vc, ks, vs)
    assert np.array_equal(bytes_of(g.k_cache), want_k)
    assert np.array_equal(bytes_of(g.v_cache), want_v)


def test_pool_quantized_on_device_equals_oracle():
    """The whole 16-bit pool of the 7B-shaped layer through the library's FP8 scatter."""
    w = W.named("llama2_7b_decode")
    g = GpuStep(w, kv_cache="fp8", k_scale=0.03, v_scale=0.02)
    kc, vc = oracle_fp8_pool(w, 0.03, 0.02, poison=False)
    assert np.array_equal(bytes_of(g.k_cache), kc)
    assert np.array_equal(bytes_of(g.v_cache), vc)


def run_fp8_decode(w, ks, vs, partition_size=None, pairs=None):
    """The E4M3 decode on the GPU and the oracle's F6 reference: [B, H_q, D], or [n, D] for an
    explicit list of (sequence, head) pairs."""
    kc, vc = oracle_fp8_pool(w, ks, vs)
    g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc),
                partition_size=partition_size)
    print(f"[fp8] decode {w.name}: H_q={w.H_q} H_kv={w.H_kv} D={w.D} {w.dtype} "
          f"partition={g.partition_size}", flush=True)
    g.copy()
    g.scatter()
    g.decode()
    torch.cuda.synchronize()
    kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
    nd = w.n_decode
    ref = oracle.decode_fp8(w.query_decode, kc, vc, w.block_tables[:nd], w.seq_lens[:nd], w.H_q,
                            w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, ks, vs, pairs=pairs)
    return g, ref


@pytest.mark.parametrize("name", ["tiny_decode", "llama2_7b_decode", "llama70b_gqa_decode"])
def test_decode_named_workload(name):
    """Every output row of the named workloads at full size (the 70B-shaped one: 32 sequences of
    8K-32K tokens, all 64 query heads)."""
    w = W.named(name)
    g, ref = run_fp8_decode(w, 0.03, 0.02)
    assert_attention_close(words_from_device(g.dec_out), ref, w.dtype, f"fp8 decode {name}",
                           absolute=True)


@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 2), (32, 8), (64, 8), (6, 2), (12, 4), (64, 2),
                                      (48, 1)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_head_groups(H_q, H_kv, D, dtype):
    lens = [0, 1, 16, 17, 31, 300, 1000, 2500]
    w = W.build(lens, H_q, H_kv, D, dtype, seed=620 + H_q + D)
    for part, (ks, vs) in ((0, (1.0, 1.0)), (256, (0.05, 0.015)), (512, (2.0 ** -5, 0.3))):
        g, ref = run_fp8_decode(w, ks, vs, partition_size=part)
        assert_attention_close(words_from_device(g.dec_out), ref, dtype,
                               f"fp8 decode H_q={H_q} H_kv={H_kv} D={D} P={part}")


def test_decode_is_deterministic():
    w = W.build([700, 1500, 90], 32, 8, 128, "bf16", seed=630)
    g, _ = run_fp8_decode(w, 0.03, 0.02, partition_size=256)
    first = words_from_device(g.dec_out)
    g.decode()
    torch.cuda.synchronize()
    assert np.array_equal(first, words_from_device(g.dec_out))


# ------------------------------------------------------------- read-once shared prefixes, E4M3
def run_fp8_shared_prefix(w, ks, vs, partition_size=None):
    kc, vc = oracle_fp8_pool(w, ks, vs)
    g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc),
                partition_size=partition_size, shared_prefix=True)
    assert g.shared_prefix
    print(f"[fp8] shared-prefix decode {w.name}: H_q={w.H_q} H_kv={w.H_kv} D={w.D} {w.dtype} "
          f"partition={g.partition_size} groups={len(g.group_starts) - 1} "
          f"max_group={g.max_group_size}", flush=True)
    g.copy()
    g.scatter()
    g.decode()
    torch.cuda.synchronize()
    kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
    nd = w.n_decode
    ref = oracle.decode_fp8(w.query_decode, kc, vc, w.block_tables[:nd], w.seq_lens[:nd], w.H_q,
                            w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, ks, vs)
    return g, ref


def test_shared_prefix_decode_named():
    """Parallel samples of the 2040-token prompt: 8 members per group read it once, E4M3."""
    w = W.named("prefix_sharing_2040")
    g, ref = run_fp8_shared_prefix(w, 0.03, 0.02)
    assert g.max_group_size == 8
    assert_attention_close(words_from_device(g.dec_out), ref, w.dtype,
                           "fp8 shared-prefix decode prefix_sharing_2040")


FP8_SHARED_GROUPS = [
    (40, [41, 60, 100]),                                        # prompt ends mid-block: CoW
    (1000, [1001, 1016, 1017, 1500, 2000, 1050, 1100, 1333]),   # 8 members
    (0, [5, 9]),                                                # nothing shared
    (16, [17]),                                                 # a group of one
    (640, [641 + 37 * i for i in range(20)]),                   # 20 members: several subgroups
]


@pytest.mark.parametrize("H_q,H_kv,D,dtype", [(4, 4, 128, "f16"), (8, 2, 128, "bf16"),
                                              (16, 4, 64, "f16"), (6, 2, 128, "bf16"),
                                              (2, 2, 64, "bf16"), (64, 2, 128, "bf16")])
@pytest.mark.parametrize("part,ks,vs", [(16, 0.05, 0.015), (512, 2.0 ** -5, 0.3)])
def test_shared_prefix_decode_groups(H_q, H_kv, D, dtype, part, ks, vs):
    w = W.build_shared_groups(FP8_SHARED_GROUPS, H_q, H_kv, D, dtype, seed=640 + H_q + D,
                              independent=[1, 33, 700])
    g, ref = run_fp8_shared_prefix(w, ks, vs, partition_size=part)
    assert_attention_close(words_from_device(g.dec_out), ref, dtype,
                           f"fp8 shared-prefix decode H_q={H_q} H_kv={H_kv} D={D} {dtype} "
                           f"part={part}")


def test_shared_prefix_decode_is_deterministic_and_matches_plain():
    """Bitwise reproducible; and within the gate of the plain E4M3 decode of the same sequences
    (which reads the shared blocks once per member)."""
    w = W.build_shared_groups(FP8_SHARED_GROUPS, 32, 8, 128, "bf16", seed=650)
    g, ref = run_fp8_shared_prefix(w, 0.03, 0.02, partition_size=256)
    first = words_from_device(g.dec_out)
    g.decode()
    torch.cuda.synchronize()
    assert np.array_equal(first, words_from_device(g.dec_out))
    plain = torch.empty_like(g.dec_out)
    binding.decode_fp8(plain, g.dec_query, g.k_cache, g.v_cache, g.dec_tables, g.dec_lens,
                       g.max_seq_len, w.scale, 0.03, 0.02, 256)
    torch.cuda.synchronize()
    # contexts of 5 to 17 tokens give outputs near 1, where the bf16 output's own rounding alone
    # reaches 2^-8 |ref| (3.9e-3 at |ref| = 1): the bf16 gate, not the absolute one
    assert_attention_close(words_from_device(plain), ref, w.dtype, "fp8 plain decode")
    assert_attention_close(first, ref, w.dtype, "fp8 shared-prefix decode")


# --------------------------------------------------------------- chunked prefill, E4M3
def run_fp8_prefill(w, ks, vs):
    kc, vc = oracle_fp8_pool(w, ks, vs)
    g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc))
    print(f"[fp8] prefill {w.name}: H_q={w.H_q} H_kv={w.H_kv} D={w.D} {w.dtype} "
          f"rows={w.query_prefill.shape[0]}", flush=True)
    g.copy()
    g.scatter()
    g.decode()
    g.prefill()
    torch.cuda.synchronize()
    kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
    nd = w.n_decode
    ref = oracle.prefill_fp8(w.query_prefill, kc, vc, w.block_tables[nd:], w.seq_lens[nd:],
                             w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale,
                             ks, vs)
    return g, ref


@pytest.mark.parametrize("H_q,H_kv", [(4, 4), (8, 2), (16, 4), (32, 2), (6, 2), (12, 12)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_chunks(H_q, H_kv, D, dtype):
    """Chunks of whole prompts (first rows see one key), chunks over cached context, a ragged
    last row tile and a context ending mid-block, plus decodes in the same step."""
    lens = [40, 700, 1300, 97, 16, 2049]
    q_lens = [40, 129, 300, 1, 16, 64]
    w = W.build([300, 1000] + lens, H_q, H_kv, D, dtype, seed=660 + H_q + D, n_decode=2,
                q_lens=q_lens)
    g, ref = run_fp8_prefill(w, 0.04, 0.025)
    assert_attention_close(words_from_device(g.pre_out), ref, dtype,
                           f"fp8 prefill H_q={H_q} H_kv={H_kv} D={D} {dtype}")


@pytest.mark.parametrize("H_q,H_kv,D,dtype", [(8, 2, 128, "bf16"), (4, 4, 64, "f16"),
                                            (12, 4, 128, "f16"), (16, 16, 64, "bf16")])
def test_prefill_widened_equals_staged(H_q, H_kv, D, dtype):
    """The step prefills over a 16-bit widened copy of the context (pa_prefill_chunk_fp8 with a
    workspace); without one the codes are converted in the tile loop. Same conversion, same LDS
    contents, same MFMAs: the outputs must be the same bits, and both within the gate."""
    lens = [40, 700, 1300, 97, 16, 2049, 777]
    q_lens = [40, 129, 300, 1, 16, 64, 700]
    w = W.build([300] + lens, H_q, H_kv, D, dtype, seed=880 + H_q + D, n_decode=1, q_lens=q_lens)
    g, ref = run_fp8_prefill(w, 0.04, 0.025)
    assert g.pre_workspace is not None
    staged = torch.empty_like(g.pre_out)
    binding.prefill_chunk_fp8(staged, g.pre_query, g.k_cache, g.v_cache, g.pre_tables, g.pre_lens,
                              g.pre_cu, g.max_q_len, w.scale, 0.04, 0.025)
    torch.cuda.synchronize()
    widened = words_from_device(g.pre_out)
    assert np.array_equal(widened, words_from_device(staged))
    assert_attention_close(widened, ref, dtype, f"fp8 widened prefill H_q={H_q} D={D} {dtype}")


def test_prefill_mixed_step_full():
    """The 2048-token mixed step over E4M3 caches: every decode row and every row of the 1856-row
    chunk (all 32 heads) against the oracle."""
    w = W.named("chunked_prefill_mixed")
    ks, vs = 0.03, 0.02
    kc, vc = oracle_fp8_pool(w, ks, vs, poison=False)
    g = GpuStep(w, kv_cache="fp8", k_scale=ks, v_scale=vs, fp8_pool=(kc, vc))
    print("[fp8] mixed step", flush=True)
    g.run()
    torch.cuda.synchronize()
    kc, vc = oracle_fp8_after_step(w, kc, vc, ks, vs)
    nd = w.n_decode
    ref_d = oracle.decode_fp8(w.query_decode, kc, vc, w.block_tables[:nd], w.seq_lens[:nd],
                              w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, ks, vs)
    assert_attention_close(words_from_device(g.dec_out), ref_d, w.dtype, "fp8 mixed decode",
                           absolute=True)
    t = time.time()
    ref_p = oracle.prefill_fp8(w.query_prefill, kc, vc, w.block_tables[nd:], w.seq_lens[nd:],
                               w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale,
                               ks, vs)
    print(f"[fp8] oracle prefill of the whole chunk: {time.time() - t:.1f}s", flush=True)
    assert_attention_close(words_from_device(g.pre_out), ref_p, w.dtype, "fp8 mixed prefill",
                           absolute=True)
    # the step prefilled over the widened copy; the in-loop conversion gives the same bits
    assert g.pre_workspace is not None
    staged = torch.empty_like(g.pre_out)
    binding.prefill_chunk_fp8(staged, g.pre_query, g.k_cache, g.v_cache, g.pre_tables, g.pre_lens,
                              g.pre_cu, g.max_q_len, w.scale, ks, vs)
    torch.cuda.synchronize()
    assert np.array_equal(words_from_device(g.pre_out), words_from_device(staged))


def test_prefill_is_deterministic():
    w = W.build([900, 2100], 32, 8, 128, "bf16", seed=680, n_decode=0, q_lens=[300, 200])
    g, _ = run_fp8_prefill(w, 0.03, 0.02)
    first = words_from_device(g.pre_out)
    g.prefill()
    torch.cuda.synchronize()
    assert np.array_equal(first, words_from_device(g.pre_out))
