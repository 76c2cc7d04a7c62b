"""The step recorded as a HIP graph and replayed (GpuStep.capture).

A graph holds the step's kernels on fixed buffers. It is the way to launch a step whose kernels are
short (small batches, one new token per sequence) without paying one host launch per kernel.
Every replay must give the eager step's results bit for bit: from the same caches and inputs, a
replay and an eager step leave the same cache words and outputs.
  * Three replays, each from the caches the eager step started from (restored by eager copies on
    the same stream, which also overwrite the outputs with NaN words), with a synchronization
    before and after.
  * A replay after new queries and new K/V rows were written in place, against an eager step on
    those inputs.
The steps: the tiny decode, 16-bit and E4M3 mixed steps, a shared-prefix step with copy-on-write
pairs, a decode of head groups of 32, and drafted rows (pa_decode_multi) beside one-token decodes
over E4M3 caches.
A step with copy-on-write pairs is not idempotent on the cache words (a shared block's holder
writes its new rows into the block the copies are taken from), hence the restored caches. The
eager step itself is checked against the float64 oracle by the parity tests; these tests pin the
replays to it.
"""
import numpy as np
import pytest
import torch

import pa_workloads as W
from paged_kv_cache_99_amd.step import GpuStep, words_from_device

pytestmark = pytest.mark.gpu

NAN_WORD = {"f16": 0x7E00, "bf16": 0x7FC0}

SHARED_GROUPS = [
    (40, [41, 60, 100]),                                        # prompt ends mid-block: copy on write
    (1000, [1001, 1016, 1017, 1500, 2000, 1050, 1100, 1333]),   # 8 members
    (0, [5, 9]),                                                # nothing shared
]

CASES = {
    "tiny_decode": (lambda: W.tiny_decode(), {}),
    "mixed_bf16": (lambda: W.build([300, 1000, 4100, 90, 2100], 32, 8, 128, "bf16", seed=710,
                                   n_decode=4, q_lens=[400]), {}),
    "mixed_e4m3": (lambda: W.build([300, 1000, 4100, 90, 2100], 32, 8, 128, "bf16", seed=711,
                                   n_decode=4, q_lens=[400]),
                   {"kv_cache": "fp8", "k_scale": 0.03, "v_scale": 0.02}),
    "shared_prefix_f16": (lambda: W.build_shared_groups(SHARED_GROUPS, 4, 4, 128, "f16",
                                                        seed=712),
                          {"shared_prefix": True, "partition_size": 256}),
    # head groups of 32 (MQA-like): the decode runs the two-column-group units
    "groups_of_32": (lambda: W.build([3000, 700, 1500, 20, 4100], 64, 2, 128, "bf16", seed=715),
                     {}),
    # drafted rows (pa_decode_multi) beside one-token decodes, E4M3 caches
    "drafts_e4m3": (lambda: W.build([700, 2500, 1300, 4100, 30], 16, 4, 128, "bf16", seed=714,
                                    n_decode=2, q_lens=[4, 7, 1]),
                    {"kv_cache": "fp8", "k_scale": 0.03, "v_scale": 0.02}),
}


def snapshot(g):
    out = {"k_cache": words_from_device(g.k_cache), "v_cache": words_from_device(g.v_cache)}
    if g.n_decode:
        out["dec_out"] = words_from_device(g.dec_out)
    if g.pre_query.shape[0]:
        out["pre_out"] = words_from_device(g.pre_out)
    return out


def assert_same(a, b, what):
    assert a.keys() == b.keys()
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs from the eager step"


def reset(g, caches, dtype):
    """Eager work on the step's stream: the caches back to their saved words, NaN outputs."""
    g.k_cache.copy_(caches[0])
    g.v_cache.copy_(caches[1])
    for t in (g.dec_out, g.pre_out):
        if t.numel():
            t.view(torch.int16).fill_(NAN_WORD[dtype])


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_step(name):
    make, kw = CASES[name]
    w = make()
    print(f"[graph] {name}: {len(w.seq_lens)} sequences, H_q={w.H_q} H_kv={w.H_kv} D={w.D}",
          flush=True)
    g = GpuStep(w, **kw)
    if kw.get("shared_prefix"):
        assert g.shared_prefix and len(w.copy_pairs) > 0
    if name.startswith("drafts"):
        assert g.multi_token
    start = (g.k_cache.clone(), g.v_cache.clone())
    g.run()
    torch.cuda.synchronize()
    eager = snapshot(g)

    graph = g.capture()
    for r in range(3):
        reset(g, start, w.dtype)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same(snapshot(g), eager, f"{name} replay {r}")

    # new inputs written in place: queries of both kinds and the step's new K/V rows
    gen = torch.Generator(device="cuda").manual_seed(713)
    for t in (g.dec_query, g.pre_query, g.new_key, g.new_value):
        if t.numel():
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda", dtype=torch.float32)
                    .to(t.dtype))
    reset(g, start, w.dtype)
    g.run()
    torch.cuda.synchronize()
    eager_new = snapshot(g)
    reset(g, start, w.dtype)
    graph.replay()
    torch.cuda.synchronize()
    assert_same(snapshot(g), eager_new, f"{name} replay on new inputs")
    if g.n_decode:
        assert not np.array_equal(eager_new["dec_out"], eager["dec_out"]), \
            "the new queries should change the decode output"
