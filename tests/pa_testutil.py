"""Shared helpers of the GPU parity tests: expected values from the oracle, and the comparison gates.

Expected values come only from oracle/ applied to the generator's inputs: the oracle's own copy and
scatter produce the pool the oracle's attention then reads.
"""
import numpy as np
import torch

import oracle

ATOL = 2e-3      # max |gpu - oracle| over every element
ROW_RTOL = 1e-2  # max over (token, head) rows of ||gpu - oracle||_inf / ||oracle||_inf
BF16_HALF_ULP = 2.0 ** -8  # largest relative rounding error of a bfloat16 output


def words_to_f64(words, dtype):
    """16-bit words to float64 (numpy / torch decoding, equal to oracle.to_double on all codes)."""
    w = np.ascontiguousarray(words, dtype=np.uint16)
    if dtype == "f16":
        return w.view(np.float16).astype(np.float64)
    return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def oracle_pool_after_step(w, poison=False):
    """The pool the attention of a step reads: copy_blocks, then reshape_and_cache, on the CPU."""
    kc, vc = w.k_cache, w.v_cache
    if poison:
        kc, vc = oracle.poison_free_slots(kc, vc, w.block_tables, w.seq_lens, w.num_blocks,
                                          w.H_kv, w.D, w.dtype)
    if len(w.copy_pairs):
        kc, vc = oracle.copy_blocks(kc, vc, w.copy_pairs, w.num_blocks, w.H_kv, w.D)
    kc, vc = oracle.reshape_and_cache(w.new_key, w.new_value, kc, vc, w.slot_mapping,
                                      w.num_blocks, w.H_kv, w.D)
    return kc, vc


def oracle_fp8_pool(w, k_scale, v_scale, poison=True):
    """The workload's pool as E4M3 codes (the oracle's quantization), free slots poisoned with the
    NaN code unless poison is False."""
    kc = oracle.quantize_e4m3(w.k_cache, w.dtype, k_scale)
    vc = oracle.quantize_e4m3(w.v_cache, w.dtype, v_scale)
    if poison:
        kc, vc = oracle.poison_free_slots_fp8(kc, vc, w.block_tables, w.seq_lens, w.num_blocks,
                                              w.H_kv, w.D)
    return kc, vc


def oracle_fp8_after_step(w, kc, vc, k_scale, v_scale):
    """The E4M3 pool a step's attention reads: copy_blocks, then the quantizing scatter."""
    if len(w.copy_pairs):
        kc, vc = oracle.copy_blocks_fp8(kc, vc, w.copy_pairs, w.num_blocks, w.H_kv, w.D)
    return oracle.reshape_and_cache_fp8(w.new_key, w.new_value, kc, vc, w.slot_mapping,
                                        w.num_blocks, w.H_kv, w.D, w.dtype, k_scale, v_scale)


def oracle_decode(w, kc, vc, pairs=None, nthreads=0):
    nd = w.n_decode
    return oracle.decode(w.query_decode, kc, vc, w.block_tables[:nd], w.seq_lens[:nd], w.H_q,
                         w.H_kv, w.D, w.num_blocks, w.dtype, w.scale, pairs=pairs,
                         nthreads=nthreads)


def oracle_prefill(w, kc, vc, rows=None, nthreads=0):
    nd = w.n_decode
    return oracle.prefill(w.query_prefill, kc, vc, w.block_tables[nd:], w.seq_lens[nd:],
                          w.cu_q_lens, w.H_q, w.H_kv, w.D, w.num_blocks, w.dtype, w.scale,
                          rows=rows, nthreads=nthreads)


def attention_errors(got_words, ref, dtype):
    """(max abs error, max row-normwise relative error) of 16-bit outputs against float64."""
    got = words_to_f64(got_words, dtype).reshape(ref.shape)
    D = ref.shape[-1]
    err = np.abs(got - ref).reshape(-1, D)
    row_ref = np.abs(ref).reshape(-1, D).max(axis=1)
    row_err = err.max(axis=1)
    zero = row_ref == 0
    rel = np.where(zero, np.where(row_err == 0, 0.0, np.inf), row_err / np.where(zero, 1, row_ref))
    return (float(err.max()) if err.size else 0.0), (float(rel.max()) if rel.size else 0.0), got


def elementwise_bound(ref, dtype):
    """Per-element bound on |gpu - oracle| for an attention output of `dtype`.

    f16 outputs: 2e-3. A binary16 output keeps 11 significant bits, so rounding it moves a value by
    at most 2^-11 |ref| (below 1e-3 for |ref| < 2), well inside the bound.
    bf16 outputs: 2e-3 + 2^-8 |ref|. A bfloat16 output keeps 8 significant bits; rounding to nearest
    moves x in [2^e, 2^(e+1)) by up to half a unit in the last place, 2^(e-8), which is 2^-8 |x| at
    the bottom of the binade. No correct kernel can do better than its own output rounding, so the
    gate adds exactly that to the 2e-3 allowed for the arithmetic.
    """
    if dtype == "bf16":
        return ATOL + BF16_HALF_ULP * np.abs(ref)
    assert dtype == "f16", dtype
    return np.full(np.shape(ref), ATOL)


def assert_attention_close(got_words, ref, dtype, what="", absolute=False):
    """Gate of an attention output against the float64 oracle (the 2e-3 / 1e-2 bound read per
    output type):
      (i)  every element: |gpu - ref| <= elementwise_bound(ref, dtype) -- 2e-3 for f16 outputs,
           2e-3 + 2^-8 |ref| for bf16 outputs;
      (ii) every (token, head) row: ||gpu - ref||_inf / ||ref||_inf <= 1e-2.
    absolute=True adds max |gpu - ref| <= 2e-3 for bf16 outputs too; the long-context workloads,
    whose outputs are small, meet it.
    """
    max_abs, max_rel, got = attention_errors(got_words, ref, dtype)
    bound = elementwise_bound(ref, dtype)
    excess = float((np.abs(got - ref) - bound).max()) if ref.size else 0.0
    print(f"[parity] {what}: {dtype} max_abs={max_abs:.3e} max_row_rel={max_rel:.3e} "
          f"max(|d| - bound)={excess:.3e} n={ref.size}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert excess <= 0, f"{what}: |d| exceeds the {dtype} element bound by {excess:.3e}"
    assert max_rel <= ROW_RTOL, f"{what}: row-normwise relative error {max_rel:.3e} > {ROW_RTOL}"
    if absolute:
        assert max_abs <= ATOL, f"{what}: max abs error {max_abs:.3e} > {ATOL}"


# ------------------------------------------------------------------ drafted-token trees
def random_parents(n, rng):
    """A drafted-token tree in topological order: node i's parent is -1 (a child of the last
    context token) or an earlier node."""
    return [int(rng.integers(-1, i)) if i else -1 for i in range(n)]


def tree_path(parents, i):
    """Chunk indices on node i's path from the root, ascending (i included)."""
    out = []
    while i >= 0:
        out.append(i)
        i = parents[i]
    return out[::-1]


def tree_masks(parents):
    """The 64-bit mask of every node: itself and its ancestors."""
    m = []
    for i, par in enumerate(parents):
        m.append((1 << i) | (m[par] if par >= 0 else 0))
    return np.array(m, dtype=np.uint64)
