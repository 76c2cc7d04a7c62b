"""Seeded synthetic inputs for the paged-attention hot path.

The tests, the benchmark and the smoke check draw every input here, for both the HIP library and
the CPU oracle. This module holds none of the method's arithmetic -- no attention, gather, scatter,
copy or merge. It draws random numbers, rounds float32 draws to 16-bit words (round to nearest
even), and does the host-side bookkeeping that a block manager does before a step: how many blocks
a sequence needs, which physical blocks it gets, which blocks are shared and copied on write, and
the slot of every new token.

Block-manager rules, from openeuler.csdn.net "高并发 AI 服务的内存瓶颈":
  * a sequence of L tokens holds ceil(L/16) blocks, a new one taken only when the last is full
    (section 机制1 按需分配; worked example 100 tokens -> 7 blocks -> 112 slots);
  * position i of a sequence is stored at slot table[i // 16] * 16 + i % 16
    (section Block Table 数据结构, get_physical_indices);
  * parallel samples share their prompt blocks with a reference count and get a private block only
    where they diverge (section 机制 2 写时复制).

Random draws use numpy's PCG64 generator seeded with the workload's seed, in this fixed order:
sequence lengths (and suffix lengths), the block permutation, decode queries, prefill queries, the
K pool, the V pool, the new keys, the new values. Every value is N(0, 1); each value array is
filled from its own sub-seed drawn in that order (see _normal_words).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence

import numpy as np

BLOCK = 16
_POOL_CHUNK = 1 << 24  # values drawn per chunk when filling a pool
_THREADS = max(1, min(8, os.cpu_count() or 1))


# ------------------------------------------------------------------------------------ rounding
def f32_to_words(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to 16-bit words, nearest-even: IEEE binary16 or bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        if not np.isfinite(x).all():
            raise ValueError("bf16 rounding here is for finite values")
        u = x.view(np.uint32)
        u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return u.astype(np.uint16)
    raise ValueError(dtype)


def _normal_words(rng: np.random.Generator, n: int, dtype: str) -> np.ndarray:
    """n N(0,1) values as 16-bit words. One 63-bit sub-seed is drawn from `rng`; chunk i of the
    array then comes from PCG64(SeedSequence([sub_seed, i])), so chunks fill in parallel threads
    and the result does not depend on the thread count."""
    sub_seed = int(rng.integers(0, 2**63 - 1))
    out = np.empty(n, dtype=np.uint16)

    def fill(i):
        a, b = i * _POOL_CHUNK, min(n, (i + 1) * _POOL_CHUNK)
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([sub_seed, i])))
        out[a:b] = f32_to_words(r.standard_normal(b - a, dtype=np.float32), dtype)

    chunks = (n + _POOL_CHUNK - 1) // _POOL_CHUNK
    if chunks <= 1:
        for i in range(chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=min(_THREADS, chunks)) as ex:
            list(ex.map(fill, range(chunks)))
    return out


# ------------------------------------------------------------------------------- block manager
def blocks_needed(L: int) -> int:
    """Blocks a sequence of L tokens holds: a block is taken only when the last one is full."""
    return (L + BLOCK - 1) // BLOCK


def slot_of(table: Sequence[int], pos: int) -> int:
    """Slot (physical_block * 16 + offset) of logical position pos under a block table."""
    return int(table[pos // BLOCK]) * BLOCK + pos % BLOCK


class BlockPool:
    """A pool of physical blocks handed out in a fixed (seeded) order, with reference counts."""

    def __init__(self, num_blocks: int, order: np.ndarray):
        self.num_blocks = int(num_blocks)
        self.free: List[int] = [int(b) for b in order]
        self.ref_cnt = np.zeros(self.num_blocks, dtype=np.int32)

    def take(self, n: int = 1) -> List[int]:
        if n > len(self.free):
            raise MemoryError(f"block pool exhausted: need {n}, have {len(self.free)}")
        got, self.free = self.free[:n], self.free[n:]
        for b in got:
            self.ref_cnt[b] += 1
        return got

    def share(self, blocks: Sequence[int]) -> List[int]:
        for b in blocks:
            self.ref_cnt[b] += 1
        return list(blocks)

    def write_block(self, table: List[int], logical: int) -> Optional[int]:
        """A writer is about to write into table[logical]. If the block is shared (ref_cnt > 1), copy
        it on write: take a fresh block, drop one reference from the shared one and repoint the
        entry; return the fresh block. The last holder (ref_cnt == 1) writes in place (None)."""
        b = table[logical]
        if self.ref_cnt[b] <= 1:
            return None
        (fresh,) = self.take(1)
        self.ref_cnt[b] -= 1
        table[logical] = fresh
        return fresh


def pad_tables(tables: List[List[int]], max_blocks: Optional[int] = None) -> np.ndarray:
    mb = max([len(t) for t in tables] + [1]) if max_blocks is None else max_blocks
    out = np.full((len(tables), mb), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, : len(t)] = t
    return out


# ------------------------------------------------------------------------------------ workload
@dataclasses.dataclass
class Workload:
    """One step of the hot path: copy_blocks, then reshape_and_cache, then decode, then prefill.

    Sequences 0..n_decode-1 decode one new token (their last position); sequences n_decode.. are
    prefill chunks whose last q_len positions are new. seq_lens count every token including new
    ones. Caches are flat uint16 word arrays of num_blocks*H_kv*16*D words.
    """
    name: str
    dtype: str
    H_q: int
    H_kv: int
    D: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray      # int32 [S, max_blocks], -1 padded
    k_cache: np.ndarray           # uint16 pool before the step
    v_cache: np.ndarray
    new_key: np.ndarray           # uint16 [T, H_kv, D]
    new_value: np.ndarray
    slot_mapping: np.ndarray      # int32 [T]
    copy_pairs: np.ndarray        # int32 [N, 2] (src, dst)
    n_decode: int
    query_decode: np.ndarray      # uint16 [n_decode, H_q, D]
    cu_q_lens: np.ndarray         # int32 [S - n_decode + 1]
    query_prefill: np.ndarray     # uint16 [total_q, H_q, D]
    scale: float
    partition_size: Optional[int] = None
    ref_cnt: Optional[np.ndarray] = None
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def block_elems(self) -> int:
        return self.H_kv * BLOCK * self.D

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def decode_seq_lens(self) -> np.ndarray:
        return self.seq_lens[: self.n_decode]

    @property
    def decode_tables(self) -> np.ndarray:
        return self.block_tables[: self.n_decode]

    @property
    def prefill_seq_lens(self) -> np.ndarray:
        return self.seq_lens[self.n_decode:]

    @property
    def prefill_tables(self) -> np.ndarray:
        return self.block_tables[self.n_decode:]

    @property
    def esize(self) -> int:
        return 2


def _finish(name, rng, dtype, H_q, H_kv, D, num_blocks, seq_lens, tables, n_decode, q_lens,
            new_positions, copy_pairs, pool, partition_size, max_blocks=None, meta=None):
    """Draw the value arrays (fixed order) and assemble the Workload."""
    S = len(seq_lens)
    total_q = int(sum(q_lens))
    q_dec = _normal_words(rng, n_decode * H_q * D, dtype).reshape(n_decode, H_q, D)
    q_pre = _normal_words(rng, total_q * H_q * D, dtype).reshape(total_q, H_q, D)
    n_pool = num_blocks * H_kv * BLOCK * D
    k_cache = _normal_words(rng, n_pool, dtype)
    v_cache = _normal_words(rng, n_pool, dtype)
    slots = [slot_of(tables[s], p) for s, p in new_positions]
    T = len(slots)
    new_key = _normal_words(rng, T * H_kv * D, dtype).reshape(T, H_kv, D)
    new_value = _normal_words(rng, T * H_kv * D, dtype).reshape(T, H_kv, D)
    cu = np.zeros(S - n_decode + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    return Workload(
        name=name, dtype=dtype, H_q=H_q, H_kv=H_kv, D=D, num_blocks=num_blocks,
        seq_lens=np.asarray(seq_lens, dtype=np.int32),
        block_tables=pad_tables(tables, max_blocks),
        k_cache=k_cache, v_cache=v_cache, new_key=new_key, new_value=new_value,
        slot_mapping=np.asarray(slots, dtype=np.int32).reshape(T),
        copy_pairs=np.asarray(copy_pairs, dtype=np.int32).reshape(-1, 2),
        n_decode=n_decode, query_decode=q_dec, cu_q_lens=cu, query_prefill=q_pre,
        scale=1.0 / math.sqrt(D), partition_size=partition_size,
        ref_cnt=pool.ref_cnt.copy(), meta=dict(meta or {}))


def build(seq_lens: Sequence[int], H_q: int, H_kv: int, D: int, dtype: str, seed: int,
          n_decode: Optional[int] = None, q_lens: Sequence[int] = (),
          num_blocks: Optional[int] = None, permute: bool = True,
          partition_size: Optional[int] = None, name: str = "custom",
          max_blocks: Optional[int] = None) -> Workload:
    """A decode (+ optional prefill) step over independent sequences.

    seq_lens are drawn by the caller (or given). Sequences [0, n_decode) decode one token; the rest
    are prefill chunks with the given q_lens. Physical blocks come from a seeded permutation of a
    pool of num_blocks (default: needed blocks + 10%, rounded up), taken in (sequence, logical
    block) order; permute=False hands them out in order 0, 1, 2, ...
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = [int(x) for x in seq_lens]
    S = len(seq_lens)
    n_decode = S if n_decode is None else int(n_decode)
    q_lens = [int(x) for x in q_lens]
    if len(q_lens) != S - n_decode:
        raise ValueError("one q_len per prefill sequence")
    for L, ql in zip(seq_lens[n_decode:], q_lens):
        if not 0 <= ql <= L:
            raise ValueError("q_len must be within the sequence")
    need = sum(blocks_needed(L) for L in seq_lens)
    nb = need + (need + 9) // 10 if num_blocks is None else int(num_blocks)
    order = rng.permutation(nb) if permute else np.arange(nb)
    pool = BlockPool(nb, order)
    tables = [pool.take(blocks_needed(L)) for L in seq_lens]
    new_positions = [(s, seq_lens[s] - 1) for s in range(n_decode) if seq_lens[s] > 0]
    for s, ql in zip(range(n_decode, S), q_lens):
        new_positions += [(s, p) for p in range(seq_lens[s] - ql, seq_lens[s])]
    return _finish(name, rng, dtype, H_q, H_kv, D, nb, seq_lens, tables, n_decode, q_lens,
                   new_positions, [], pool, partition_size, max_blocks)


def build_shared_groups(groups, H_q: int, H_kv: int, D: int, dtype: str, seed: int,
                        independent: Sequence[int] = (), partition_size: Optional[int] = None,
                        name: str = "shared_groups") -> Workload:
    """Groups of parallel samples, each sharing a prompt, followed by independent sequences.

    groups: list of (prefix_tokens, [total length of each member]) -- every member holds the
    prompt's blocks with a reference count equal to the group size. When the prompt ends inside a
    block, that block is copied on write for every member but the last holder (copy_blocks pairs);
    each member then writes its own tokens of that block and its newest token (reshape_and_cache).
    independent: lengths of sequences in no group (one new token each).
    meta: group_starts [groups + 1] and shared_prefix [S] = tokens of the blocks all members still
    hold in common (the prompt rounded down to whole blocks; 0 outside a group).
    Blocks are taken from one seeded permutation: per group its prompt blocks, then per member its
    copy-on-write block (if any) and its private blocks; then the independent sequences' blocks.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    need = 0
    for prefix, lens in groups:
        n_pre = blocks_needed(prefix)
        need += n_pre + sum(blocks_needed(L) - n_pre for L in lens)
        if prefix % BLOCK:
            need += len(lens) - 1
    need += sum(blocks_needed(L) for L in independent)
    nb = need + (need + 9) // 10
    pool = BlockPool(nb, rng.permutation(nb))
    tables, pairs, new_positions, seq_lens, shared, starts = [], [], [], [], [], [0]
    for prefix, lens in groups:
        if any(L <= prefix for L in lens):
            raise ValueError("every member extends its prompt")
        n_pre = blocks_needed(prefix)
        common = pool.take(n_pre)
        pool.share([b for b in common for _ in range(len(lens) - 1)])
        for L in lens:
            s = len(seq_lens)
            t = list(common)
            if prefix % BLOCK:
                src = t[n_pre - 1]
                fresh = pool.write_block(t, n_pre - 1)
                if fresh is not None:
                    pairs.append((src, fresh))
            t += pool.take(blocks_needed(L) - n_pre)
            tables.append(t)
            seq_lens.append(int(L))
            shared.append((prefix // BLOCK) * BLOCK)
            pos = list(range(prefix, min(n_pre * BLOCK, L)))
            if L - 1 not in pos:
                pos.append(L - 1)
            new_positions += [(s, q) for q in pos]
        starts.append(len(seq_lens))
    for L in independent:
        s = len(seq_lens)
        tables.append(pool.take(blocks_needed(L)))
        seq_lens.append(int(L))
        shared.append(0)
        if L > 0:
            new_positions.append((s, L - 1))
    return _finish(name, rng, dtype, H_q, H_kv, D, nb, seq_lens, tables, len(seq_lens), [],
                   new_positions, pairs, pool, partition_size,
                   meta={"group_starts": np.asarray(starts, np.int32),
                         "shared_prefix": np.asarray(shared, np.int32)})


def build_prefix_sharing(groups: int, samples: int, prefix: int, suffix_max: int, H: int, D: int,
                         dtype: str, seed: int, partition_size: Optional[int] = None,
                         name: str = "prefix_sharing") -> Workload:
    """`groups` groups of `samples` parallel samples: each group shares a `prefix`-token prompt
    (its blocks have ref_cnt == samples), each sample then holds a private suffix of U{1..suffix_max}
    tokens (drawn first, group by group). See build_shared_groups for the step it describes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    suffix = rng.integers(1, suffix_max, size=groups * samples, endpoint=True)
    spec = [(prefix, [prefix + int(x) for x in suffix[g * samples:(g + 1) * samples]])
            for g in range(groups)]
    w = build_shared_groups(spec, H, H, D, dtype, int(rng.integers(0, 2**31 - 1)),
                            partition_size=partition_size, name=name)
    w.meta.update({"groups": groups, "samples": samples, "prefix": prefix})
    return w


# ------------------------------------------------------------------------- the named workloads
def tiny_decode(seed: int = 1) -> Workload:
    """4 sequences of {1, 7, 16, 33} tokens (counting the new one), 4 q = 4 kv heads, head_dim 64,
    fp16, a pool of 16 blocks handed out by a seeded permutation; one new token per sequence."""
    return build([1, 7, 16, 33], 4, 4, 64, "f16", seed, num_blocks=16, name="tiny_decode")


def llama2_7b_decode(seed: int = 2, batch: int = 64) -> Workload:
    """LLaMA-2-7B-shaped single-layer decode: 64 sequences of U{512..4096} tokens, 32 q = 32 kv
    heads of 128, fp16, pool = needed blocks + 10% in a seeded permutation, one new token each."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 4096, size=batch, endpoint=True)
    return build(lens, 32, 32, 128, "f16", seed + 1000, name="llama2_7b_decode")


def llama2_7b_spec_decode(seed: int = 2, batch: int = 64, drafts: int = 4) -> Workload:
    """The LLaMA-2-7B-shaped layer of llama2_7b_decode (same seeded U{512..4096} contexts, 32 q =
    32 kv heads of 128, fp16) in a speculative step: every sequence appends `drafts` drafted tokens
    (its last positions), verified together as one short chunk of that many rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 4096, size=batch, endpoint=True) + (drafts - 1)
    return build(lens, 32, 32, 128, "f16", seed + 1000, n_decode=0, q_lens=[drafts] * batch,
                 name=f"llama2_7b_spec{drafts}")


def llama70b_gqa_decode(seed: int = 3, batch: int = 32) -> Workload:
    """70B-GQA-shaped long-context decode: 32 sequences of U{8192..32768} tokens, 64 q / 8 kv heads
    of 128, bf16, split into partitions of 512 tokens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(8192, 32768, size=batch, endpoint=True)
    return build(lens, 64, 8, 128, "bf16", seed + 1000, partition_size=512,
                 name="llama70b_gqa_decode")


def llama70b_gqa_spec_decode(seed: int = 3, batch: int = 32, drafts: int = 4) -> Workload:
    """The 70B-GQA-shaped layer of llama70b_gqa_decode (same seeded U{8192..32768} contexts, 64 q /
    8 kv heads of 128, bf16, 512-token parts) in a speculative step: every sequence appends `drafts`
    drafted tokens, verified together as one short chunk (drafts x 8 query heads per kv head)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(8192, 32768, size=batch, endpoint=True) + (drafts - 1)
    return build(lens, 64, 8, 128, "bf16", seed + 1000, n_decode=0, q_lens=[drafts] * batch,
                 partition_size=512, name=f"llama70b_gqa_spec{drafts}")


def prefix_sharing_sampling(prefix: int = 2040, seed: int = 4) -> Workload:
    """32 groups x 8 parallel samples sharing a prompt of `prefix` tokens (128 blocks, ref_cnt 8),
    private suffixes U{1..512}, 32 q = 32 kv heads of 128, fp16. With prefix 2040 the last shared
    block is half full and is copied on write for 7 of the 8 samples (224 pairs); with 2048 it is
    full and nothing is copied."""
    return build_prefix_sharing(32, 8, prefix, 512, 32, 128, "f16", seed,
                                name=f"prefix_sharing_{prefix}")


def chunked_prefill_mixed(seed: int = 5) -> Workload:
    """A 2048-token budget step: 192 decodes (U{256..8192} tokens each, one budget token each) plus
    a 1856-token prefill chunk of a sequence with 6144 tokens already cached; 32 q / 8 kv heads of
    128, bf16. The scatter writes all 2048 new tokens (decode tokens first)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [int(x) for x in rng.integers(256, 8192, size=192, endpoint=True)]
    budget, cached = 2048, 6144
    chunk = budget - len(lens)
    return build(lens + [cached + chunk], 32, 8, 128, "bf16", seed + 1000, n_decode=192,
                 q_lens=[chunk], name="chunked_prefill_mixed")


NAMED = {
    "tiny_decode": tiny_decode,
    "llama2_7b_decode": llama2_7b_decode,
    "llama70b_gqa_decode": llama70b_gqa_decode,
    "llama2_7b_spec4": llama2_7b_spec_decode,
    "llama70b_gqa_spec4": llama70b_gqa_spec_decode,
    "prefix_sharing_2040": lambda seed=4: prefix_sharing_sampling(2040, seed),
    "prefix_sharing_2048": lambda seed=4: prefix_sharing_sampling(2048, seed),
    "chunked_prefill_mixed": chunked_prefill_mixed,
}


def named(name: str, seed: Optional[int] = None) -> Workload:
    f = NAMED[name]
    return f() if seed is None else f(seed=seed)
