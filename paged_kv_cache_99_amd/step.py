"""One step of the paged-attention hot path on the GPU.

The order is the one the pages give for a layer of a serving step: blocks that diverge are copied
on write (openeuler.csdn.net "高并发 AI 服务的内存瓶颈", 机制 2 写时复制), the step's new keys and
values are written into their slots (lecture 32 "LLM 在线推理两阶段" §3.1), then the decodes and the
prefill chunk attend their paged context (§5.4, §5.5: decodes first, the remaining token budget to a
prefill chunk). Every stage is a call into libpa.so; this class only holds the device buffers.

A step description is any object with the fields of a workload: dtype ("f16"/"bf16"), H_q, H_kv, D,
num_blocks, seq_lens, block_tables, k_cache, v_cache (16-bit words), new_key, new_value,
slot_mapping, copy_pairs, n_decode, query_decode, cu_q_lens, query_prefill, scale and optionally
partition_size.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}

# (row, query head) pairs per kv head up to which GpuStep sends short chunks to pa_decode_multi by
# default: one wave's two column groups. Measured on 64 sequences of U{1024..4096} tokens (bf16):
# 16 pairs 146-153 us and 32 pairs 160 us against 236-248 us for the chunk kernel; 64 pairs (two
# subgroups) 253 us against 245 us.
MULTI_AUTO_PAIRS = 32


def words_to_device(words: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload 16-bit words (numpy uint16) as a float16/bfloat16 tensor of the same shape."""
    a = np.ascontiguousarray(words, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(TORCH_DTYPE[dtype]).to(device)


def words_from_device(t: torch.Tensor) -> np.ndarray:
    """Download a float16/bfloat16 tensor as its 16-bit words (numpy uint16)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ints_to_device(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def check_shared_prefix(group_starts, prefix_lens, seq_lens, block_tables) -> None:
    """Host-side check of the groups given to pa_decode_shared_prefix{,_fp8}, on the numpy arrays
    the caller already holds: the library takes them as device memory and trusts them (a group
    that breaks them gives unspecified output). Raises ValueError naming the first violation.

    group_starts [G+1] starts at 0 and does not decrease; prefix_lens [B] is a multiple of 16, equal
    across the members of a group, at most every member's length, 0 outside the groups; the table
    entries of a group's shared blocks are the same for every member (openeuler.csdn.net
    "高并发 AI 服务的内存瓶颈", 机制 2: shared blocks are one physical copy)."""
    gs = np.asarray(group_starts, np.int64)
    pl = np.asarray(prefix_lens, np.int64)
    lens = np.asarray(seq_lens, np.int64)
    bt = np.asarray(block_tables)
    B = len(pl)
    if len(gs) == 0 or gs[0] != 0 or np.any(np.diff(gs) < 0) or gs[-1] > B:
        raise ValueError("group_starts must rise from 0 to at most num_seqs")
    if np.any(pl < 0) or np.any(pl % binding.BLOCK_SIZE) or np.any(pl > lens[:B]):
        raise ValueError("prefix_lens must be multiples of 16 within [0, seq_lens]")
    if np.any(pl[gs[-1]:] != 0):
        raise ValueError("a sequence in no group must have prefix_lens 0")
    for g in range(len(gs) - 1):
        a, b = int(gs[g]), int(gs[g + 1])
        if b == a:
            continue
        if np.any(pl[a:b] != pl[a]):
            raise ValueError(f"group {g}: members have different prefix_lens")
        nb = int(pl[a]) // binding.BLOCK_SIZE
        if nb and np.any(bt[a:b, :nb] != bt[a, :nb]):
            raise ValueError(f"group {g}: members do not share the prefix blocks")


class GpuStep:
    """Device buffers of one step and its stages.

    kv_cache="fp8" keeps the caches as E4M3 codes (lecture 34 §4.4) with scales k_scale, v_scale:
    fp8_pool gives their initial bytes (numpy uint8, the pool layout); without it the 16-bit pool is
    quantized on the device by the library's own FP8 scatter, each slot being one token. Such a
    step runs every stage over the E4M3 caches (the *_fp8 entry points). Its chunks are prefilled
    over a widened 16-bit copy of their context (pa_prefill_chunk_fp8 with a workspace) when that
    copy takes at most widen_limit bytes, else with the codes converted inside the tile loop.

    multi_token: chunks of at most 16 rows each (drafted tokens to verify, lecture 32 §5.4) go
    through pa_decode_multi, which reads each context like a decode, instead of the chunk kernel of
    pa_prefill_chunk; None picks it when every chunk is that short and a kv head's rows times its
    query heads come to at most MULTI_AUTO_PAIRS (more pairs re-read the context per 16 of them).
    """

    def __init__(self, w, device="cuda", partition_size: Optional[int] = None,
                 shared_prefix: bool = False, kv_cache: str = "auto", k_scale: float = 1.0,
                 v_scale: float = 1.0, fp8_pool=None, widen_limit: int = 1 << 30,
                 multi_token: Optional[bool] = None):
        self.w = w
        self.device = torch.device(device)
        dt, dev = w.dtype, self.device
        shape = (w.num_blocks, w.H_kv, binding.BLOCK_SIZE, w.D)
        self.fp8 = kv_cache == "fp8"
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.new_key = words_to_device(w.new_key, dt, dev)
        self.new_value = words_to_device(w.new_value, dt, dev)
        self.slot_mapping = ints_to_device(w.slot_mapping, dev)
        if self.fp8:
            if fp8_pool is not None:
                self.k_cache = torch.from_numpy(np.ascontiguousarray(fp8_pool[0], np.uint8)).to(
                    dev).view(shape)
                self.v_cache = torch.from_numpy(np.ascontiguousarray(fp8_pool[1], np.uint8)).to(
                    dev).view(shape)
            else:
                self.k_cache = torch.empty(shape, dtype=torch.uint8, device=dev)
                self.v_cache = torch.empty(shape, dtype=torch.uint8, device=dev)
                self.quantize_pool_on_device(w)
        else:
            self.k_cache = words_to_device(w.k_cache, dt, dev).view(shape)
            self.v_cache = words_to_device(w.v_cache, dt, dev).view(shape)
        self.copy_pairs = ints_to_device(np.asarray(w.copy_pairs).reshape(-1, 2), dev)
        nd = int(w.n_decode)
        self.n_decode = nd
        self.dec_tables = ints_to_device(w.block_tables[:nd], dev)
        self.dec_lens = ints_to_device(w.seq_lens[:nd], dev)
        self.dec_query = words_to_device(w.query_decode, dt, dev)
        self.dec_out = torch.empty_like(self.dec_query)
        self.max_seq_len = int(np.max(w.seq_lens[:nd])) if nd else 0
        if partition_size is None:
            partition_size = getattr(w, "partition_size", None)
        given_partition = partition_size  # the caller's or the workload's, else None
        meta = getattr(w, "meta", {}) or {}
        self.shared_prefix = bool(shared_prefix and "group_starts" in meta and nd)
        if partition_size is None:
            # read-once shared prefixes keep 512-token parts: their own-token ranges are short
            partition_size = 512 if self.shared_prefix else binding.default_partition_size(
                self.max_seq_len, w.H_q // w.H_kv)
        self.partition_size = int(partition_size)
        self.workspace = binding.alloc_decode_workspace(nd, w.H_q, w.D, self.max_seq_len,
                                                        self.partition_size, dev) if nd else None
        # read-once shared prefixes: groups of sequences that hold common leading blocks
        if self.shared_prefix:
            gs = np.asarray(meta["group_starts"], np.int32)
            pl = np.asarray(meta["shared_prefix"], np.int32)[:nd]
            check_shared_prefix(gs, pl, w.seq_lens[:nd], w.block_tables[:nd])
            self.group_starts = ints_to_device(gs, dev)
            self.prefix_lens = ints_to_device(pl, dev)
            self.max_group_size = int(np.max(np.diff(gs))) if len(gs) > 1 else 1
            self.max_prefix_len = int(pl.max()) if len(pl) else 0
            # the longest own range (positions after the shared prefix) sizes the own units
            self.max_own_len = int((np.asarray(w.seq_lens[:nd], np.int64) - pl).max())
            if self.partition_size == 0:
                self.partition_size = 512
            self.workspace = torch.empty(max(16, binding.decode_shared_prefix_workspace_size(
                nd, w.H_q, w.D, self.max_seq_len, self.max_prefix_len, self.partition_size)),
                dtype=torch.uint8, device=dev)
        self.pre_tables = ints_to_device(w.block_tables[nd:], dev)
        self.pre_lens = ints_to_device(w.seq_lens[nd:], dev)
        self.pre_cu = ints_to_device(w.cu_q_lens, dev)
        self.pre_query = words_to_device(w.query_prefill, dt, dev)
        self.pre_out = torch.empty_like(self.pre_query)
        cu = np.asarray(w.cu_q_lens)
        self.max_q_len = int(np.max(np.diff(cu))) if len(cu) > 1 else 0
        self.pre_max_seq_len = int(np.max(w.seq_lens[nd:])) if len(w.seq_lens) > nd else 0
        short = 0 < self.max_q_len <= binding.MULTI_MAX_ROWS
        if multi_token is None:
            multi_token = short and self.max_q_len * (w.H_q // w.H_kv) <= MULTI_AUTO_PAIRS
        self.multi_token = bool(multi_token)
        if self.multi_token and not short:
            raise ValueError(f"chunks of up to {self.max_q_len} rows: pa_decode_multi takes "
                             f"{binding.MULTI_MAX_ROWS}")
        self.multi_partition = (int(given_partition) if given_partition is not None else
                                binding.default_partition_size(self.pre_max_seq_len, 3))
        self.multi_workspace = binding.alloc_decode_multi_workspace(
            int(self.pre_tables.shape[0]), self.max_q_len, w.H_q, w.D, self.pre_max_seq_len,
            self.multi_partition, dev) if self.multi_token else None
        self.pre_workspace = None
        if self.fp8 and self.pre_query.shape[0] and not self.multi_token:
            n = binding.prefill_fp8_workspace_size(int(self.pre_tables.shape[0]),
                                                   int(self.pre_tables.shape[1]), w.H_kv, w.D)
            if 0 < n <= widen_limit:
                self.pre_workspace = torch.empty(n, dtype=torch.uint8, device=dev)

    def quantize_pool_on_device(self, w):
        """E4M3 caches holding the codes of the workload's 16-bit pool: every slot of the pool is
        written as one token by pa_reshape_and_cache_fp8 (slot s = block s / 16, offset s % 16)."""
        nb, H, D = w.num_blocks, w.H_kv, w.D
        slots = torch.arange(nb * binding.BLOCK_SIZE, dtype=torch.int32, device=self.device)

        def as_tokens(words):
            pool = words_to_device(words, w.dtype, self.device).view(nb, H, binding.BLOCK_SIZE, D)
            return pool.permute(0, 2, 1, 3).contiguous().view(nb * binding.BLOCK_SIZE, H, D)

        binding.reshape_and_cache_fp8(as_tokens(w.k_cache), as_tokens(w.v_cache), self.k_cache,
                                      self.v_cache, slots, self.k_scale, self.v_scale)
        torch.cuda.synchronize(self.device)

    # ---- stages
    def copy(self, stream=None):
        binding.copy_blocks(self.k_cache, self.v_cache, self.copy_pairs, stream)

    def scatter(self, stream=None):
        if self.fp8:
            binding.reshape_and_cache_fp8(self.new_key, self.new_value, self.k_cache, self.v_cache,
                                          self.slot_mapping, self.k_scale, self.v_scale, stream)
        else:
            binding.reshape_and_cache(self.new_key, self.new_value, self.k_cache, self.v_cache,
                                      self.slot_mapping, stream)

    def decode(self, stream=None):
        if self.n_decode and self.fp8 and self.shared_prefix:
            binding.decode_shared_prefix_fp8(
                self.dec_out, self.dec_query, self.k_cache, self.v_cache, self.dec_tables,
                self.dec_lens, self.max_seq_len, self.group_starts, self.prefix_lens,
                self.max_group_size, self.max_prefix_len, self.w.scale, self.k_scale,
                self.v_scale, self.partition_size, self.workspace, stream,
                max_own_len=self.max_own_len)
        elif self.n_decode and self.fp8:
            binding.decode_fp8(self.dec_out, self.dec_query, self.k_cache, self.v_cache,
                               self.dec_tables, self.dec_lens, self.max_seq_len, self.w.scale,
                               self.k_scale, self.v_scale, self.partition_size, self.workspace,
                               stream)
        elif self.n_decode and self.shared_prefix:
            binding.decode_shared_prefix(self.dec_out, self.dec_query, self.k_cache, self.v_cache,
                                         self.dec_tables, self.dec_lens, self.max_seq_len,
                                         self.group_starts, self.prefix_lens,
                                         self.max_group_size, self.max_prefix_len, self.w.scale,
                                         self.partition_size, self.workspace, stream,
                                         max_own_len=self.max_own_len)
        elif self.n_decode:
            binding.decode(self.dec_out, self.dec_query, self.k_cache, self.v_cache,
                           self.dec_tables, self.dec_lens, self.max_seq_len, self.w.scale,
                           self.partition_size, self.workspace, stream)

    def prefill(self, stream=None):
        if self.pre_query.shape[0] and self.multi_token:
            binding.decode_multi(self.pre_out, self.pre_query, self.k_cache, self.v_cache,
                                 self.pre_tables, self.pre_lens, self.pre_cu, self.max_q_len,
                                 self.pre_max_seq_len, self.w.scale, self.multi_partition,
                                 self.multi_workspace, stream,
                                 k_scale=self.k_scale if self.fp8 else None,
                                 v_scale=self.v_scale if self.fp8 else None)
        elif self.pre_query.shape[0] and self.fp8:
            binding.prefill_chunk_fp8(self.pre_out, self.pre_query, self.k_cache, self.v_cache,
                                      self.pre_tables, self.pre_lens, self.pre_cu, self.max_q_len,
                                      self.w.scale, self.k_scale, self.v_scale, stream,
                                      workspace=self.pre_workspace)
        elif self.pre_query.shape[0]:
            binding.prefill_chunk(self.pre_out, self.pre_query, self.k_cache, self.v_cache,
                                  self.pre_tables, self.pre_lens, self.pre_cu, self.max_q_len,
                                  self.w.scale, stream)

    def run(self, stream=None):
        self.copy(stream)
        self.scatter(stream)
        self.decode(stream)
        self.prefill(stream)

    def capture(self):
        """The whole step recorded once as a HIP graph (torch.cuda.CUDAGraph) and returned; each
        graph.replay() then launches the same kernels on the same buffers with one call. The
        library's entry points allocate nothing and issue no memset, so every node is a kernel.
        Replays read the buffers as they are at replay time: new tokens, queries, slots and
        seq_lens written in place are picked up, as long as each seq_lens[s] stays within the
        max_seq_len (and the shared-prefix bounds) the launch was sized for."""
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(graph):
            self.run()
        torch.cuda.synchronize(self.device)
        return graph
