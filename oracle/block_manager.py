"""Plain-Python model of the KV-cache block manager -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only tests/ may import this module. It is the slow, obviously correct statement of the bookkeeping
that the C++ manager of the library (pa_block_manager.h) must reproduce exactly: same block for
every position, same copy-on-write pairs, same prefix-cache hits, same free-queue order. It shares
no code with the library. The free queue is a plain Python list (taking from its middle is a
linear search: correct, not fast), and the prefix cache is keyed by the exact tuple of every token
id from position 0 to the end of the block, so it can have no collisions.

Rules and where they come from:
  openeuler.csdn.net "高并发 AI 服务的内存瓶颈"
    - 机制1 按需分配: a sequence of L tokens holds ceil(L/16) blocks; a block is taken only when
      the last one is full.
    - Block Table 数据结构 (get_physical_indices): position i is stored at slot
      table[i // 16] * 16 + i % 16.
    - 机制 2 写时复制: forked samples share blocks by reference count; a private block is allocated
      only at divergence. Reading adopted for WHEN: a write into a partly filled block that others
      still hold copies it to a fresh block (the shared one loses a reference); the last holder
      writes in place.
  lilinji.mintlify.site lecture 34 "vLLM 生产级系统架构全景剖析…"
    - §1.2 allocate_slots appends into the last block while it has room, else takes a new block;
      free(req) releases blocks in strict reverse order; free blocks wait in one queue.
    - §2.2 a new request reuses the longest run of leading cached blocks, raising their counts.
      Reading adopted: only whole blocks are cached, and at most (n - 1) // 16 blocks of an
      n-token prompt are reused so that its last token is still computed.
    - §2.3 a block whose count drops to 0 keeps its contents and stays findable at the queue's
      tail; allocation takes from the head, evicting the least recently freed cached block; a block
      with count > 0 is never evicted.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

BLOCK = 16


class OutOfBlocks(Exception):
    """The free queue holds fewer blocks than a request needs (nothing was changed)."""


class _Seq:
    def __init__(self):
        self.table: List[int] = []
        self.num_tokens = 0
        self.ids: Optional[List[int]] = []   # every token id so far, None once one is unknown


class OracleBlockManager:
    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None,
                 prefix_caching: bool = False):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.prefix_caching = prefix_caching
        self.free_queue: List[int] = order           # head = index 0
        self.ref_cnt: List[int] = [0] * num_blocks
        self.cache: Dict[Tuple[int, ...], int] = {}  # prefix contents -> block
        self.key_of: Dict[int, Tuple[int, ...]] = {}  # block -> prefix contents it caches
        self.seqs: Dict[int, _Seq] = {}

    # -------------------------------------------------------------------------------- the pool
    def _take(self) -> int:
        b = self.free_queue.pop(0)
        if b in self.key_of:                          # evict from the prefix cache
            del self.cache[self.key_of.pop(b)]
        self.ref_cnt[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref_cnt[b] -= 1
        if self.ref_cnt[b] == 0:
            self.free_queue.append(b)

    # ---------------------------------------------------------------------------- sequences
    def add_sequence(self, sid: int) -> None:
        if sid in self.seqs:
            raise KeyError(sid)
        self.seqs[sid] = _Seq()

    def match_prefix(self, sid: int, token_ids: Sequence[int]) -> int:
        s = self.seqs[sid]
        if s.num_tokens != 0:
            raise ValueError("sequence is not empty")
        if not self.prefix_caching:
            return 0
        ids = [int(t) for t in token_ids]
        for j in range(max(0, (len(ids) - 1) // BLOCK)):
            key = tuple(ids[: (j + 1) * BLOCK])
            b = self.cache.get(key)
            if b is None:
                break
            if self.ref_cnt[b] == 0:
                self.free_queue.remove(b)
            self.ref_cnt[b] += 1
            s.table.append(b)
        s.num_tokens = len(s.table) * BLOCK
        s.ids = ids[: s.num_tokens]
        return s.num_tokens

    def allocate_slots(self, sid: int, num_tokens: int,
                       token_ids: Optional[Sequence[int]] = None
                       ) -> Tuple[List[int], Optional[Tuple[int, int]]]:
        s = self.seqs[sid]
        if num_tokens == 0:
            return [], None
        L0, L1 = s.num_tokens, s.num_tokens + num_tokens
        cow = L0 % BLOCK != 0 and self.ref_cnt[s.table[-1]] > 1
        need = -(-L1 // BLOCK) - len(s.table) + (1 if cow else 0)
        if need > len(self.free_queue):
            raise OutOfBlocks(need)
        pair = None
        if cow:
            shared = s.table[-1]
            fresh = self._take()
            self.ref_cnt[shared] -= 1
            s.table[-1] = fresh
            pair = (shared, fresh)
        known = token_ids is not None and s.ids is not None
        ids = s.ids + [int(t) for t in token_ids] if known else None
        slots = []
        for pos in range(L0, L1):          # one position at a time, in order
            if pos // BLOCK == len(s.table):
                s.table.append(self._take())
            slots.append(s.table[pos // BLOCK] * BLOCK + pos % BLOCK)
            if known and self.prefix_caching and (pos + 1) % BLOCK == 0:
                # this position completes its block: cache it unless those contents already are
                key, b = tuple(ids[: pos + 1]), s.table[pos // BLOCK]
                if key not in self.cache and b not in self.key_of:
                    self.cache[key] = b
                    self.key_of[b] = key
        s.ids = ids
        s.num_tokens = L1
        return slots, pair

    def fork(self, parent: int, child: int) -> None:
        if child in self.seqs:
            raise KeyError(child)
        p = self.seqs[parent]
        c = _Seq()
        c.table = list(p.table)
        c.num_tokens = p.num_tokens
        c.ids = None if p.ids is None else list(p.ids)
        for b in c.table:
            self.ref_cnt[b] += 1
        self.seqs[child] = c

    def free(self, sid: int) -> None:
        s = self.seqs.pop(sid)
        for b in reversed(s.table):
            self._release(b)

    # ------------------------------------------------------------------------------- queries
    def block_table(self, sid: int) -> List[int]:
        return list(self.seqs[sid].table)

    def sequence_info(self, sid: int) -> Tuple[int, int]:
        s = self.seqs[sid]
        return s.num_tokens, len(s.table)

    def is_cached(self, b: int) -> bool:
        return b in self.key_of
