"""ctypes binding of the host-side block manager (include/pa_block_manager.h).

Argument marshalling only: every decision -- which block a position lands in, copy-on-write,
prefix-cache hits, eviction order -- is taken by the C++ manager in libpa.so. Outputs are numpy
int32 arrays ready to be copied to the device for pa_reshape_and_cache (slots), pa_copy_blocks
(copy pairs) and pa_decode / pa_prefill_chunk (block tables).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import binding

PA_ERR_NO_BLOCKS = 5

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_i32p = ctypes.POINTER(ctypes.c_int32)
_configured = False


class NoFreeBlocks(binding.PAError):
    """The pool's free queue is too short for the request (PA_ERR_NO_BLOCKS)."""


def _lib():
    global _configured
    L = binding.lib()
    if not _configured:
        L.pa_bm_create.restype = _i32
        L.pa_bm_create.argtypes = [_i32, _p, _i32, ctypes.POINTER(_p)]
        L.pa_bm_destroy.restype = None
        L.pa_bm_destroy.argtypes = [_p]
        L.pa_bm_add_sequence.restype = _i32
        L.pa_bm_add_sequence.argtypes = [_p, _i64]
        L.pa_bm_match_prefix.restype = _i32
        L.pa_bm_match_prefix.argtypes = [_p, _i64, _p, _i32, _i32p]
        L.pa_bm_allocate_slots.restype = _i32
        L.pa_bm_allocate_slots.argtypes = [_p, _i64, _p, _i32, _p, _p]
        L.pa_bm_fork.restype = _i32
        L.pa_bm_fork.argtypes = [_p, _i64, _i64]
        L.pa_bm_free.restype = _i32
        L.pa_bm_free.argtypes = [_p, _i64]
        L.pa_bm_sequence_info.restype = _i32
        L.pa_bm_sequence_info.argtypes = [_p, _i64, _i32p, _i32p]
        L.pa_bm_block_tables.restype = _i32
        L.pa_bm_block_tables.argtypes = [_p, _p, _i32, _i32, _p]
        L.pa_bm_num_free_blocks.restype = _i32
        L.pa_bm_num_free_blocks.argtypes = [_p]
        L.pa_bm_free_queue.restype = _i32
        L.pa_bm_free_queue.argtypes = [_p, _p, _i32]
        L.pa_bm_block_state.restype = _i32
        L.pa_bm_block_state.argtypes = [_p, _i32, _i32p, _i32p]
        _configured = True
    return L


def _check(status: int) -> None:
    if status == 0:
        return
    L = binding.lib()
    msg = f"{L.pa_status_string(status).decode()}: {L.pa_last_error().decode()}"
    if status == PA_ERR_NO_BLOCKS:
        raise NoFreeBlocks(status, msg)
    raise binding.PAError(status, msg)


def _ids(token_ids, n: int) -> Tuple[Optional[np.ndarray], ctypes.c_void_p]:
    if token_ids is None:
        return None, None
    a = np.ascontiguousarray(token_ids, dtype=np.int32)
    if a.ndim != 1 or a.shape[0] != n:
        raise ValueError(f"token_ids must be 1-d of length {n}")
    return a, a.ctypes.data_as(_p)


class BlockManager:
    """Handle on one C++ block manager (pa_bm_*). Not thread-safe, like the manager itself."""

    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None,
                 prefix_caching: bool = False):
        L = _lib()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        h = _p()
        _check(L.pa_bm_create(int(num_blocks), None if order is None else order.ctypes.data_as(_p),
                              int(bool(prefix_caching)), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id: int) -> None:
        _check(_lib().pa_bm_add_sequence(self._h, int(seq_id)))

    def match_prefix(self, seq_id: int, token_ids: Sequence[int]) -> int:
        a, ptr = _ids(token_ids, len(token_ids))
        n = _i32()
        _check(_lib().pa_bm_match_prefix(self._h, int(seq_id), ptr, len(token_ids),
                                         ctypes.byref(n)))
        return int(n.value)

    def allocate_slots(self, seq_id: int, num_tokens: int,
                       token_ids: Optional[Sequence[int]] = None
                       ) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        """Slots of the appended positions, and the (src, dst) copy-on-write pair or None."""
        a, ptr = _ids(token_ids, num_tokens)
        slots = np.empty(max(1, num_tokens), dtype=np.int32)
        cow = np.empty(2, dtype=np.int32)
        _check(_lib().pa_bm_allocate_slots(self._h, int(seq_id), ptr, int(num_tokens),
                                           slots.ctypes.data_as(_p), cow.ctypes.data_as(_p)))
        pair = None if cow[0] < 0 else (int(cow[0]), int(cow[1]))
        return slots[:num_tokens], pair

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(_lib().pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def free(self, seq_id: int) -> None:
        _check(_lib().pa_bm_free(self._h, int(seq_id)))

    def sequence_info(self, seq_id: int) -> Tuple[int, int]:
        t, b = _i32(), _i32()
        _check(_lib().pa_bm_sequence_info(self._h, int(seq_id), ctypes.byref(t), ctypes.byref(b)))
        return int(t.value), int(b.value)

    def block_tables(self, seq_ids: Sequence[int], max_blocks_per_seq: int) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        out = np.empty((len(ids), max(1, max_blocks_per_seq)), dtype=np.int32)
        _check(_lib().pa_bm_block_tables(self._h, ids.ctypes.data_as(_p), len(ids),
                                         int(max_blocks_per_seq), out.ctypes.data_as(_p)))
        return out[:, :max_blocks_per_seq]

    def block_table(self, seq_id: int) -> np.ndarray:
        _, nb = self.sequence_info(seq_id)
        return self.block_tables([seq_id], nb)[0]

    @property
    def num_free_blocks(self) -> int:
        return int(_lib().pa_bm_num_free_blocks(self._h))

    def free_queue(self) -> np.ndarray:
        out = np.empty(max(1, self.num_blocks), dtype=np.int32)
        n = _lib().pa_bm_free_queue(self._h, out.ctypes.data_as(_p), self.num_blocks)
        if n < 0:
            raise binding.PAError(1, "pa_bm_free_queue failed")
        return out[:n]

    def block_state(self, block: int) -> Tuple[int, bool]:
        r, c = _i32(), _i32()
        _check(_lib().pa_bm_block_state(self._h, int(block), ctypes.byref(r), ctypes.byref(c)))
        return int(r.value), bool(c.value)
