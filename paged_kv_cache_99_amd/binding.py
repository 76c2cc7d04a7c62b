"""Thin ctypes binding of libpa.so (include/pa.h).

Argument marshalling only: each wrapper checks tensor shapes, dtypes and devices, passes raw device
pointers, sizes and the current HIP stream to the C entry point of the same name, and raises on a
non-zero status. All work runs in the library's HIP kernels; there is no fallback path, and loading
fails loudly when the library has not been built.

Tensors are torch tensors on the GPU: float16 or bfloat16 for queries/keys/values/caches/outputs,
int32 for tables and index arrays. Caches have shape [num_blocks, num_kv_heads, 16, head_dim]. The
``*_fp8`` wrappers take E4M3 caches as uint8 (or float8_e4m3fn) tensors of that shape.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
BLOCK_SIZE = 16
DECODE_SCRATCH_BYTES = 64 << 20  # PA_DECODE_SCRATCH_BYTES: pa_decode_noalloc's static scratch

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
_DTYPE = {torch.float16: 0, torch.bfloat16: 1}
PA_DTYPE_FP8_E4M3 = 2
FP8_CACHE_DTYPES = (torch.uint8, torch.float8_e4m3fn)

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int32
_f = ctypes.c_float
_sz = ctypes.c_size_t


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libpa.so. Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libpa.so not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.pa_status_string.restype = ctypes.c_char_p
        L.pa_status_string.argtypes = [_i]
        L.pa_last_error.restype = ctypes.c_char_p
        L.pa_last_error.argtypes = []
        L.pa_reshape_and_cache.restype = _i
        L.pa_reshape_and_cache.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p]
        L.pa_copy_blocks.restype = _i
        L.pa_copy_blocks.argtypes = [_i, _i, _i, _i, _p, _p, _p, _i, _p]
        L.pa_decode_workspace_size.restype = _sz
        L.pa_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        L.pa_decode.restype = _i
        L.pa_decode.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _f, _i,
                                _p, _sz, _p]
        L.pa_decode_noalloc.restype = _i
        L.pa_decode_noalloc.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i,
                                        _f, _i, _p]
        L.pa_decode_shared_prefix_workspace_size.restype = _sz
        L.pa_decode_shared_prefix_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
        L.pa_decode_shared_prefix.restype = _i
        L.pa_decode_shared_prefix.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i,
                                              _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _sz, _p]
        L.pa_decode_shared_prefix_fp8.restype = _i
        L.pa_decode_shared_prefix_fp8.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _i,
                                                  _i, _p, _p, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                                  _p, _sz, _p]
        L.pa_reshape_and_cache_fp8.restype = _i
        L.pa_reshape_and_cache_fp8.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _f, _f, _p]
        L.pa_decode_fp8.restype = _i
        L.pa_decode_fp8.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _i, _i, _i, _f, _f,
                                    _f, _i, _p, _sz, _p]
        L.pa_prefill_chunk_fp8_workspace_size.restype = _sz
        L.pa_prefill_chunk_fp8_workspace_size.argtypes = [_i, _i, _i, _i]
        L.pa_prefill_chunk_fp8.restype = _i
        L.pa_prefill_chunk_fp8.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _i, _i,
                                           _i, _i, _f, _f, _f, _p, _sz, _p]
        L.pa_prefill_chunk_tree.restype = _i
        L.pa_prefill_chunk_tree.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p,
                                            _i, _i, _i, _i, _f, _p]
        L.pa_prefill_chunk.restype = _i
        L.pa_prefill_chunk.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _i, _i, _i,
                                       _i, _f, _p]
        L.pa_decode_multi_workspace_size.restype = _sz
        L.pa_decode_multi_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
        L.pa_decode_multi.restype = _i
        L.pa_decode_multi.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p, _i, _i,
                                      _i, _i, _i, _f, _i, _p, _sz, _p]
        L.pa_decode_multi_fp8.restype = _i
        L.pa_decode_multi_fp8.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p, _i,
                                          _i, _i, _i, _i, _f, _f, _f, _i, _p, _sz, _p]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != PA_OK:
        L = lib()
        msg = L.pa_last_error().decode() or L.pa_status_string(status).decode()
        raise PAError(status, f"{L.pa_status_string(status).decode()}: {msg}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor, fp8: bool = False):
    """(pa dtype, num_blocks, num_kv_heads, head_dim) of a pair of caches: 16-bit caches, or with
    fp8 set E4M3 caches (dtype then PA_DTYPE_FP8_E4M3)."""
    if k_cache.dim() != 4 or k_cache.shape[2] != BLOCK_SIZE:
        raise ValueError("caches must be [num_blocks, num_kv_heads, 16, head_dim]")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache differ in shape or dtype")
    if fp8:
        if k_cache.dtype not in FP8_CACHE_DTYPES:
            raise ValueError(f"E4M3 cache dtype {k_cache.dtype}: uint8 or float8_e4m3fn")
    elif k_cache.dtype not in _DTYPE:
        raise ValueError(f"cache dtype {k_cache.dtype}: float16 or bfloat16")
    for t in (k_cache, v_cache):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("caches must be contiguous GPU tensors")
    nb, hkv, _, d = k_cache.shape
    return (PA_DTYPE_FP8_E4M3 if fp8 else _DTYPE[k_cache.dtype]), int(nb), int(hkv), int(d)


def _gpu(t: torch.Tensor, name: str, dtype=None) -> None:
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """pa_reshape_and_cache: key/value [T, H_kv, D] into the slots slot_mapping[T] (int32)."""
    dt, nb, hkv, d = _cache_dims(k_cache, v_cache)
    T = int(slot_mapping.shape[0])
    for t, n in ((key, "key"), (value, "value")):
        _gpu(t, n, k_cache.dtype)
        if tuple(t.shape) != (T, hkv, d):
            raise ValueError(f"{n} must be [{T}, {hkv}, {d}]")
    _gpu(slot_mapping, "slot_mapping", torch.int32)
    _check(lib().pa_reshape_and_cache(dt, nb, hkv, d, key.data_ptr(), value.data_ptr(),
                                      k_cache.data_ptr(), v_cache.data_ptr(),
                                      slot_mapping.data_ptr(), T, _stream(stream)))


def copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """pa_copy_blocks: whole-block copies of the (src, dst) rows of block_mapping [N, 2] int32;
    16-bit or E4M3 (uint8 / float8_e4m3fn) caches."""
    dt, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=k_cache.dtype in FP8_CACHE_DTYPES)
    _gpu(block_mapping, "block_mapping", torch.int32)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N, 2]")
    n = int(block_mapping.shape[0])
    _check(lib().pa_copy_blocks(dt, nb, hkv, d, k_cache.data_ptr(), v_cache.data_ptr(),
                                block_mapping.data_ptr() if n else None, n, _stream(stream)))


def decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size) -> int:
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                              partition_size))


def default_partition_size(max_seq_len: int, group: int = 1) -> int:
    """Tokens per split-K part for pa_decode: short contexts run unsplit; head groups of 1-2
    (the vector-ALU kernel) take 1024-token parts over contexts of more than 2048 tokens, where
    the library runs eight-wave units on them; everything else 512-token parts."""
    if max_seq_len <= 512:
        return 0
    return 1024 if group <= 2 and max_seq_len > 2048 else 512


def alloc_decode_workspace(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size,
                           device=None) -> Optional[torch.Tensor]:
    n = decode_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def decode(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int, scale: float,
           partition_size: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> None:
    """pa_decode: out/query [B, H_q, D]; block_tables [B, max_blocks] int32; seq_lens [B] int32."""
    dt, nb, hkv, d = _cache_dims(k_cache, v_cache)
    B, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, k_cache.dtype)
        if tuple(t.shape) != (B, hq, d):
            raise ValueError(f"{n} must be [{B}, {hq}, {d}]")
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(seq_lens, "seq_lens", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and seq_lens [B]")
    if partition_size is None:
        partition_size = default_partition_size(max_seq_len, hq // hkv)
    need = decode_workspace_size(B, hq, d, max_seq_len, partition_size)
    if need and workspace is None:
        workspace = alloc_decode_workspace(B, hq, d, max_seq_len, partition_size, query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(), k_cache.data_ptr(),
                           v_cache.data_ptr(), block_tables.data_ptr(),
                           int(block_tables.shape[1]), seq_lens.data_ptr(), B, int(max_seq_len),
                           hq, float(scale), int(partition_size), _ptr(workspace), ws_bytes,
                           _stream(stream)))


def decode_noalloc(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
                   scale: float, partition_size: Optional[int] = None, stream=None) -> None:
    """pa_decode_noalloc: pa_decode with its partial results in the library's static scratch (no
    workspace, nothing allocated); arguments as decode."""
    dt, nb, hkv, d = _cache_dims(k_cache, v_cache)
    B, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, k_cache.dtype)
        if tuple(t.shape) != (B, hq, d):
            raise ValueError(f"{n} must be [{B}, {hq}, {d}]")
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(seq_lens, "seq_lens", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and seq_lens [B]")
    if partition_size is None:
        partition_size = default_partition_size(max_seq_len, hq // hkv)
    _check(lib().pa_decode_noalloc(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(),
                                   k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                                   int(block_tables.shape[1]), seq_lens.data_ptr(), B,
                                   int(max_seq_len), hq, float(scale), int(partition_size),
                                   _stream(stream)))


def decode_shared_prefix_workspace_size(num_seqs, num_q_heads, head_dim, max_seq_len,
                                        max_prefix_len, partition_size) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_seq_len, max_prefix_len,
                                                            partition_size))


def _shared_prefix_args(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len,
                        group_starts, prefix_lens, max_group_size, max_prefix_len,
                        partition_size, workspace, fp8, max_own_len=0):
    """Checked arguments of pa_decode_shared_prefix{,_fp8} up to num_q_heads, and the workspace
    (pointer, bytes)."""
    _, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=fp8)
    dt = _act_dtype(query, "query")
    if not fp8 and query.dtype != k_cache.dtype:
        raise ValueError("query dtype differs from the caches'")
    B, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, query.dtype)
        if tuple(t.shape) != (B, hq, d):
            raise ValueError(f"{n} must be [{B}, {hq}, {d}]")
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"),
                 (group_starts, "group_starts"), (prefix_lens, "prefix_lens")):
        _gpu(t, n, torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,) \
            or prefix_lens.shape != (B,) or group_starts.dim() != 1:
        raise ValueError("block_tables [B, max_blocks], seq_lens and prefix_lens [B], "
                         "group_starts [G + 1]")
    G = int(group_starts.shape[0]) - 1
    need = decode_shared_prefix_workspace_size(B, hq, d, max_seq_len, max_prefix_len,
                                               partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=query.device)
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    args = (dt, nb, hkv, d, out.data_ptr(), query.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), block_tables.data_ptr(), int(block_tables.shape[1]),
            seq_lens.data_ptr(), B, int(max_seq_len), group_starts.data_ptr(),
            prefix_lens.data_ptr(), max(G, 0), int(max_group_size), int(max_prefix_len),
            int(max_own_len), hq)
    return args, ws


def decode_shared_prefix(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
                         group_starts, prefix_lens, max_group_size: int, max_prefix_len: int,
                         scale: float, partition_size: int = 512,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         max_own_len: int = 0) -> None:
    """pa_decode_shared_prefix: pa_decode whose groups of sequences (group_starts [G+1], int32)
    read their common leading blocks (prefix_lens [B], int32) once. max_own_len bounds every
    seq_lens[s] - prefix_lens[s] (0: max_seq_len)."""
    args, ws = _shared_prefix_args(out, query, k_cache, v_cache, block_tables, seq_lens,
                                   max_seq_len, group_starts, prefix_lens, max_group_size,
                                   max_prefix_len, partition_size, workspace, False, max_own_len)
    _check(lib().pa_decode_shared_prefix(*args, float(scale), int(partition_size), *ws,
                                         _stream(stream)))


def decode_shared_prefix_fp8(out, query, k_cache, v_cache, block_tables, seq_lens,
                             max_seq_len: int, group_starts, prefix_lens, max_group_size: int,
                             max_prefix_len: int, scale: float, k_scale: float, v_scale: float,
                             partition_size: int = 512, workspace: Optional[torch.Tensor] = None,
                             stream=None, max_own_len: int = 0) -> None:
    """pa_decode_shared_prefix_fp8: decode_shared_prefix over E4M3 caches (uint8 or
    float8_e4m3fn; elements = code value * k_scale / v_scale)."""
    args, ws = _shared_prefix_args(out, query, k_cache, v_cache, block_tables, seq_lens,
                                   max_seq_len, group_starts, prefix_lens, max_group_size,
                                   max_prefix_len, partition_size, workspace, True, max_own_len)
    _check(lib().pa_decode_shared_prefix_fp8(*args, float(scale), float(k_scale), float(v_scale),
                                             int(partition_size), *ws, _stream(stream)))


def prefill_chunk(out, query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens,
                  max_q_len: int, scale: float, stream=None, tree_mask=None) -> None:
    """pa_prefill_chunk: out/query [total_q, H_q, D]; cu_q_lens [S+1]; seq_lens [S]; tables
    [S, max_blocks]. With tree_mask (int64 or uint64 [total_q], the 64-bit mask of each row)
    pa_prefill_chunk_tree: chunks of drafted-token trees, at most 64 rows each."""
    dt, nb, hkv, d = _cache_dims(k_cache, v_cache)
    tq, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, k_cache.dtype)
        if tuple(t.shape) != (tq, hq, d):
            raise ValueError(f"{n} must be [{tq}, {hq}, {d}]")
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"), (cu_q_lens, "cu_q_lens")):
        _gpu(t, n, torch.int32)
    S = int(seq_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != S or cu_q_lens.shape != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and cu_q_lens [S + 1]")
    if tree_mask is not None:
        if not (tree_mask.is_cuda and tree_mask.is_contiguous()) or \
                tree_mask.dtype not in (torch.int64, torch.uint64) or tuple(tree_mask.shape) != (tq,):
            raise ValueError(f"tree_mask must be a contiguous int64/uint64 GPU tensor [{tq}]")
        _check(lib().pa_prefill_chunk_tree(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(),
                                           k_cache.data_ptr(), v_cache.data_ptr(),
                                           block_tables.data_ptr(), int(block_tables.shape[1]),
                                           seq_lens.data_ptr(), cu_q_lens.data_ptr(),
                                           tree_mask.data_ptr(), S, tq, int(max_q_len), hq,
                                           float(scale), _stream(stream)))
        return
    _check(lib().pa_prefill_chunk(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(),
                                  k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                                  int(block_tables.shape[1]), seq_lens.data_ptr(),
                                  cu_q_lens.data_ptr(), S, tq, int(max_q_len), hq, float(scale),
                                  _stream(stream)))


def prefill_fp8_workspace_size(num_seqs: int, max_blocks_per_seq: int, num_kv_heads: int,
                               head_dim: int) -> int:
    """pa_prefill_chunk_fp8_workspace_size: bytes of the widened 16-bit copy of the context."""
    return int(lib().pa_prefill_chunk_fp8_workspace_size(num_seqs, max_blocks_per_seq,
                                                         num_kv_heads, head_dim))


def alloc_prefill_fp8_workspace(num_seqs, max_blocks_per_seq, num_kv_heads, head_dim,
                                device=None) -> Optional[torch.Tensor]:
    n = prefill_fp8_workspace_size(num_seqs, max_blocks_per_seq, num_kv_heads, head_dim)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def prefill_chunk_fp8(out, query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens,
                      max_q_len: int, scale: float, k_scale: float, v_scale: float,
                      stream=None, workspace: Optional[torch.Tensor] = None) -> None:
    """pa_prefill_chunk_fp8: pa_prefill_chunk over E4M3 caches (uint8 or float8_e4m3fn;
    elements = code value * k_scale / v_scale); query/out float16 or bfloat16. With a workspace
    (alloc_prefill_fp8_workspace) the context is first widened to 16 bits and read by the 16-bit
    kernel; the results are the same bits."""
    _, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=True)
    dt = _act_dtype(query, "query")
    tq, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, query.dtype)
        if tuple(t.shape) != (tq, hq, d):
            raise ValueError(f"{n} must be [{tq}, {hq}, {d}]")
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"), (cu_q_lens, "cu_q_lens")):
        _gpu(t, n, torch.int32)
    S = int(seq_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != S or cu_q_lens.shape != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and cu_q_lens [S + 1]")
    if workspace is not None:
        _gpu(workspace, "workspace", torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_prefill_chunk_fp8(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(),
                                      k_cache.data_ptr(), v_cache.data_ptr(),
                                      block_tables.data_ptr(), int(block_tables.shape[1]),
                                      seq_lens.data_ptr(), cu_q_lens.data_ptr(), S, tq,
                                      int(max_q_len), hq, float(scale), float(k_scale),
                                      float(v_scale), _ptr(workspace), ws_bytes, _stream(stream)))


# ------------------------------------------------------------------------- multi-token decode
MULTI_MAX_ROWS = 16  # rows per sequence pa_decode_multi takes


def decode_multi_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim, max_seq_len,
                                partition_size) -> int:
    return int(lib().pa_decode_multi_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim,
                                                    max_seq_len, partition_size))


def alloc_decode_multi_workspace(num_seqs, max_q_len, num_q_heads, head_dim, max_seq_len,
                                 partition_size, device=None) -> Optional[torch.Tensor]:
    n = decode_multi_workspace_size(num_seqs, max_q_len, num_q_heads, head_dim, max_seq_len,
                                    partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def decode_multi(out, query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens, max_q_len: int,
                 max_seq_len: int, scale: float, partition_size: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None, tree_mask=None,
                 k_scale: Optional[float] = None, v_scale: Optional[float] = None) -> None:
    """pa_decode_multi (pa_decode_multi_fp8 when k_scale and v_scale are given, over E4M3 caches):
    up to 16 query rows per sequence, out/query [total_q, H_q, D] by cu_q_lens [S+1]; seq_lens [S];
    tables [S, max_blocks]; tree_mask None or int64/uint64 [total_q]. The result is
    prefill_chunk's for the same rows."""
    fp8 = k_scale is not None or v_scale is not None
    _, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=fp8)
    dt = _act_dtype(query, "query")
    tq, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, query.dtype)
        if tuple(t.shape) != (tq, hq, d):
            raise ValueError(f"{n} must be [{tq}, {hq}, {d}]")
    if not fp8 and query.dtype != k_cache.dtype:
        raise ValueError("query and the 16-bit caches differ in dtype")
    for t, n in ((block_tables, "block_tables"), (seq_lens, "seq_lens"), (cu_q_lens, "cu_q_lens")):
        _gpu(t, n, torch.int32)
    S = int(seq_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != S or cu_q_lens.shape != (S + 1,):
        raise ValueError("block_tables must be [S, max_blocks] and cu_q_lens [S + 1]")
    if tree_mask is not None:
        if not (tree_mask.is_cuda and tree_mask.is_contiguous()) or \
                tree_mask.dtype not in (torch.int64, torch.uint64) or tuple(tree_mask.shape) != (tq,):
            raise ValueError(f"tree_mask must be a contiguous int64/uint64 GPU tensor [{tq}]")
    if partition_size is None:
        partition_size = default_partition_size(max_seq_len, 3)
    need = decode_multi_workspace_size(S, max_q_len, hq, d, max_seq_len, partition_size)
    if need and workspace is None:
        workspace = alloc_decode_multi_workspace(S, max_q_len, hq, d, max_seq_len, partition_size,
                                                 query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [dt, nb, hkv, d, out.data_ptr(), query.data_ptr(), k_cache.data_ptr(),
            v_cache.data_ptr(), block_tables.data_ptr(), int(block_tables.shape[1]),
            seq_lens.data_ptr(), cu_q_lens.data_ptr(), _ptr(tree_mask), S, tq, int(max_q_len),
            int(max_seq_len), hq, float(scale)]
    if fp8:
        _check(lib().pa_decode_multi_fp8(*args, float(k_scale), float(v_scale),
                                         int(partition_size), _ptr(workspace), ws_bytes,
                                         _stream(stream)))
    else:
        _check(lib().pa_decode_multi(*args, int(partition_size), _ptr(workspace), ws_bytes,
                                     _stream(stream)))


# ------------------------------------------------------------------------- E4M3 caches
def _act_dtype(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DTYPE:
        raise ValueError(f"{name} dtype {t.dtype}: float16 or bfloat16")
    return _DTYPE[t.dtype]


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale: float,
                          v_scale: float, stream=None) -> None:
    """pa_reshape_and_cache_fp8: key/value [T, H_kv, D] (float16/bfloat16) quantized to E4M3 codes
    of x / k_scale and x / v_scale in the slots slot_mapping[T]."""
    _, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=True)
    dt = _act_dtype(key, "key")
    T = int(slot_mapping.shape[0])
    for t, n in ((key, "key"), (value, "value")):
        _gpu(t, n, key.dtype)
        if tuple(t.shape) != (T, hkv, d):
            raise ValueError(f"{n} must be [{T}, {hkv}, {d}]")
    _gpu(slot_mapping, "slot_mapping", torch.int32)
    _check(lib().pa_reshape_and_cache_fp8(dt, nb, hkv, d, key.data_ptr(), value.data_ptr(),
                                          k_cache.data_ptr(), v_cache.data_ptr(),
                                          slot_mapping.data_ptr(), T, float(k_scale),
                                          float(v_scale), _stream(stream)))


def decode_fp8(out, query, k_cache, v_cache, block_tables, seq_lens, max_seq_len: int,
               scale: float, k_scale: float, v_scale: float,
               partition_size: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> None:
    """pa_decode_fp8: pa_decode over E4M3 caches (elements = code value * k_scale / v_scale)."""
    _, nb, hkv, d = _cache_dims(k_cache, v_cache, fp8=True)
    dt = _act_dtype(query, "query")
    B, hq = int(query.shape[0]), int(query.shape[1])
    for t, n in ((query, "query"), (out, "out")):
        _gpu(t, n, query.dtype)
        if tuple(t.shape) != (B, hq, d):
            raise ValueError(f"{n} must be [{B}, {hq}, {d}]")
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(seq_lens, "seq_lens", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and seq_lens [B]")
    if partition_size is None:
        partition_size = default_partition_size(max_seq_len, hq // hkv)
    need = decode_workspace_size(B, hq, d, max_seq_len, partition_size)
    if need and workspace is None:
        workspace = alloc_decode_workspace(B, hq, d, max_seq_len, partition_size, query.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_decode_fp8(dt, nb, hkv, d, out.data_ptr(), query.data_ptr(),
                               k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                               int(block_tables.shape[1]), seq_lens.data_ptr(), B,
                               int(max_seq_len), hq, float(scale), float(k_scale), float(v_scale),
                               int(partition_size), _ptr(workspace), ws_bytes, _stream(stream)))
