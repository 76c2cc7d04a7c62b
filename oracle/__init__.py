"""CPU float64 oracle of the paged-attention hot path -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package. It wraps the plain C implementation in ``pa_oracle.c`` (see that file's header for the
passages of the pages each function follows) with numpy-facing helpers. It imports nothing from the
HIP library and the library imports nothing from here.

Every pool/cache argument is the 16-bit word array (numpy uint16) in the layout
[num_blocks][num_kv_heads][16][head_dim]; queries, keys and values are uint16 words as well, and
``dtype`` is "f16" or "bf16". The ``*_fp8`` functions take caches of E4M3 codes (numpy uint8) in
the same layout, with one scale per cache.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")
_DTYPES = {"f16": 0, "bf16": 1}
BLOCK = 16

OK, BAD_INDEX, DUP_SLOT, BAD_MAPPING, BAD_ARG, NO_MEM = range(6)

_lib = None

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(dtype=np.uint64, flags="C_CONTIGUOUS")
_c_int, _c_double = ctypes.c_int, ctypes.c_double


def lib():
    """Load libpa_oracle.so (built by oracle/build.py or __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"oracle library missing: {_LIB_PATH}; run `python oracle/build.py`")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_to_double.restype = _c_double
        L.oracle_to_double.argtypes = [ctypes.c_uint16, _c_int]
        L.oracle_reshape_and_cache.argtypes = [_u16p, _u16p, _u16p, _u16p, _i32p, _c_int, _c_int,
                                               _c_int, _c_int]
        L.oracle_copy_blocks.argtypes = [_u16p, _u16p, _i32p, _c_int, _c_int, _c_int, _c_int]
        L.oracle_gather.argtypes = [_u16p, _i32p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _f64p]
        L.oracle_attention.argtypes = [_f64p, _f64p, _f64p, _c_int, _c_int, _c_double, _f64p]
        L.oracle_decode.argtypes = [_u16p, _u16p, _u16p, _i32p, _c_int, _i32p, _c_int, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_double, ctypes.c_void_p,
                                    _c_int, _c_int, _f64p]
        L.oracle_prefill.argtypes = [_u16p, _u16p, _u16p, _i32p, _c_int, _i32p, _i32p, _c_int,
                                     _c_int, _c_int, _c_int, _c_int, _c_int, _c_double,
                                     ctypes.c_void_p, _c_int, _c_int, _f64p]
        L.oracle_prefill_fp8.argtypes = [_u16p, _u8p, _u8p, _i32p, _c_int, _i32p, _i32p, _c_int,
                                         _c_int, _c_int, _c_int, _c_int, _c_int, _c_double,
                                         _c_double, _c_double, ctypes.c_void_p, _c_int, _c_int,
                                         _f64p]
        L.oracle_prefill_tree.argtypes = [_u16p, _u16p, _u16p, _i32p, _c_int, _i32p, _i32p,
                                          _u64p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_double, _c_int, _f64p]
        L.oracle_split_merge.argtypes = [_f64p, _f64p, _f64p, _c_int, _c_int, _c_double, _c_int,
                                         _f64p]
        L.oracle_poison_free_slots.restype = ctypes.c_long
        L.oracle_poison_free_slots.argtypes = [_u16p, _u16p, _i32p, _c_int, _i32p, _c_int, _c_int,
                                               _c_int, _c_int, ctypes.c_uint16]
        L.oracle_poison_free_slots_fp8.restype = ctypes.c_long
        L.oracle_poison_free_slots_fp8.argtypes = [_u8p, _u8p, _i32p, _c_int, _i32p, _c_int,
                                                   _c_int, _c_int, _c_int, ctypes.c_uint8]
        L.oracle_e4m3_to_double.restype = _c_double
        L.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_from_float.restype = ctypes.c_uint8
        L.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
        L.oracle_quantize_e4m3.restype = ctypes.c_uint8
        L.oracle_quantize_e4m3.argtypes = [ctypes.c_uint16, _c_int, ctypes.c_float]
        L.oracle_quantize_e4m3_n.restype = None
        L.oracle_quantize_e4m3_n.argtypes = [_u16p, ctypes.c_long, _c_int, ctypes.c_float, _u8p]
        L.oracle_reshape_and_cache_fp8.argtypes = [_u16p, _u16p, _u8p, _u8p, _i32p, _c_int,
                                                   _c_int, _c_int, _c_int, _c_int, ctypes.c_float,
                                                   ctypes.c_float]
        L.oracle_copy_blocks_fp8.argtypes = [_u8p, _u8p, _i32p, _c_int, _c_int, _c_int, _c_int]
        L.oracle_gather_fp8.argtypes = [_u8p, _i32p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _c_double, _f64p]
        L.oracle_decode_fp8.argtypes = [_u16p, _u8p, _u8p, _i32p, _c_int, _i32p, _c_int, _c_int,
                                        _c_int, _c_int, _c_int, _c_int, _c_double, _c_double,
                                        _c_double, ctypes.c_void_p, _c_int, _c_int, _f64p]
        L.oracle_max_threads.restype = _c_int
        _lib = L
    return _lib


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc, what):
    if rc != OK:
        raise ValueError(f"oracle {what}: status {rc}")


def to_double(bits, dtype):
    """O1: decode 16-bit words (any shape) to float64, element by element."""
    flat = _u16(bits).ravel()
    f = lib().oracle_to_double
    code = _DTYPES[dtype]
    return np.array([f(int(b), code) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_blocks, H_kv, D):
    """O2: scatter, in place on copies of the caches; returns (k_cache', v_cache')."""
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    sm = _i32(slot_mapping)
    rc = lib().oracle_reshape_and_cache(_u16(key), _u16(value), kc, vc, sm, len(sm), num_blocks,
                                        H_kv, D)
    _check(rc, "reshape_and_cache")
    return kc, vc


def copy_blocks(k_cache, v_cache, mapping, num_blocks, H_kv, D):
    """O3: whole-block copies of (src, dst) pairs; returns new (k_cache', v_cache')."""
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    mp = _i32(np.asarray(mapping).reshape(-1, 2))
    rc = lib().oracle_copy_blocks(kc, vc, mp, mp.shape[0], num_blocks, H_kv, D)
    _check(rc, "copy_blocks")
    return kc, vc


def gather(cache, table_row, L, kvh, num_blocks, H_kv, D, dtype):
    """O4: contiguous float64 rows [L][D] of kv head kvh of one sequence."""
    out = np.zeros((max(L, 1), D), dtype=np.float64)
    rc = lib().oracle_gather(_u16(cache), _i32(table_row), L, kvh, num_blocks, H_kv, D,
                             _DTYPES[dtype], out)
    _check(rc, "gather")
    return out[:L]


def attention(q, K, V, scale):
    """O5: softmax(scale q K^T) V for one query row over contiguous float64 rows."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    L, D = (K.shape[0], q.shape[0])
    out = np.zeros(D, dtype=np.float64)
    Kc = K if L else np.zeros((1, D))
    Vc = V if L else np.zeros((1, D))
    rc = lib().oracle_attention(q, _f64(Kc), _f64(Vc), L, D, scale, out)
    _check(rc, "attention")
    return out


def split_merge(q, K, V, scale, part):
    """O8: the partitioned computation merged by running-max rescaling."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    L, D = K.shape[0], q.shape[0]
    out = np.zeros(D, dtype=np.float64)
    Kc = K if L else np.zeros((1, D))
    Vc = V if L else np.zeros((1, D))
    rc = lib().oracle_split_merge(q, _f64(Kc), _f64(Vc), L, D, scale, part, out)
    _check(rc, "split_merge")
    return out


def decode(query, k_cache, v_cache, block_tables, seq_lens, H_q, H_kv, D, num_blocks, dtype,
           scale, pairs=None, nthreads=0):
    """O6: paged decode. query [B][H_q][D] words. Returns float64 [B][H_q][D], or [n][D] for an
    explicit list of (seq, head) pairs."""
    bt = _i32(block_tables)
    B = bt.shape[0]
    if pairs is None:
        out = np.zeros((B, H_q, D), dtype=np.float64)
        pp, n = None, 0
    else:
        pairs = _i32(np.asarray(pairs).reshape(-1, 2))
        out = np.zeros((pairs.shape[0], D), dtype=np.float64)
        pp, n = pairs.ctypes.data_as(ctypes.c_void_p), pairs.shape[0]
    rc = lib().oracle_decode(_u16(query), _u16(k_cache), _u16(v_cache), bt, bt.shape[1],
                             _i32(seq_lens), B, H_q, H_kv, D, num_blocks, _DTYPES[dtype], scale,
                             pp, n, nthreads, out)
    _check(rc, "decode")
    return out


def prefill(query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens, H_q, H_kv, D, num_blocks,
            dtype, scale, rows=None, nthreads=0):
    """O7: paged causal prefill of chunks. query [total_q][H_q][D] words. Returns float64
    [total_q][H_q][D], or [n][D] for an explicit list of (row, head) pairs."""
    bt = _i32(block_tables)
    cu = _i32(cu_q_lens)
    S = bt.shape[0]
    if rows is None:
        out = np.zeros((int(cu[-1]), H_q, D), dtype=np.float64)
        rp, n = None, 0
    else:
        rows = _i32(np.asarray(rows).reshape(-1, 2))
        out = np.zeros((rows.shape[0], D), dtype=np.float64)
        rp, n = rows.ctypes.data_as(ctypes.c_void_p), rows.shape[0]
    rc = lib().oracle_prefill(_u16(query), _u16(k_cache), _u16(v_cache), bt, bt.shape[1],
                              _i32(seq_lens), cu, S, H_q, H_kv, D, num_blocks, _DTYPES[dtype],
                              scale, rp, n, nthreads, out)
    _check(rc, "prefill")
    return out


def prefill_tree(query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens, tree_mask, H_q, H_kv,
                 D, num_blocks, dtype, scale, nthreads=0):
    """T1: paged prefill of drafted-token trees (at most 64 rows per sequence): row i of a sequence
    sees its context and chunk rows j <= i whose bit j is set in tree_mask[row] (uint64 [total_q]).
    query [total_q][H_q][D] words. Returns float64 [total_q][H_q][D]."""
    bt = _i32(block_tables)
    cu = _i32(cu_q_lens)
    tm = np.ascontiguousarray(tree_mask, dtype=np.uint64)
    out = np.zeros((int(cu[-1]), H_q, D), dtype=np.float64)
    rc = lib().oracle_prefill_tree(_u16(query), _u16(k_cache), _u16(v_cache), bt, bt.shape[1],
                                   _i32(seq_lens), cu, tm, bt.shape[0], H_q, H_kv, D, num_blocks,
                                   _DTYPES[dtype], scale, nthreads, out)
    _check(rc, "prefill_tree")
    return out


NAN_WORD = {"f16": 0x7E00, "bf16": 0x7FC0}


def poison_free_slots(k_cache, v_cache, block_tables, seq_lens, num_blocks, H_kv, D, dtype):
    """Return copies of the caches with every slot that holds no valid token set to NaN."""
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    bt = _i32(block_tables)
    n = lib().oracle_poison_free_slots(kc, vc, bt, bt.shape[1], _i32(seq_lens), bt.shape[0],
                                       num_blocks, H_kv, D, NAN_WORD[dtype])
    if n < 0:
        raise ValueError("oracle poison_free_slots: bad table entry")
    return kc, vc


# ------------------------------------------------------------------------- FP8 (E4M3) caches
NAN_E4M3 = 0x7F


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def e4m3_to_double(codes):
    """F1: E4M3 codes (any shape) to float64, element by element."""
    flat = _u8(codes).ravel()
    f = lib().oracle_e4m3_to_double
    return np.array([f(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def e4m3_from_float(x):
    """F1: float32 values (any shape) to E4M3 codes: nearest, ties to even, saturating at 448."""
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().oracle_e4m3_from_float
    return np.array([f(float(v)) for v in flat], dtype=np.uint8).reshape(np.shape(x))


def quantize_e4m3(words, dtype, scale):
    """F2: 16-bit words (any shape) to the E4M3 codes of x / scale (division in float32)."""
    flat = _u16(words).ravel()
    out = np.empty(flat.size, dtype=np.uint8)
    lib().oracle_quantize_e4m3_n(flat, flat.size, _DTYPES[dtype], float(scale), out)
    return out.reshape(np.shape(words))


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, num_blocks, H_kv, D, dtype,
                          k_scale, v_scale):
    """F3: quantizing scatter into copies of E4M3 caches; returns (k_cache', v_cache')."""
    kc, vc = _u8(k_cache).copy(), _u8(v_cache).copy()
    sm = _i32(slot_mapping)
    rc = lib().oracle_reshape_and_cache_fp8(_u16(key), _u16(value), kc, vc, sm, len(sm),
                                            num_blocks, H_kv, D, _DTYPES[dtype], k_scale, v_scale)
    _check(rc, "reshape_and_cache_fp8")
    return kc, vc


def copy_blocks_fp8(k_cache, v_cache, mapping, num_blocks, H_kv, D):
    """F4: whole-block copies on E4M3 caches; returns new (k_cache', v_cache')."""
    kc, vc = _u8(k_cache).copy(), _u8(v_cache).copy()
    mp = _i32(np.asarray(mapping).reshape(-1, 2))
    rc = lib().oracle_copy_blocks_fp8(kc, vc, mp, mp.shape[0], num_blocks, H_kv, D)
    _check(rc, "copy_blocks_fp8")
    return kc, vc


def gather_fp8(cache, table_row, L, kvh, num_blocks, H_kv, D, cache_scale):
    """F5: contiguous float64 rows [L][D] of an E4M3 cache, times its scale."""
    out = np.zeros((max(L, 1), D), dtype=np.float64)
    rc = lib().oracle_gather_fp8(_u8(cache), _i32(table_row), L, kvh, num_blocks, H_kv, D,
                                 cache_scale, out)
    _check(rc, "gather_fp8")
    return out[:L]


def decode_fp8(query, k_cache, v_cache, block_tables, seq_lens, H_q, H_kv, D, num_blocks, dtype,
               scale, k_scale, v_scale, pairs=None, nthreads=0):
    """F6: paged decode over E4M3 caches. query [B][H_q][D] words of dtype."""
    bt = _i32(block_tables)
    B = bt.shape[0]
    if pairs is None:
        out = np.zeros((B, H_q, D), dtype=np.float64)
        pp, n = None, 0
    else:
        pairs = _i32(np.asarray(pairs).reshape(-1, 2))
        out = np.zeros((pairs.shape[0], D), dtype=np.float64)
        pp, n = pairs.ctypes.data_as(ctypes.c_void_p), pairs.shape[0]
    rc = lib().oracle_decode_fp8(_u16(query), _u8(k_cache), _u8(v_cache), bt, bt.shape[1],
                                 _i32(seq_lens), B, H_q, H_kv, D, num_blocks, _DTYPES[dtype],
                                 scale, k_scale, v_scale, pp, n, nthreads, out)
    _check(rc, "decode_fp8")
    return out


def prefill_fp8(query, k_cache, v_cache, block_tables, seq_lens, cu_q_lens, H_q, H_kv, D,
                num_blocks, dtype, scale, k_scale, v_scale, rows=None, nthreads=0):
    """F7: paged causal prefill over E4M3 caches. query [total_q][H_q][D] words of dtype. Returns
    float64 [total_q][H_q][D], or [n][D] for an explicit list of (row, head) pairs."""
    bt = _i32(block_tables)
    cu = _i32(cu_q_lens)
    if rows is None:
        out = np.zeros((int(cu[-1]), H_q, D), dtype=np.float64)
        rp, n = None, 0
    else:
        rows = _i32(np.asarray(rows).reshape(-1, 2))
        out = np.zeros((rows.shape[0], D), dtype=np.float64)
        rp, n = rows.ctypes.data_as(ctypes.c_void_p), rows.shape[0]
    rc = lib().oracle_prefill_fp8(_u16(query), _u8(k_cache), _u8(v_cache), bt, bt.shape[1],
                                  _i32(seq_lens), cu, bt.shape[0], H_q, H_kv, D, num_blocks,
                                  _DTYPES[dtype], scale, k_scale, v_scale, rp, n, nthreads, out)
    _check(rc, "prefill_fp8")
    return out


def poison_free_slots_fp8(k_cache, v_cache, block_tables, seq_lens, num_blocks, H_kv, D):
    """Copies of E4M3 caches with every slot that holds no valid token set to the NaN code."""
    kc, vc = _u8(k_cache).copy(), _u8(v_cache).copy()
    bt = _i32(block_tables)
    n = lib().oracle_poison_free_slots_fp8(kc, vc, bt, bt.shape[1], _i32(seq_lens), bt.shape[0],
                                           num_blocks, H_kv, D, NAN_E4M3)
    if n < 0:
        raise ValueError("oracle poison_free_slots_fp8: bad table entry")
    return kc, vc


def max_threads():
    return int(lib().oracle_max_threads())
