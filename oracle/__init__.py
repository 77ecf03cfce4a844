"""CPU oracle for paged decode attention (numpy front end over libpa_oracle.so).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports the product package.

Arrays are numpy: 16-bit float data travels as ``uint16`` bit patterns,
pools are ``[num_blocks][block_size][num_kv_heads][head_dim]``, queries
``[S][Hq][D]``, block tables ``int32 [S][max_blocks]``, context lengths
``int32 [S]`` and slot mappings ``int64 [N]``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

DTYPES = {"f16": 0, "bf16": 1}
ERRORS = {
    -1: "bad argument",
    -2: "slot out of range",
    -3: "duplicate slot",
    -4: "block id out of range",
    -5: "bad context length",
}

_lib = None


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("PA_ORACLE_LIB")   # mutation tests load a planted copy
        if not path:
            if not os.path.exists(_build.LIB):
                _build.build()
            path = _build.LIB
        L = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.pao_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.pao_f16_to_f32.restype = ctypes.c_float
        L.pao_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.pao_bf16_to_f32.restype = ctypes.c_float
        L.pao_f32_to_f16.argtypes = [ctypes.c_float]
        L.pao_f32_to_f16.restype = ctypes.c_uint16
        L.pao_f32_to_bf16.argtypes = [ctypes.c_float]
        L.pao_f32_to_bf16.restype = ctypes.c_uint16
        L.pao_widen.argtypes = [u16p, f32p, i64, i32]
        L.pao_widen.restype = None
        L.pao_narrow.argtypes = [f32p, u16p, i64, i32]
        L.pao_narrow.restype = None
        L.pao_cache_write.argtypes = [u16p, u16p, u16p, u16p, i64p, i32, i32, i32, i32, i32]
        L.pao_cache_write.restype = i32
        L.pao_slot.argtypes = [i32p, i32, i32]
        L.pao_slot.restype = i64
        L.pao_gather.argtypes = [f32p, f32p, u16p, u16p, i32p, i32, i32, i32, i32, i32, i32, i32]
        L.pao_gather.restype = i32
        common = [u16p, u16p, u16p, i32p, i32, i32p, i32, i32, i32, i32, i32, i32,
                  ctypes.c_float, i32]
        L.pao_decode_pairs.argtypes = [f32p, u16p] + common + [i32p, i32, i32]
        L.pao_decode_pairs.restype = i32
        L.pao_decode.argtypes = [f32p, u16p] + common + [i32]
        L.pao_decode.restype = i32
        L.pao_decode_partitioned.argtypes = [f32p, u16p] + common + [i32]
        L.pao_decode_partitioned.restype = i32
        L.pao_prefill.argtypes = [f32p, u16p, u16p, u16p, u16p, i32p, i32, i32p, i32p, i32, i32,
                                  i32, i32, i32, i32, ctypes.c_float, i32, i32]
        L.pao_prefill.restype = i32
        i8p = ctypes.POINTER(ctypes.c_int8)
        L.pao_quantize_rows.argtypes = [u16p, i64, i32, i32, i8p, f32p]
        L.pao_quantize_rows.restype = i32
        L.pao_cache_write_int8.argtypes = [u16p, u16p, i8p, i8p, f32p, f32p, i64p, i32, i32, i32,
                                           i32, i32, i32]
        L.pao_cache_write_int8.restype = i32
        L.pao_gather_int8.argtypes = [f32p, f32p, i8p, i8p, f32p, f32p, i32p, i32, i32, i32, i32,
                                      i32, i32]
        L.pao_gather_int8.restype = i32
        L.pao_decode_int8_pairs.argtypes = [f32p, u16p, u16p, i8p, i8p, f32p, f32p, i32p, i32,
                                            i32p, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                            i32, i32p, i32, i32]
        L.pao_decode_int8_pairs.restype = i32
        L.pao_kv_bytes_per_token.argtypes = [i32, i32, i32, i32]
        L.pao_kv_bytes_per_token.restype = ctypes.c_uint64
        L.pao_kv_bytes_gathered.argtypes = [i32p, i32, i32, i32, i32]
        L.pao_kv_bytes_gathered.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc):
    if rc != 0:
        raise OracleError(ERRORS.get(rc, f"error {rc}"))


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous {np.dtype(dtype).name} array")
    return a


# -- conversions --------------------------------------------------------------

def f16_to_f32(h: int) -> float:
    return lib().pao_f16_to_f32(h)


def bf16_to_f32(b: int) -> float:
    return lib().pao_bf16_to_f32(b)


def f32_to_f16(x: float) -> int:
    return lib().pao_f32_to_f16(x)


def f32_to_bf16(x: float) -> int:
    return lib().pao_f32_to_bf16(x)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().pao_widen(_ptr(bits, ctypes.c_uint16), _ptr(out, ctypes.c_float), bits.size,
                    DTYPES[dtype])
    return out


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().pao_narrow(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size,
                     DTYPES[dtype])
    return out


# -- cache write, slots, gather ----------------------------------------------------

def cache_write(key, value, key_cache, value_cache, slot_mapping):
    """Write each token's K/V into its slot of the pools (in place)."""
    _need(key, np.uint16, "key"); _need(value, np.uint16, "value")
    _need(key_cache, np.uint16, "key_cache"); _need(value_cache, np.uint16, "value_cache")
    _need(slot_mapping, np.int64, "slot_mapping")
    nb, bs, hkv, d = key_cache.shape
    n = slot_mapping.shape[0]
    if key.shape != (n, hkv, d) or value.shape != (n, hkv, d) or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    _check(lib().pao_cache_write(
        _ptr(key, ctypes.c_uint16), _ptr(value, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
        _ptr(slot_mapping, ctypes.c_int64), n, hkv, d, bs, nb))


def slot(block_table_row: np.ndarray, pos: int, block_size: int) -> int:
    row = np.ascontiguousarray(block_table_row, dtype=np.int32)
    return int(lib().pao_slot(_ptr(row, ctypes.c_int32), pos, block_size))


def gather(key_cache, value_cache, block_table_row, L, g, dtype):
    nb, bs, hkv, d = key_cache.shape
    row = np.ascontiguousarray(block_table_row, dtype=np.int32)
    k = np.empty((L, d), np.float32)
    v = np.empty((L, d), np.float32)
    _check(lib().pao_gather(_ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                            _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
                            _ptr(row, ctypes.c_int32), L, g, hkv, d, bs, nb, DTYPES[dtype]))
    return k, v


# -- decode -------------------------------------------------------------------------

def _decode_common(q, key_cache, value_cache, block_tables, context_lens):
    _need(q, np.uint16, "q"); _need(key_cache, np.uint16, "key_cache")
    _need(value_cache, np.uint16, "value_cache")
    _need(block_tables, np.int32, "block_tables"); _need(context_lens, np.int32, "context_lens")
    s, hq, d = q.shape
    nb, bs, hkv, d2 = key_cache.shape
    if d2 != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("metadata shape mismatch")
    mb = block_tables.shape[1]
    return s, hq, hkv, d, bs, nb, mb


def decode(q, key_cache, value_cache, block_tables, context_lens, scale, dtype, nthreads=1):
    """Single-pass fp32 decode of every (sequence, q head).

    Returns (out_f32 [S][Hq][D] float32, out_t [S][Hq][D] uint16)."""
    s, hq, hkv, d, bs, nb, mb = _decode_common(q, key_cache, value_cache, block_tables,
                                               context_lens)
    out_f32 = np.empty((s, hq, d), np.float32)
    out_t = np.empty((s, hq, d), np.uint16)
    _check(lib().pao_decode(
        _ptr(out_f32, ctypes.c_float), _ptr(out_t, ctypes.c_uint16), _ptr(q, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
        _ptr(block_tables, ctypes.c_int32), mb, _ptr(context_lens, ctypes.c_int32),
        s, hq, hkv, d, bs, nb, float(scale), DTYPES[dtype], int(nthreads)))
    return out_f32, out_t


def decode_pairs(q, key_cache, value_cache, block_tables, context_lens, scale, dtype, pairs,
                 nthreads=1):
    """Decode only the listed (seq, q head) pairs; returns ([n][D] f32, [n][D] u16)."""
    s, hq, hkv, d, bs, nb, mb = _decode_common(q, key_cache, value_cache, block_tables,
                                               context_lens)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    n = pairs.shape[0]
    out_f32 = np.empty((n, d), np.float32)
    out_t = np.empty((n, d), np.uint16)
    _check(lib().pao_decode_pairs(
        _ptr(out_f32, ctypes.c_float), _ptr(out_t, ctypes.c_uint16), _ptr(q, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
        _ptr(block_tables, ctypes.c_int32), mb, _ptr(context_lens, ctypes.c_int32),
        s, hq, hkv, d, bs, nb, float(scale), DTYPES[dtype], _ptr(pairs, ctypes.c_int32), n,
        int(nthreads)))
    return out_f32, out_t


def decode_partitioned(q, key_cache, value_cache, block_tables, context_lens, scale, dtype,
                       partition_size):
    s, hq, hkv, d, bs, nb, mb = _decode_common(q, key_cache, value_cache, block_tables,
                                               context_lens)
    out_f32 = np.empty((s, hq, d), np.float32)
    out_t = np.empty((s, hq, d), np.uint16)
    _check(lib().pao_decode_partitioned(
        _ptr(out_f32, ctypes.c_float), _ptr(out_t, ctypes.c_uint16), _ptr(q, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
        _ptr(block_tables, ctypes.c_int32), mb, _ptr(context_lens, ctypes.c_int32),
        s, hq, hkv, d, bs, nb, float(scale), DTYPES[dtype], int(partition_size)))
    return out_f32, out_t


# -- multi-token (chunked-prefill) attention -----------------------------------------------

def prefill(q, key_cache, value_cache, block_tables, context_lens, query_start, scale, dtype,
            nthreads=1):
    """Causal attention of each sequence's query chunk (its last n_i cached
    tokens) over its paged cache.  q [T][Hq][D] u16; query_start int32 [S+1].
    Returns (out_f32 [T][Hq][D], out_t [T][Hq][D] u16)."""
    _need(q, np.uint16, "q"); _need(key_cache, np.uint16, "key_cache")
    _need(value_cache, np.uint16, "value_cache")
    _need(block_tables, np.int32, "block_tables"); _need(context_lens, np.int32, "context_lens")
    _need(query_start, np.int32, "query_start")
    T, hq, d = q.shape
    nb, bs, hkv, d2 = key_cache.shape
    s = context_lens.shape[0]
    if d2 != d or value_cache.shape != key_cache.shape or block_tables.shape[0] != s or \
            query_start.shape != (s + 1,) or int(query_start[-1]) != T:
        raise ValueError("shape mismatch")
    out_f32 = np.empty((T, hq, d), np.float32)
    out_t = np.empty((T, hq, d), np.uint16)
    _check(lib().pao_prefill(
        _ptr(out_f32, ctypes.c_float), _ptr(out_t, ctypes.c_uint16), _ptr(q, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_uint16), _ptr(value_cache, ctypes.c_uint16),
        _ptr(block_tables, ctypes.c_int32), block_tables.shape[1],
        _ptr(context_lens, ctypes.c_int32), _ptr(query_start, ctypes.c_int32), s, hq, hkv, d, bs,
        nb, float(scale), DTYPES[dtype], int(nthreads)))
    return out_f32, out_t


# -- INT8 KV cache ------------------------------------------------------------------------
# codes int8 [nb][bs][hkv][d]; scales float32 [nb][hkv][bs]

def quantize_rows(x_bits, dtype):
    """Rows [..., d] of 16-bit patterns -> (int8 codes [..., d], float32 scales [...])."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.empty(x.shape, np.int8)
    scales = np.empty(x.shape[:-1], np.float32)
    _check(lib().pao_quantize_rows(_ptr(x, ctypes.c_uint16), rows, d, DTYPES[dtype],
                                   _ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_float)))
    return codes, scales


def cache_write_int8(key, value, key_cache, value_cache, key_scale, value_scale, slot_mapping,
                     dtype):
    """Quantise each token's K/V rows into its slot of the INT8 pools (in place)."""
    _need(key, np.uint16, "key"); _need(value, np.uint16, "value")
    _need(key_cache, np.int8, "key_cache"); _need(value_cache, np.int8, "value_cache")
    _need(key_scale, np.float32, "key_scale"); _need(value_scale, np.float32, "value_scale")
    _need(slot_mapping, np.int64, "slot_mapping")
    nb, bs, hkv, d = key_cache.shape
    n = slot_mapping.shape[0]
    if (key.shape != (n, hkv, d) or value.shape != (n, hkv, d) or
            value_cache.shape != key_cache.shape or key_scale.shape != (nb, hkv, bs) or
            value_scale.shape != (nb, hkv, bs)):
        raise ValueError("shape mismatch")
    _check(lib().pao_cache_write_int8(
        _ptr(key, ctypes.c_uint16), _ptr(value, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_int8), _ptr(value_cache, ctypes.c_int8),
        _ptr(key_scale, ctypes.c_float), _ptr(value_scale, ctypes.c_float),
        _ptr(slot_mapping, ctypes.c_int64), n, hkv, d, bs, nb, DTYPES[dtype]))


def gather_int8(key_cache, value_cache, key_scale, value_scale, block_table_row, L, g):
    nb, bs, hkv, d = key_cache.shape
    row = np.ascontiguousarray(block_table_row, dtype=np.int32)
    k = np.empty((L, d), np.float32)
    v = np.empty((L, d), np.float32)
    _check(lib().pao_gather_int8(
        _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), _ptr(key_cache, ctypes.c_int8),
        _ptr(value_cache, ctypes.c_int8), _ptr(key_scale, ctypes.c_float),
        _ptr(value_scale, ctypes.c_float), _ptr(row, ctypes.c_int32), L, g, hkv, d, bs, nb))
    return k, v


def decode_int8(q, key_cache, value_cache, key_scale, value_scale, block_tables, context_lens,
                scale, dtype, pairs=None, nthreads=1):
    """fp32 decode over the INT8 cache, rows dequantised as scale x code.
    pairs None: every (sequence, q head), outputs [S][Hq][D]; else [n][D]."""
    _need(q, np.uint16, "q"); _need(key_cache, np.int8, "key_cache")
    _need(value_cache, np.int8, "value_cache"); _need(key_scale, np.float32, "key_scale")
    _need(value_scale, np.float32, "value_scale")
    _need(block_tables, np.int32, "block_tables"); _need(context_lens, np.int32, "context_lens")
    s, hq, d = q.shape
    nb, bs, hkv, d2 = key_cache.shape
    if (d2 != d or value_cache.shape != key_cache.shape or key_scale.shape != (nb, hkv, bs) or
            value_scale.shape != key_scale.shape):
        raise ValueError("shape mismatch")
    if block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("metadata shape mismatch")
    mb = block_tables.shape[1]
    shape = None
    if pairs is None:
        pairs = np.stack(np.meshgrid(np.arange(s), np.arange(hq), indexing="ij"), -1)
        shape = (s, hq, d)
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    n = pairs.shape[0]
    out_f32 = np.empty((n, d), np.float32)
    out_t = np.empty((n, d), np.uint16)
    _check(lib().pao_decode_int8_pairs(
        _ptr(out_f32, ctypes.c_float), _ptr(out_t, ctypes.c_uint16), _ptr(q, ctypes.c_uint16),
        _ptr(key_cache, ctypes.c_int8), _ptr(value_cache, ctypes.c_int8),
        _ptr(key_scale, ctypes.c_float), _ptr(value_scale, ctypes.c_float),
        _ptr(block_tables, ctypes.c_int32), mb, _ptr(context_lens, ctypes.c_int32),
        s, hq, hkv, d, bs, nb, float(scale), DTYPES[dtype], _ptr(pairs, ctypes.c_int32), n,
        int(nthreads)))
    if shape is not None:
        return out_f32.reshape(shape), out_t.reshape(shape)
    return out_f32, out_t


# -- byte accounting -------------------------------------------------------------------

def kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes) -> int:
    return int(lib().pao_kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes))


def kv_bytes_gathered(context_lens, kv_heads, head_dim, elem_bytes) -> int:
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    return int(lib().pao_kv_bytes_gathered(_ptr(cl, ctypes.c_int32), cl.size, kv_heads,
                                           head_dim, elem_bytes))
