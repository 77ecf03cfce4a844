"""ctypes binding of libpa.so.  Argument marshalling only: every step of the
decode path runs in libpa's HIP kernels or its C++ allocator.

Device entry points take torch tensors that already live on the GPU (torch
supplies device memory and the current stream) and keep the C names.
The allocator is host-only and takes/returns numpy arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_OOM, PA_ERR_UNSUPPORTED, PA_ERR_HIP = range(5)
PA_F16, PA_BF16 = 0, 1
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_OOM", 3: "PA_ERR_UNSUPPORTED",
                4: "PA_ERR_HIP"}


class PaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PaOOM(PaError):
    pass


# torch ships its own HIP runtime (libamdhip64.so.7).  Loading torch first makes
# libpa's dependency of the same soname resolve to that copy, so both share one
# runtime, one device context and one set of streams; loading libpa first would
# bring in a second runtime in which torch's device pointers are not valid.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python paged_kv_cache_106_amd/build.py` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _sig(name, restype, argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = argtypes
    return f


_sig("pa_last_error", ctypes.c_char_p, [])
_sig("pa_version", ctypes.c_char_p, [])
_sig("pa_reshape_and_cache", _i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp])
_DEC = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32]
_sig("pa_decode", _i32, _DEC + [_vp, _vp, _vp])
_sig("pa_decode_partitioned_workspace_size", _sz, [_i32, _i32, _i32, _i32, _i32])
_sig("pa_decode_partitioned", _i32, _DEC + [_i32, _vp, _i32, _vp, _sz, _vp, _vp, _vp])
_sig("pa_decode_partitioned_noalloc", _i32, _DEC + [_i32, _vp, _i32, _vp, _vp, _vp])
_sig("pa_decode_partitioned_noalloc_max_workspace", _sz, [])
_sig("pa_copy_blocks", _i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp])
_sig("pa_reshape_and_cache_int8", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _vp])
_sig("pa_write_step_int8", _i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp])
_DEC8 = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
         _f32, _i32]
_sig("pa_decode_int8", _i32, _DEC8 + [_vp, _vp, _vp])
_sig("pa_decode_partitioned_int8", _i32, _DEC8 + [_i32, _vp, _i32, _vp, _sz, _vp, _vp, _vp])
_sig("pa_prefill", _i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                          _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp])
_sig("pa_copy_blocks_int8", _i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp])
_sig("pa_alloc_create", _i32, [_i32, _i32, _i32p, ctypes.POINTER(_vp)])
_sig("pa_alloc_destroy", None, [_vp])
_sig("pa_alloc_allocate", _i32, [_vp, _i64, _i32])
_sig("pa_alloc_append_slot", _i32, [_vp, _i64, _i64p, _i32p, _i32p])
_sig("pa_alloc_append_slots", _i32, [_vp, _i64p, _i32, _i64p, _i32p, _i32p, _i32p])
_sig("pa_update_block_tables", _i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp])
_sig("pa_write_step", _i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _vp, _vp])
_sig("pa_alloc_share_prefix", _i32, [_vp, _i64, _i64, _i32])
_sig("pa_alloc_fork", _i32, [_vp, _i64, _i64])
_sig("pa_alloc_free", _i32, [_vp, _i64])
_sig("pa_alloc_set_prefix_caching", _i32, [_vp, _i32])
_sig("pa_alloc_allocate_prompt", _i32, [_vp, _i64, _i32p, _i32, _i32p])
_sig("pa_alloc_num_cached_blocks", _i32, [_vp])
_sig("pa_alloc_block_table", _i32, [_vp, _i64, _i32p, _i32, _i32p])
_sig("pa_alloc_block_tables", _i32, [_vp, _i64p, _i32, _i32p, _i32, _i32, _i32p])
_sig("pa_alloc_slots", _i32, [_vp, _i64, _i32, _i32, _i64p])
_sig("pa_alloc_num_tokens", _i32, [_vp, _i64])
_sig("pa_alloc_num_free", _i32, [_vp])
_sig("pa_alloc_refcount", _i32, [_vp, _i32])
_sig("pa_alloc_num_shared_blocks", _i32, [_vp])
_sig("pa_alloc_free_list", _i32, [_vp, _i32p, _i32, _i32p])
_sig("pa_partition_work_items", _i32, [_vp, _i32, _i32, _i32, _vp, _i32, _i32p])


def lib():
    return _lib


def _check(status):
    if status != PA_OK:
        msg = _lib.pa_last_error().decode()
        raise (PaOOM if status == PA_ERR_OOM else PaError)(status, msg)


def _dtype_code(dtype):
    if dtype in ("f16", PA_F16):
        return PA_F16
    if dtype in ("bf16", PA_BF16):
        return PA_BF16
    s = str(dtype)
    if s == "torch.float16":
        return PA_F16
    if s == "torch.bfloat16":
        return PA_BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _event(e):
    """hipEvent_t of an event object from ._hip (or None)."""
    return None if e is None else e.handle


def _dptr(t, name, elem_size=None):
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    return t.data_ptr()


def _pinned_ptr(t, name, elem_size):
    if getattr(t, "is_cuda", True) or not t.is_pinned():
        raise ValueError(f"{name} must be a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements")
    return t.data_ptr()


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

def pa_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, dtype, stream=None):
    """key/value [N][Hkv][D]; caches [NB][bs][Hkv][D]; slot_mapping int64 [N]."""
    nb, bs, hkv, d = key_cache.shape
    n = slot_mapping.shape[0]
    if tuple(key.shape) != (n, hkv, d) or tuple(value.shape) != (n, hkv, d):
        raise ValueError("key/value must be [N][Hkv][D] matching the caches and slot_mapping")
    if tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("key_cache and value_cache shapes differ")
    _check(_lib.pa_reshape_and_cache(
        _dptr(key, "key", 2), _dptr(value, "value", 2), _dptr(key_cache, "key_cache", 2),
        _dptr(value_cache, "value_cache", 2), _dptr(slot_mapping, "slot_mapping", 8), n, hkv, d,
        bs, nb, _dtype_code(dtype), _stream(stream)))


def pa_write_step(staged_slots, staged_lens, staged_items, slot_mapping, context_lens, work_items,
                  block_tables, key, value, key_cache, value_cache, stream=None, done_event=None):
    """One decode step's metadata copy, table update and cache write in one
    launch.  staged_slots int64 [S], staged_lens int32 [S] and staged_items
    int32 [n][2] (or None) are pinned host tensors; the rest are GPU tensors:
    slot_mapping int64 [S], context_lens int32 [S], work_items int32 [>= n][2],
    block_tables int32 [S][MB], key/value [S][Hkv][D], caches [NB][bs][Hkv][D]."""
    nb, bs, hkv, d = key_cache.shape
    s = staged_slots.shape[0]
    if tuple(staged_lens.shape) != (s,) or tuple(slot_mapping.shape) != (s,) or \
            tuple(context_lens.shape) != (s,):
        raise ValueError("staged and device slots / lengths must be [S]")
    if block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("block_tables must be [S][MB]")
    if tuple(key.shape) != (s, hkv, d) or tuple(value.shape) != (s, hkv, d):
        raise ValueError("key/value must be [S][Hkv][D] matching the caches")
    if tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("key_cache and value_cache shapes differ")
    n = 0 if staged_items is None else int(staged_items.shape[0])
    if n and (staged_items.dim() != 2 or staged_items.shape[1] != 2 or
              work_items.shape[0] < n or work_items.shape[1] != 2):
        raise ValueError("work lists must be [n][2], the device one at least as long")
    _check(_lib.pa_write_step(
        _pinned_ptr(staged_slots, "staged_slots", 8), _pinned_ptr(staged_lens, "staged_lens", 4),
        _pinned_ptr(staged_items, "staged_items", 4) if n else None, n,
        _dptr(slot_mapping, "slot_mapping", 8), _dptr(context_lens, "context_lens", 4),
        _dptr(work_items, "work_items", 4) if n else None, _dptr(block_tables, "block_tables", 4),
        block_tables.shape[1], _dptr(key, "key", 2), _dptr(value, "value", 2),
        _dptr(key_cache, "key_cache", 2), _dptr(value_cache, "value_cache", 2), s, hkv, d, bs, nb,
        _stream(stream), _event(done_event)))


def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len,
                 scale, dtype):
    s, hq, d = query.shape
    nb, bs, hkv, d2 = key_cache.shape
    if d2 != d or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("cache shapes do not match the query")
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the query's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(context_lens.shape) != (s,):
        raise ValueError("block_tables must be [S][MB] and context_lens [S]")
    mb = block_tables.shape[1]
    return [_dptr(out, "out", 2), _dptr(query, "query", 2), _dptr(key_cache, "key_cache", 2),
            _dptr(value_cache, "value_cache", 2), _dptr(block_tables, "block_tables", 4), mb,
            _dptr(context_lens, "context_lens", 4), s, hq, hkv, d, bs, nb, int(max_context_len),
            float(scale), _dtype_code(dtype)]


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, max_context_len,
              scale, dtype, stream=None, start_event=None, stop_event=None):
    """Single-pass paged decode; writes out [S][Hq][D].  start/stop events
    (._hip.Event with timing, or None) are recorded by the launch itself."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                        max_context_len, scale, dtype)
    _check(_lib.pa_decode(*args, _stream(stream), _event(start_event), _event(stop_event)))


def _work_list(work_items):
    """(pointer, count) of an optional [n][2] int32 work list.  An empty list
    would name no partition (the C call rejects it): None asks for the full
    grid."""
    if work_items is None:
        return None, 0
    if work_items.dim() != 2 or work_items.shape[1] != 2:
        raise ValueError("work_items must be [n][2]")
    if work_items.shape[0] == 0:
        raise ValueError("an empty work list names no partition: pass None for the full grid")
    return _dptr(work_items, "work_items", 4), work_items.shape[0]


def pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                         partition_size):
    return int(_lib.pa_decode_partitioned_workspace_size(num_seqs, num_q_heads, head_dim,
                                                         max_context_len, partition_size))


def pa_decode_partitioned(out, query, key_cache, value_cache, block_tables, context_lens,
                          max_context_len, scale, dtype, partition_size, workspace,
                          work_items=None, stream=None, start_event=None, stop_event=None):
    """Split-context paged decode + merge; workspace is a uint8 GPU tensor;
    work_items an optional int32 GPU tensor [n][2] of (sequence, partition);
    start/stop events as for pa_decode."""
    wi, nwi = _work_list(work_items)
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                        max_context_len, scale, dtype)
    _check(_lib.pa_decode_partitioned(*args, int(partition_size), wi, int(nwi),
                                      _dptr(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream), _event(start_event), _event(stop_event)))


def pa_decode_partitioned_noalloc(out, query, key_cache, value_cache, block_tables,
                                  context_lens, max_context_len, scale, dtype, partition_size,
                                  work_items=None, stream=None, start_event=None,
                                  stop_event=None):
    """pa_decode_partitioned with its split workspace in libpa's per-GPU
    scratch array (no allocation by the call; workspaces above
    pa_decode_partitioned_noalloc_max_workspace() bytes are refused)."""
    wi, nwi = _work_list(work_items)
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                        max_context_len, scale, dtype)
    _check(_lib.pa_decode_partitioned_noalloc(*args, int(partition_size), wi, int(nwi),
                                              _stream(stream), _event(start_event),
                                              _event(stop_event)))


def pa_decode_partitioned_noalloc_max_workspace():
    return int(_lib.pa_decode_partitioned_noalloc_max_workspace())


# -- INT8 pools: codes int8 [NB][bs][Hkv][D], scales float32 [NB][Hkv][bs] ---------------

def _check_q8_pools(key_cache, value_cache, key_scale, value_scale):
    nb, bs, hkv, d = key_cache.shape
    if tuple(value_cache.shape) != (nb, bs, hkv, d):
        raise ValueError("key_cache and value_cache shapes differ")
    if tuple(key_scale.shape) != (nb, hkv, bs) or tuple(value_scale.shape) != (nb, hkv, bs):
        raise ValueError("scales must be [NB][Hkv][bs]")
    return nb, bs, hkv, d


def _q8_ptrs(key_cache, value_cache, key_scale, value_scale):
    return [_dptr(key_cache, "key_cache", 1), _dptr(value_cache, "value_cache", 1),
            _dptr(key_scale, "key_scale", 4), _dptr(value_scale, "value_scale", 4)]


def pa_reshape_and_cache_int8(key, value, key_cache, value_cache, key_scale, value_scale,
                              slot_mapping, dtype, stream=None):
    """Quantise key/value [N][Hkv][D] (16-bit) into the INT8 pools at slot_mapping."""
    nb, bs, hkv, d = _check_q8_pools(key_cache, value_cache, key_scale, value_scale)
    n = slot_mapping.shape[0]
    if tuple(key.shape) != (n, hkv, d) or tuple(value.shape) != (n, hkv, d):
        raise ValueError("key/value must be [N][Hkv][D] matching the caches and slot_mapping")
    _check(_lib.pa_reshape_and_cache_int8(
        _dptr(key, "key", 2), _dptr(value, "value", 2),
        *_q8_ptrs(key_cache, value_cache, key_scale, value_scale),
        _dptr(slot_mapping, "slot_mapping", 8), n, hkv, d, bs, nb, _dtype_code(dtype),
        _stream(stream)))


def pa_write_step_int8(staged_slots, staged_lens, staged_items, slot_mapping, context_lens,
                       work_items, block_tables, key, value, key_cache, value_cache, key_scale,
                       value_scale, dtype, stream=None, done_event=None):
    """pa_write_step into INT8 pools (arguments as there, plus the scales)."""
    nb, bs, hkv, d = _check_q8_pools(key_cache, value_cache, key_scale, value_scale)
    s = staged_slots.shape[0]
    if tuple(staged_lens.shape) != (s,) or tuple(slot_mapping.shape) != (s,) or \
            tuple(context_lens.shape) != (s,):
        raise ValueError("staged and device slots / lengths must be [S]")
    if block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("block_tables must be [S][MB]")
    if tuple(key.shape) != (s, hkv, d) or tuple(value.shape) != (s, hkv, d):
        raise ValueError("key/value must be [S][Hkv][D] matching the caches")
    n = 0 if staged_items is None else int(staged_items.shape[0])
    if n and (staged_items.dim() != 2 or staged_items.shape[1] != 2 or
              work_items.shape[0] < n or work_items.shape[1] != 2):
        raise ValueError("work lists must be [n][2], the device one at least as long")
    _check(_lib.pa_write_step_int8(
        _pinned_ptr(staged_slots, "staged_slots", 8), _pinned_ptr(staged_lens, "staged_lens", 4),
        _pinned_ptr(staged_items, "staged_items", 4) if n else None, n,
        _dptr(slot_mapping, "slot_mapping", 8), _dptr(context_lens, "context_lens", 4),
        _dptr(work_items, "work_items", 4) if n else None, _dptr(block_tables, "block_tables", 4),
        block_tables.shape[1], _dptr(key, "key", 2), _dptr(value, "value", 2),
        *_q8_ptrs(key_cache, value_cache, key_scale, value_scale), s, hkv, d, bs, nb,
        _dtype_code(dtype), _stream(stream), _event(done_event)))


def _decode_int8_args(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                      context_lens, max_context_len, scale, dtype):
    s, hq, d = query.shape
    nb, bs, hkv, d2 = _check_q8_pools(key_cache, value_cache, key_scale, value_scale)
    if d2 != d:
        raise ValueError("cache shapes do not match the query")
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the query's shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(context_lens.shape) != (s,):
        raise ValueError("block_tables must be [S][MB] and context_lens [S]")
    return [_dptr(out, "out", 2), _dptr(query, "query", 2),
            *_q8_ptrs(key_cache, value_cache, key_scale, value_scale),
            _dptr(block_tables, "block_tables", 4), block_tables.shape[1],
            _dptr(context_lens, "context_lens", 4), s, hq, hkv, d, bs, nb, int(max_context_len),
            float(scale), _dtype_code(dtype)]


def pa_decode_int8(out, query, key_cache, value_cache, key_scale, value_scale, block_tables,
                   context_lens, max_context_len, scale, dtype, stream=None, start_event=None,
                   stop_event=None):
    """Single-pass paged decode over INT8 pools; writes out [S][Hq][D] (16-bit)."""
    args = _decode_int8_args(out, query, key_cache, value_cache, key_scale, value_scale,
                             block_tables, context_lens, max_context_len, scale, dtype)
    _check(_lib.pa_decode_int8(*args, _stream(stream), _event(start_event), _event(stop_event)))


def pa_decode_partitioned_int8(out, query, key_cache, value_cache, key_scale, value_scale,
                               block_tables, context_lens, max_context_len, scale, dtype,
                               partition_size, workspace, work_items=None, stream=None,
                               start_event=None, stop_event=None):
    """Split-context paged decode + merge over INT8 pools (workspace as for
    pa_decode_partitioned)."""
    wi, nwi = _work_list(work_items)
    args = _decode_int8_args(out, query, key_cache, value_cache, key_scale, value_scale,
                             block_tables, context_lens, max_context_len, scale, dtype)
    _check(_lib.pa_decode_partitioned_int8(*args, int(partition_size), wi, int(nwi),
                                           _dptr(workspace, "workspace"),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream), _event(start_event),
                                           _event(stop_event)))


def pa_copy_blocks_int8(key_cache, value_cache, key_scale, value_scale, block_pairs, stream=None):
    """Copy-on-write copies of INT8 blocks (codes and scales); block_pairs int32 [n][2]."""
    nb, bs, hkv, d = _check_q8_pools(key_cache, value_cache, key_scale, value_scale)
    n = block_pairs.shape[0]
    _check(_lib.pa_copy_blocks_int8(*_q8_ptrs(key_cache, value_cache, key_scale, value_scale),
                                    _dptr(block_pairs, "block_pairs", 4) if n else None, n, hkv,
                                    d, bs, nb, _stream(stream)))


def pa_prefill(out, query, key_cache, value_cache, block_tables, context_lens, query_start,
               max_query_len, scale, dtype, seq_order=None, stream=None, start_event=None,
               stop_event=None):
    """Causal attention of each sequence's query chunk (its last n_i cached
    tokens) over its paged cache.  query/out [T][Hq][D] 16-bit; query_start
    int32 GPU tensor [S+1]; context_lens int32 [S]; block_tables int32 [S][MB];
    seq_order an optional int32 GPU tensor [S] (dispatch order, longest first)."""
    t, hq, d = query.shape
    nb, bs, hkv, d2 = key_cache.shape
    if d2 != d or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("cache shapes do not match the query")
    if tuple(out.shape) != tuple(query.shape):
        raise ValueError("out must have the query's shape")
    s = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(query_start.shape) != (s + 1,):
        raise ValueError("block_tables must be [S][MB] and query_start [S+1]")
    _check(_lib.pa_prefill(
        _dptr(out, "out", 2), _dptr(query, "query", 2), _dptr(key_cache, "key_cache", 2),
        _dptr(value_cache, "value_cache", 2), _dptr(block_tables, "block_tables", 4),
        block_tables.shape[1], _dptr(context_lens, "context_lens", 4),
        _dptr(query_start, "query_start", 4),
        None if seq_order is None else _dptr(seq_order, "seq_order", 4), s, t,
        int(max_query_len), hq, hkv, d, bs, nb,
        float(scale), _dtype_code(dtype), _stream(stream), _event(start_event),
        _event(stop_event)))


def partition_work_items(context_lens, partition_size, max_parts=None, out=None):
    """Host-side work list for pa_decode_partitioned (pa_partition_work_items):
    (sequence, partition) for every live partition, dealt to one queue per
    XCD (list position i runs on XCD i % 8) in runs of one sequence's
    partitions, longest first, to the queue with the fewest tokens (whole
    sequences when that balances the queues to 1 %, shorter runs otherwise);
    per queue the full partitions, then the ragged ones by decreasing length;
    queues read out round-robin.  context_lens: int
    array [S].  Returns int32 [n][2] (a view of `out` if given)."""
    L = np.ascontiguousarray(context_lens, dtype=np.int32)
    if out is None:
        P = int(partition_size)
        cap = int(((L.astype(np.int64) + P - 1) // P).sum()) if P > 0 else 0
        out = np.empty((max(cap, 1), 2), np.int32)
    n = ctypes.c_int32()
    _check(_lib.pa_partition_work_items(L.ctypes.data, L.shape[0], int(partition_size),
                                        -1 if max_parts is None else int(max_parts),
                                        out.ctypes.data, out.shape[0], ctypes.byref(n)))
    return out[: n.value]


def pa_update_block_tables(block_tables, context_lens, slot_mapping, block_size, num_blocks,
                           stream=None):
    """block_tables int32 [S][MB] (updated in place); context_lens int32 [S]; slot_mapping int64 [S]."""
    s, mb = block_tables.shape
    if tuple(context_lens.shape) != (s,) or tuple(slot_mapping.shape) != (s,):
        raise ValueError("context_lens and slot_mapping must be [S]")
    _check(_lib.pa_update_block_tables(_dptr(block_tables, "block_tables", 4), mb,
                                       _dptr(context_lens, "context_lens", 4),
                                       _dptr(slot_mapping, "slot_mapping", 8), s, int(block_size),
                                       int(num_blocks), _stream(stream)))


def pa_copy_blocks(key_cache, value_cache, block_pairs, dtype, stream=None):
    """block_pairs: int32 GPU tensor [n][2] of (src, dst) block ids."""
    nb, bs, hkv, d = key_cache.shape
    n = block_pairs.shape[0]
    _check(_lib.pa_copy_blocks(_dptr(key_cache, "key_cache", 2), _dptr(value_cache, "value_cache", 2),
                               _dptr(block_pairs, "block_pairs", 4), n, hkv, d, bs, nb,
                               _dtype_code(dtype), _stream(stream)))


# ---------------------------------------------------------------------------
# host allocator
# ---------------------------------------------------------------------------

def _np_ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Allocator:
    """Owns one pa_allocator handle; each method is one pa_alloc_* call."""

    def __init__(self, num_blocks, block_size, initial_free_order=None, prefix_caching=False):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        h = _vp()
        order = None
        if initial_free_order is not None:
            self._order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if self._order.shape != (self.num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
            order = _np_ptr(self._order, ctypes.c_int32)
        _check(_lib.pa_alloc_create(self.num_blocks, self.block_size, order, ctypes.byref(h)))
        self._h = h
        if prefix_caching:
            self.set_prefix_caching(True)

    def close(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pa_alloc_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def allocate(self, seq_id, num_tokens):
        _check(_lib.pa_alloc_allocate(self._h, int(seq_id), int(num_tokens)))

    def append_slot(self, seq_id):
        """Returns (slot, cow) with cow None or (src_block, dst_block)."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.pa_alloc_append_slot(self._h, int(seq_id), ctypes.byref(slot),
                                         ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_slots(self, seq_ids, slots_out=None, context_lens_out=None, cow_src=None,
                     cow_dst=None):
        """Batched append_slot; returns (slots int64[n], context_lens int32[n],
        cow_src int32[n], cow_dst int32[n])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        slots = slots_out if slots_out is not None else np.empty(n, np.int64)
        lens = context_lens_out if context_lens_out is not None else np.empty(n, np.int32)
        src = cow_src if cow_src is not None else np.empty(n, np.int32)
        dst = cow_dst if cow_dst is not None else np.empty(n, np.int32)
        _check(_lib.pa_alloc_append_slots(self._h, _np_ptr(ids, ctypes.c_int64), n,
                                          _np_ptr(slots, ctypes.c_int64),
                                          _np_ptr(lens, ctypes.c_int32),
                                          _np_ptr(src, ctypes.c_int32), _np_ptr(dst, ctypes.c_int32)))
        return slots, lens, src, dst

    def share_prefix(self, src_seq, dst_seq, num_tokens):
        _check(_lib.pa_alloc_share_prefix(self._h, int(src_seq), int(dst_seq), int(num_tokens)))

    def fork(self, src_seq, dst_seq):
        _check(_lib.pa_alloc_fork(self._h, int(src_seq), int(dst_seq)))

    def free(self, seq_id):
        _check(_lib.pa_alloc_free(self._h, int(seq_id)))

    def set_prefix_caching(self, enabled):
        _check(_lib.pa_alloc_set_prefix_caching(self._h, 1 if enabled else 0))

    def allocate_prompt(self, seq_id, tokens):
        """New sequence holding the prompt; returns the number of leading
        tokens whose K/V the prefix cache already holds."""
        ids = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
        cached = ctypes.c_int32()
        _check(_lib.pa_alloc_allocate_prompt(self._h, int(seq_id), _np_ptr(ids, ctypes.c_int32),
                                             ids.shape[0], ctypes.byref(cached)))
        return cached.value

    def num_cached_blocks(self):
        return int(_lib.pa_alloc_num_cached_blocks(self._h))

    def block_table(self, seq_id):
        n = ctypes.c_int32()
        cap = self.num_blocks
        out = np.empty(cap, np.int32)
        _check(_lib.pa_alloc_block_table(self._h, int(seq_id), _np_ptr(out, ctypes.c_int32), cap,
                                         ctypes.byref(n)))
        return out[: n.value].copy()

    def block_tables(self, seq_ids, max_blocks_per_seq, pad=0, out=None, context_lens_out=None):
        """Dense [n][max_blocks_per_seq] int32 tables and int32 [n] token counts."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        tbl = out if out is not None else np.empty((n, max_blocks_per_seq), np.int32)
        lens = context_lens_out if context_lens_out is not None else np.empty(n, np.int32)
        _check(_lib.pa_alloc_block_tables(self._h, _np_ptr(ids, ctypes.c_int64), n,
                                          _np_ptr(tbl, ctypes.c_int32), int(max_blocks_per_seq),
                                          int(pad), _np_ptr(lens, ctypes.c_int32)))
        return tbl, lens

    def slots(self, seq_id, begin, end):
        out = np.empty(max(end - begin, 0), np.int64)
        _check(_lib.pa_alloc_slots(self._h, int(seq_id), int(begin), int(end),
                                   _np_ptr(out, ctypes.c_int64)))
        return out

    def num_tokens(self, seq_id):
        return int(_lib.pa_alloc_num_tokens(self._h, int(seq_id)))

    def num_free(self):
        return int(_lib.pa_alloc_num_free(self._h))

    def refcount(self, block_id):
        return int(_lib.pa_alloc_refcount(self._h, int(block_id)))

    def num_shared_blocks(self):
        return int(_lib.pa_alloc_num_shared_blocks(self._h))

    def free_list(self):
        n = ctypes.c_int32()
        out = np.empty(self.num_blocks, np.int32)
        _check(_lib.pa_alloc_free_list(self._h, _np_ptr(out, ctypes.c_int32), self.num_blocks,
                                       ctypes.byref(n)))
        return out[: n.value].copy()
