"""A paged KV cache on one GPU and its decode step.

``PagedKVCache`` owns the two device pools ([num_blocks][block_size][Hkv][D],
16-bit, or INT8 codes with fp32 row scales [num_blocks][Hkv][block_size]) and
the host block allocator.  ``DecodeStep`` runs one decode step for
a fixed batch of sequences, in the order the pages describe for a step
("vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.1 data flow and §3.3):

  a1  host: append_slot for every sequence -> slot mapping and context
      lengths (libpa's allocator, written straight into pinned host buffers);
  a2  one async host-to-device copy of that metadata (12 bytes per sequence,
      copy-on-write pairs when there are any, and the list of live
      (sequence, partition) work items for the split kernel) on the step's
      stream;
  a3  pa_copy_blocks for copy-on-write, pa_update_block_tables (the device-
      resident tables gain each new token's block), pa_reshape_and_cache (the
      new tokens' K/V into their slots);
  a4  pa_decode (single pass)  or  a5+a6  pa_decode_partitioned (+ merge).

Pinned metadata buffers are double-buffered: the host prepares step k+1
while the GPU still runs step k, and waits on an event only before reusing
a buffer whose copy may not have run yet.
"""
import collections
import ctypes

import numpy as np
import torch

from . import _native as pa
from ._hip import Event

POISON = {"f16": 0x7E00, "bf16": 0x7FC0}   # quiet-NaN patterns for unused slots
POISON_CODE = -128                          # no quantised row holds it (codes are within +-127)


def _dtype(dtype):
    return "f16" if pa._dtype_code(dtype) == pa.PA_F16 else "bf16"


class PagedKVCache:
    """kv_dtype None: pools in the model's 16-bit dtype; "int8": INT8 codes
    with one fp32 scale per (token, KV head) row (key_scale / value_scale
    [num_blocks][Hkv][block_size]), quantised by the library's writes."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                 initial_free_order=None, device="cuda", poison=True, kv_dtype=None,
                 prefix_caching=False):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.dtype = _dtype(dtype)
        if kv_dtype not in (None, "int8"):
            raise ValueError(f"kv_dtype must be None or 'int8', not {kv_dtype!r}")
        self.int8 = kv_dtype == "int8"
        self.device = torch.device(device)
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if self.int8:
            fill = POISON_CODE if poison else 0
            self.key_cache = torch.full(shape, fill, dtype=torch.int8, device=self.device)
            self.value_cache = torch.full(shape, fill, dtype=torch.int8, device=self.device)
            sshape = (self.num_blocks, self.num_kv_heads, self.block_size)
            sfill = float("nan") if poison else 0.0
            self.key_scale = torch.full(sshape, sfill, dtype=torch.float32, device=self.device)
            self.value_scale = torch.full(sshape, sfill, dtype=torch.float32, device=self.device)
        else:
            fill = POISON[self.dtype] if poison else 0
            self.key_cache = torch.full(shape, fill, dtype=torch.int16, device=self.device)
            self.value_cache = torch.full(shape, fill, dtype=torch.int16, device=self.device)
            self.key_scale = self.value_scale = None
        self.allocator = pa.Allocator(self.num_blocks, self.block_size, initial_free_order,
                                      prefix_caching=prefix_caching)

    # -- writing tokens that are already in the sequence (history) ----------------
    def write_positions(self, spans, keys, values, stream=None):
        """spans: list of (seq_id, begin, end); keys/values: [sum(end-begin)][Hkv][D]
        16-bit arrays (numpy uint16/int16 or GPU tensors) in span order."""
        slots = np.concatenate([self.allocator.slots(s, b, e) for s, b, e in spans]) \
            if spans else np.empty(0, np.int64)
        if slots.size == 0:
            return
        dev = self.device
        k = keys if torch.is_tensor(keys) else torch.from_numpy(np.ascontiguousarray(keys).view(np.int16))
        v = values if torch.is_tensor(values) else torch.from_numpy(np.ascontiguousarray(values).view(np.int16))
        k = k.to(dev, non_blocking=False)
        v = v.to(dev, non_blocking=False)
        sl = torch.from_numpy(slots).to(dev)
        if self.int8:
            pa.pa_reshape_and_cache_int8(k, v, self.key_cache, self.value_cache, self.key_scale,
                                         self.value_scale, sl, self.dtype, stream)
        else:
            pa.pa_reshape_and_cache(k, v, self.key_cache, self.value_cache, sl, self.dtype, stream)

    def copy_blocks(self, pairs, stream=None):
        """Copy-on-write copies; pairs: int32 GPU tensor [n][2] of (src, dst)."""
        if self.int8:
            pa.pa_copy_blocks_int8(self.key_cache, self.value_cache, self.key_scale,
                                   self.value_scale, pairs, stream)
        else:
            pa.pa_copy_blocks(self.key_cache, self.value_cache, pairs, self.dtype, stream)

    def kv_bytes_per_token(self):
        """Bytes of K and V one cached token holds (INT8: codes and scales)."""
        if self.int8:
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        return 2 * self.num_kv_heads * self.head_dim * 2


class DecodeStep:
    """One decode step for the sequences ``seq_ids`` (fixed order).

    The block tables live on the GPU: they are uploaded whole once (and again
    by ``sync_tables`` after any allocator change other than this step's own
    appends); each step stages only the new tokens' slots, the context
    lengths, any copy-on-write pairs and the work list in pinned memory, and
    one pa_write_step launch brings them to the device, records each new
    token's block in the tables and writes the new K/V.

    ``grid`` picks the partitioned decode's grid: "list" (the work list of
    live partitions), "dense" (every partition slot, empty ones exit at
    once) or "auto" (see ``dense_grid``); ``last_grid`` names the one the
    last prepared step used.
    """

    RING = 8            # pinned staging buffers
    EVENT_EVERY = 4     # write launches per recorded event (<= RING)
    DENSE_RATIO = 3     # "auto": dense grid while it has <= this many times the list's workgroups

    def __init__(self, cache, seq_ids, num_q_heads, kernel="partitioned", partition_size=512,
                 max_context_len=None, scale=None, stream=None, grid="auto"):
        self.cache = cache
        self.seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        self.S = int(self.seq_ids.shape[0])
        self.num_q_heads = int(num_q_heads)
        if kernel not in ("partitioned", "single"):
            raise ValueError(kernel)
        if grid not in ("auto", "list", "dense"):
            raise ValueError(grid)
        self.kernel = kernel
        self.grid = grid
        self.last_grid = None        # the partitioned decode's grid of the last prepared step
        self.partition_size = int(partition_size)
        bs = cache.block_size
        if max_context_len is None:
            max_context_len = cache.num_blocks * bs
        self.max_context_len = int(max_context_len)
        self.mb = -(-self.max_context_len // bs)
        self.max_parts = -(-self.max_context_len // self.partition_size)
        self.scale = float(np.float32(1.0 / np.sqrt(cache.head_dim))) if scale is None else float(scale)
        self.stream = stream if stream is not None else torch.cuda.current_stream(cache.device)
        dev = cache.device

        # per-step metadata: built in ordinary (cached) host memory, copied in one
        # memcpy into a ring of pinned staging buffers (CPU stores straight into
        # pinned pages can be very slow), which the step's write launch reads.
        # Step k uses buffer k % RING; every EVENT_EVERY-th write launch records
        # an event when it has run, and before reusing a buffer the host waits
        # for the first such event at or after the buffer's previous step.
        # (Every event costs the stream a few microseconds, so not one per step.)
        self._stage = np.zeros(self._meta_bytes(), np.uint8)
        self._host = [torch.empty(self._meta_bytes(), dtype=torch.uint8, pin_memory=True)
                      for _ in range(self.RING)]
        self._num_items = [0] * self.RING
        self._num_cow = [0] * self.RING
        self._step = 0                               # steps prepared so far
        self._cur = 0
        self._recorded = collections.deque()         # (step, event) of recorded write launches
        self._spare = [Event(timing=True) for _ in range(self.RING // self.EVENT_EVERY + 2)]
        self._dev_meta = torch.empty(self._meta_bytes(), dtype=torch.uint8, device=dev)
        self.slot_mapping, self.context_lens, self.cow_pairs, self.work_items = \
            self._views(self._dev_meta)
        self.block_tables = torch.zeros((self.S, self.mb), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.S, self.num_q_heads, cache.head_dim), dtype=torch.int16,
                               device=dev)
        ws = pa.pa_decode_partitioned_workspace_size(self.S, self.num_q_heads, cache.head_dim,
                                                     self.max_context_len, self.partition_size)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.host_context_lens = np.zeros(self.S, np.int32)
        self.sync_tables()
        self._bind_calls()

    def _bind_calls(self):
        """Argument lists of the per-step library calls, built once: every
        buffer they name belongs to this object and is never reallocated, so
        a step fills in only what changes (counts, the new K/V and q, events).
        The per-step inputs are checked against the shapes fixed here."""
        c = self.cache
        S = self.S
        L = pa.lib()
        self._sm, self._cl, self._cow, self._items = \
            (t.numpy() for t in self._views(torch.from_numpy(self._stage)))
        self._src = np.empty(S, np.int32)
        self._dst = np.empty(S, np.int32)
        self._nitems = ctypes.c_int32()
        i64p, i32p = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
        self._append_call = (L.pa_alloc_append_slots, (
            c.allocator._h, self.seq_ids.ctypes.data_as(i64p), S, self._sm.ctypes.data_as(i64p),
            self._cl.ctypes.data_as(i32p), self._src.ctypes.data_as(i32p),
            self._dst.ctypes.data_as(i32p)))
        self._items_call = (L.pa_partition_work_items, (
            self._cl.ctypes.data, S, self.partition_size, self.max_parts, self._items.ctypes.data,
            self._items.shape[0], ctypes.byref(self._nitems)))
        o1, _, o3 = self._offsets()
        stream = self.stream.cuda_stream
        pools = [c.key_cache.data_ptr(), c.value_cache.data_ptr()]
        if c.int8:
            pools += [c.key_scale.data_ptr(), c.value_scale.data_ptr()]
        dt = [pa._dtype_code(c.dtype)] if c.int8 else []
        self._write_fn = L.pa_write_step_int8 if c.int8 else L.pa_write_step
        self._write_args = []
        for h in self._host:
            base = h.data_ptr()
            self._write_args.append([
                base, base + o1, base + o3, 0, self.slot_mapping.data_ptr(),
                self.context_lens.data_ptr(), self.work_items.data_ptr(),
                self.block_tables.data_ptr(), self.mb, None, None] + pools +
                [S, c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks] + dt + [stream, None])
        self._kv_shape = (S, c.num_kv_heads, c.head_dim)
        self._q_shape = (S, self.num_q_heads, c.head_dim)
        dec = [self.out.data_ptr(), None] + pools + [
            self.block_tables.data_ptr(), self.mb, self.context_lens.data_ptr(), S,
            self.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.num_blocks,
            self.max_context_len, self.scale, pa._dtype_code(c.dtype)]
        if self.kernel == "single":
            self._decode_fn = L.pa_decode_int8 if c.int8 else L.pa_decode
            self._decode_args = dec + [stream, None, None]
        else:
            self._decode_fn = L.pa_decode_partitioned_int8 if c.int8 else L.pa_decode_partitioned
            self._nitems_arg = len(dec) + 2
            self._decode_args = dec + [self.partition_size, self.work_items.data_ptr(), 0,
                                       self.workspace.data_ptr(),
                                       self.workspace.numel(), stream, None, None]

    def _check_input(self, t, shape, name):
        if tuple(t.shape) != shape or not t.is_cuda or t.element_size() != 2 or \
                not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 16-bit GPU tensor of shape {shape}")
        return t.data_ptr()

    # layout: slots int64 [S] | context_lens int32 [S] (+pad to 8 bytes) |
    #         cow pairs int32 [S][2] | work items int32 [S * max_parts][2]
    def _offsets(self):
        S = self.S
        o1 = 8 * S
        o2 = o1 + 4 * (S + (S & 1))
        o3 = o2 + 8 * S
        return o1, o2, o3

    def _meta_bytes(self):
        return self._offsets()[2] + 8 * self.S * self.max_parts

    def _views(self, buf):
        S = self.S
        o1, o2, o3 = self._offsets()
        sm = buf[:o1].view(torch.int64)
        cl = buf[o1:o1 + 4 * S].view(torch.int32)
        cow = buf[o2:o3].view(torch.int32).view(S, 2)
        items = buf[o3:].view(torch.int32).view(-1, 2)
        return sm, cl, cow, items

    def sync_tables(self):
        """Upload the allocator's current tables and lengths (blocking)."""
        tbl, lens = self.cache.allocator.block_tables(self.seq_ids, self.mb, pad=0)
        if int(lens.max(initial=0)) > self.max_context_len:
            raise ValueError("a sequence is longer than max_context_len")
        with torch.cuda.stream(self.stream):
            self.block_tables.copy_(torch.from_numpy(tbl))
            self.context_lens.copy_(torch.from_numpy(lens))
        self.stream.synchronize()
        self.host_context_lens[:] = lens

    @staticmethod
    def dense_grid(grid, max_parts, num_seqs, num_items, ratio, shared):
        """Whether the partitioned decode runs on its dense grid instead of
        the work list.  The work list has no empty workgroups and keeps each
        sequence's partitions on one XCD.  The dense grid, (max_parts | 1)
        partitions per (sequence, KV head) with empty ones exiting at once,
        puts partition p of KV head k on XCD (p + 3k) mod 8 for every
        sequence, so sequences that share prefix blocks read them through one
        XCD's L2: with 256 sequences sharing a 1024-token prefix it is ~5 %
        faster than the list, while without shared blocks the list is faster
        (16 long contexts: ~1.5 %).  "auto" takes the dense grid when the
        allocator holds shared blocks (`shared`) and the dense grid has at
        most `ratio` times the list's workgroups."""
        if grid == "dense":
            return True
        if grid == "list" or num_items <= 0:
            return False
        return bool(shared) and (max_parts | 1) * num_seqs <= ratio * num_items

    def prepare(self):
        """a1: one slot per sequence from the host allocator, staged in pinned
        memory with the lengths, copy-on-write pairs and work list.  Returns
        the index of the staging buffer."""
        k = self._step
        b = k % self.RING
        if k >= self.RING:                          # step k - RING's write must have run
            while self._recorded and self._recorded[0][0] < k - self.RING:
                self._spare.append(self._recorded.popleft()[1])
            if self._recorded:
                self._recorded[0][1].synchronize()
        if int(self.host_context_lens.max(initial=0)) >= self.max_context_len:
            raise ValueError("a sequence would outgrow max_context_len")
        fn, args = self._append_call
        pa._check(fn(*args))                        # slots and lengths into the staging area
        self.host_context_lens[:] = self._cl
        cow = np.flatnonzero(self._src >= 0)
        self._num_cow[b] = int(cow.size)
        if cow.size:
            self._cow[: cow.size, 0] = self._src[cow]
            self._cow[: cow.size, 1] = self._dst[cow]
        n = self._offsets()[1] + 8 * int(cow.size)
        if self.kernel == "partitioned":
            fn, args = self._items_call
            pa._check(fn(*args))
            nitems = self._nitems.value
            if self.dense_grid(self.grid, self.max_parts, self.S, nitems, self.DENSE_RATIO,
                               self.grid == "auto" and self.cache.allocator.num_shared_blocks() > 0):
                nitems = 0                          # no list: the decode takes the dense grid
            self.last_grid = "list" if nitems else "dense"
            self._num_items[b] = nitems
            n = self._offsets()[2] + 8 * nitems
        self._host[b].numpy()[:n] = self._stage[:n]
        return b

    def upload(self, b):
        """a2: the staged metadata reaches the device inside write_new's launch
        (pa_write_step reads the pinned staging buffer over the bus); only
        copy-on-write pairs, which pa_copy_blocks reads before that launch,
        are copied here."""
        self._cur = b
        self._step += 1
        self._ncow_dev = self._num_cow[b]
        self._nitems_dev = self._num_items[b]
        if self._ncow_dev:
            o2 = self._offsets()[1]
            n = 8 * self._ncow_dev
            with torch.cuda.stream(self.stream):
                self._dev_meta[o2:o2 + n].copy_(self._host[b][o2:o2 + n], non_blocking=True)

    def write_new(self, k_new, v_new):
        """a3: copy-on-write copies (if any), then one launch that copies the
        staged slots, lengths and work list to the device, records the new
        tokens' blocks in the tables and writes their K/V ([S][Hkv][D]) into
        their slots."""
        c = self.cache
        b = self._cur
        if self._ncow_dev:
            c.copy_blocks(self.cow_pairs[: self._ncow_dev], self.stream)
        args = self._write_args[b]
        args[3] = self._nitems_dev
        args[9] = self._check_input(k_new, self._kv_shape, "k_new")
        args[10] = self._check_input(v_new, self._kv_shape, "v_new")
        k = self._step - 1
        ev = None
        if k % self.EVENT_EVERY == self.EVENT_EVERY - 1:
            ev = self._spare.pop()                 # the launch records it when it has run
            self._recorded.append((k, ev))
        args[-1] = None if ev is None else ev.handle
        pa._check(self._write_fn(*args))

    def attend(self, q, start_event=None, stop_event=None):
        """a4 or a5+a6: decode for q [S][Hq][D] into self.out.  Optional
        ._hip.Event objects are recorded by the decode's launches themselves
        when it starts and ends."""
        args = self._decode_args
        args[1] = self._check_input(q, self._q_shape, "q")
        if self.kernel == "partitioned":
            # a list with no items would mean no live partition: the dense
            # grid is asked for with a NULL list
            n = self._nitems_dev
            args[self._nitems_arg - 1] = self.work_items.data_ptr() if n else None
            args[self._nitems_arg] = n
        args[-2] = None if start_event is None else start_event.handle
        args[-1] = None if stop_event is None else stop_event.handle
        pa._check(self._decode_fn(*args))
        return self.out

    def __call__(self, q, k_new, v_new):
        """The whole step: a1, a2, a3, then the decode.  Asynchronous on the stream."""
        b = self.prepare()
        self.upload(b)
        self.write_new(k_new, v_new)
        return self.attend(q)

    def kv_bytes(self):
        """Logical K+V bytes the last prepared step's decode reads."""
        return int(self.host_context_lens.astype(np.int64).sum()) * self.cache.kv_bytes_per_token()
