"""A paged KV cache on one GPU and its decode step.

``PagedKVCache`` owns the two device pools ([num_blocks][block_size][Hkv][D],
16-bit) and the host block allocator.  ``DecodeStep`` runs one decode step for
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

import numpy as np
import torch

from . import _native as pa
from ._hip import Event

POISON = {"f16": 0x7E00, "bf16": 0x7FC0}   # quiet-NaN patterns for unused slots


def _dtype(dtype):
    return "f16" if pa._dtype_code(dtype) == pa.PA_F16 else "bf16"


class PagedKVCache:
    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                 initial_free_order=None, device="cuda", poison=True):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.dtype = _dtype(dtype)
        self.device = torch.device(device)
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        fill = POISON[self.dtype] if poison else 0
        self.key_cache = torch.full(shape, fill, dtype=torch.int16, device=self.device)
        self.value_cache = torch.full(shape, fill, dtype=torch.int16, device=self.device)
        self.allocator = pa.Allocator(self.num_blocks, self.block_size, initial_free_order)

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
        pa.pa_reshape_and_cache(k, v, self.key_cache, self.value_cache, sl, self.dtype, stream)

    def kv_bytes_per_token(self):
        return 2 * self.num_kv_heads * self.head_dim * 2


class DecodeStep:
    """One decode step for the sequences ``seq_ids`` (fixed order).

    The block tables live on the GPU: they are uploaded whole once (and again
    by ``sync_tables`` after any allocator change other than this step's own
    appends); each step stages only the new tokens' slots, the context
    lengths, any copy-on-write pairs and the work list in pinned memory, and
    one pa_write_step launch brings them to the device, records each new
    token's block in the tables and writes the new K/V.
    """

    RING = 8            # pinned staging buffers
    EVENT_EVERY = 4     # write launches per recorded event (<= RING)

    def __init__(self, cache, seq_ids, num_q_heads, kernel="partitioned", partition_size=512,
                 max_context_len=None, scale=None, stream=None):
        self.cache = cache
        self.seq_ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        self.S = int(self.seq_ids.shape[0])
        self.num_q_heads = int(num_q_heads)
        if kernel not in ("partitioned", "single"):
            raise ValueError(kernel)
        self.kernel = kernel
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

    def prepare(self):
        """a1: one slot per sequence from the host allocator, staged in pinned
        memory.  Returns the index of the staging buffer."""
        k = self._step
        b = k % self.RING
        if k >= self.RING:                          # step k - RING's write must have run
            while self._recorded and self._recorded[0][0] < k - self.RING:
                self._spare.append(self._recorded.popleft()[1])
            if self._recorded:
                self._recorded[0][1].synchronize()
        sm, cl, cow, items = (t.numpy() for t in self._views(torch.from_numpy(self._stage)))
        if int(self.host_context_lens.max(initial=0)) >= self.max_context_len:
            raise ValueError("a sequence would outgrow max_context_len")
        _, _, src, dst = self.cache.allocator.append_slots(
            self.seq_ids, slots_out=sm, context_lens_out=self.host_context_lens)
        cl[:] = self.host_context_lens
        k = np.flatnonzero(src >= 0)
        self._num_cow[b] = int(k.size)
        if k.size:
            cow[: k.size, 0] = src[k]
            cow[: k.size, 1] = dst[k]
        n = self._offsets()[1] + 8 * int(k.size)
        if self.kernel == "partitioned":
            wl = pa.partition_work_items(self.host_context_lens, self.partition_size, self.max_parts)
            items[: wl.shape[0]] = wl
            self._num_items[b] = int(wl.shape[0])
            n = self._offsets()[2] + 8 * int(wl.shape[0])
        self._host[b].numpy()[:n] = self._stage[:n]
        self._nbytes = n
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
            pa.pa_copy_blocks(c.key_cache, c.value_cache, self.cow_pairs[: self._ncow_dev],
                              c.dtype, self.stream)
        sm, cl, _, items = self._views(self._host[b])
        n = self._nitems_dev
        k = self._step - 1
        ev = None
        if k % self.EVENT_EVERY == self.EVENT_EVERY - 1:
            ev = self._spare.pop()                 # the launch records it when it has run
            self._recorded.append((k, ev))
        pa.pa_write_step(sm, cl, items[:n] if n else None, self.slot_mapping, self.context_lens,
                         self.work_items, self.block_tables, k_new, v_new, c.key_cache,
                         c.value_cache, self.stream, done_event=ev)

    def attend(self, q, start_event=None, stop_event=None):
        """a4 or a5+a6: decode for q [S][Hq][D] into self.out.  Optional
        ._hip.Event objects are recorded by the decode's launches themselves
        when it starts and ends."""
        c = self.cache
        if self.kernel == "single":
            pa.pa_decode(self.out, q, c.key_cache, c.value_cache, self.block_tables,
                         self.context_lens, self.max_context_len, self.scale, c.dtype, self.stream,
                         start_event, stop_event)
        else:
            pa.pa_decode_partitioned(self.out, q, c.key_cache, c.value_cache, self.block_tables,
                                     self.context_lens, self.max_context_len, self.scale, c.dtype,
                                     self.partition_size, self.workspace,
                                     self.work_items[: self._nitems_dev], self.stream,
                                     start_event, stop_event)
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
