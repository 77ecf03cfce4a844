"""Reference model of the paged-KV block allocator, in plain Python lists.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

It follows the BlockManager pseudocode of page
"LLM推理优化：vLLM PagedAttention深度解析与工程实践", §3.2 (Block Manager core
flow), extended with the sharing rules of page
"vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.3 (BlockSpaceManager:
append_slot / free / copy-on-write sharing):

* the free pool is a list; blocks are taken from its head (``pop(0)``) and
  returned to its tail (``append``);
* ``allocate(seq, n)`` grows a sequence to hold ``n`` tokens: nothing happens
  when the blocks it already has cover ``n`` tokens; otherwise it needs
  ``ceil((n - have) / bs)`` more blocks, and if the pool holds fewer it
  raises OOM *before* taking any (the garbled comparisons of the pseudocode
  are read as ``>=`` and ``<``);
* ``append_slot(seq)`` writes one more token: into the current block if it is
  not full, else into a fresh block from the pool.  The slot of position ``p``
  is ``table[p // bs] * bs + p % bs``;
* blocks can be shared by reference (a shared prefix, a fork); each block has
  a reference count, and a block goes back to the pool only when its count
  reaches zero;
* a shared block is copied only when a sharer is about to write into it
  (copy-on-write): the writer gets a fresh block, the old one loses a
  reference, and the caller is told (old, new) so it can copy the contents.
"""


class OOM(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        if initial_free_order is None:
            initial_free_order = list(range(num_blocks))
        initial_free_order = [int(b) for b in initial_free_order]
        if sorted(initial_free_order) != list(range(num_blocks)):
            raise ValueError("initial free order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_blocks = list(initial_free_order)
        self.tables = {}        # seq_id -> [physical block ids]
        self.num_tokens = {}    # seq_id -> tokens held
        self.refcount = [0] * num_blocks

    # -- growth ----------------------------------------------------------------
    def allocate(self, seq_id, num_tokens):
        table = self.tables.get(seq_id, [])
        have = len(table) * self.block_size
        if have >= num_tokens:
            self.tables.setdefault(seq_id, table)
            self.num_tokens[seq_id] = max(self.num_tokens.get(seq_id, 0), num_tokens)
            return
        needed = -(-(num_tokens - have) // self.block_size)
        if len(self.free_blocks) < needed:
            raise OOM("not enough free blocks")
        for _ in range(needed):
            block = self.free_blocks.pop(0)
            self.refcount[block] = 1
            table.append(block)
        self.tables[seq_id] = table
        self.num_tokens[seq_id] = max(self.num_tokens.get(seq_id, 0), num_tokens)

    def append_slot(self, seq_id):
        """Returns (slot, cow) where cow is None or (old_block, new_block)."""
        p = self.num_tokens.get(seq_id, 0)
        table = self.tables.get(seq_id, [])
        idx = p // self.block_size
        need_new = idx >= len(table)
        need_cow = (not need_new) and self.refcount[table[idx]] > 1
        if (need_new or need_cow) and not self.free_blocks:
            raise OOM("not enough free blocks")
        cow = None
        if need_new:
            self.allocate(seq_id, p + 1)
            table = self.tables[seq_id]
        elif need_cow:
            old = table[idx]
            new = self.free_blocks.pop(0)
            self.refcount[old] -= 1
            self.refcount[new] = 1
            table[idx] = new
            cow = (old, new)
        self.tables[seq_id] = table
        self.num_tokens[seq_id] = p + 1
        slot = table[idx] * self.block_size + p % self.block_size
        return slot, cow

    # -- sharing ---------------------------------------------------------------
    def share_prefix(self, src_seq, dst_seq, num_tokens):
        """dst (new) references the first num_tokens (block-aligned) of src."""
        if num_tokens % self.block_size != 0:
            raise ValueError("shared prefix must be block-aligned")
        if dst_seq in self.tables:
            raise ValueError("destination sequence already exists")
        if num_tokens > self.num_tokens.get(src_seq, 0) or num_tokens <= 0:
            raise ValueError("prefix longer than the source")
        blocks = self.tables[src_seq][: num_tokens // self.block_size]
        for b in blocks:
            self.refcount[b] += 1
        self.tables[dst_seq] = list(blocks)
        self.num_tokens[dst_seq] = num_tokens

    def fork(self, src_seq, dst_seq):
        """dst (new) references every block of src, partial last block included."""
        if dst_seq in self.tables:
            raise ValueError("destination sequence already exists")
        if src_seq not in self.tables:
            raise ValueError("unknown source sequence")
        for b in self.tables[src_seq]:
            self.refcount[b] += 1
        self.tables[dst_seq] = list(self.tables[src_seq])
        self.num_tokens[dst_seq] = self.num_tokens[src_seq]

    # -- release -----------------------------------------------------------------
    def free(self, seq_id):
        for block_id in self.tables.get(seq_id, []):
            self.refcount[block_id] -= 1
            if self.refcount[block_id] == 0:
                self.free_blocks.append(block_id)
        self.tables.pop(seq_id, None)
        self.num_tokens.pop(seq_id, None)

    # -- queries -------------------------------------------------------------------
    def block_table(self, seq_id):
        return list(self.tables[seq_id])

    def slot(self, seq_id, pos):
        table = self.tables[seq_id]
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def slots(self, seq_id, begin, end):
        return [self.slot(seq_id, p) for p in range(begin, end)]

    def num_free(self):
        return len(self.free_blocks)
