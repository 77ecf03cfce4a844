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

    def _take_free(self):
        return self.free_blocks.pop(0)

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
            block = self._take_free()
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
            new = self._take_free()
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


class PrefixCachingBlockManagerModel(BlockManagerModel):
    """The block manager with automatic prefix caching, as the pages describe
    it: page "LLM推理优化：vLLM PagedAttention深度解析与工程实践", §4.2 (a block
    whose KV equals the same prefix of an earlier request is reused), and the
    Qwen2.5-7B vLLM 0.6.3 deployment page, §3.2 (prompts are cut into
    fixed-size blocks, each block keyed by a hash of its token ids; a hit needs
    a token-exact prefix that ends on a block boundary, so a change in the
    first block loses every later one).

    The cache is written here by its definition, not by hashing: the key of
    the i-th full block of a prompt is the tuple of ALL prompt tokens up to
    the end of that block, which is exactly what a chained block hash stands
    for, with no possible collision.

    Readings where the pages are silent (each stated, none of them theirs):

    * only full blocks are cached; a prompt's full blocks are registered when
      the prompt is allocated (its prefill writes them before anything later
      in the stream can read them);
    * the longest cached prefix is reused, but never the block that holds the
      prompt's last token: that token's query is needed for the next token,
      so at least one token is always computed, into a block the sequence
      owns;
    * a block whose count falls to zero stays cached while it waits in the
      free pool, and loses its cache entry only when the pool hands it out
      again; a hit on such a block takes it out of the pool;
    * a cached block keeps its entry when a block of a shorter prefix loses
      its own (its KV still belongs to the same tokens); the walk stops at
      the first block that is not cached, so such a block is reused again
      once the shorter prefix is cached anew;
    * a key that is already cached keeps its block (a duplicate block of the
      same prefix is simply not registered);
    * with caching on, a freed sequence returns its blocks to the pool tail
      deepest first (reverse table order), so that the ends of cached
      prefixes are handed out before their beginnings.
    """

    def __init__(self, num_blocks, block_size, initial_free_order=None, prefix_caching=True):
        super().__init__(num_blocks, block_size, initial_free_order)
        self.prefix_caching = bool(prefix_caching)
        self.cached = {}        # tuple(prompt tokens up to the end of a block) -> block id
        self.block_key = {}     # block id -> its key, for cached blocks

    def set_prefix_caching(self, enabled):
        """Turning caching off (or on again) forgets every cached block."""
        self.prefix_caching = bool(enabled)
        self.cached = {}
        self.block_key = {}

    def _forget(self, block):
        key = self.block_key.pop(block, None)
        if key is not None:
            del self.cached[key]

    def _take_free(self):
        block = self.free_blocks.pop(0)
        self._forget(block)
        return block

    def cached_prefix_blocks(self, tokens):
        """Cached blocks for the longest reusable block-aligned prefix."""
        tokens = list(tokens)
        bs = self.block_size
        hits = []
        if not self.prefix_caching:
            return hits
        for i in range((len(tokens) - 1) // bs if tokens else 0):
            key = tuple(tokens[: (i + 1) * bs])
            if key not in self.cached:
                break
            hits.append(self.cached[key])
        return hits

    def allocate_prompt(self, seq_id, tokens):
        """New sequence holding the prompt; returns the number of leading
        tokens whose KV is already cached (a multiple of block_size)."""
        tokens = [int(t) for t in tokens]
        if seq_id in self.tables:
            raise ValueError("sequence already exists")
        bs = self.block_size
        n = len(tokens)
        hits = self.cached_prefix_blocks(tokens)
        fresh = -(-n // bs) - len(hits)
        taken_from_pool = fresh + sum(1 for b in hits if self.refcount[b] == 0)
        if taken_from_pool > len(self.free_blocks):
            raise OOM("not enough free blocks")
        for b in hits:
            if self.refcount[b] == 0:
                self.free_blocks.remove(b)
            self.refcount[b] += 1
        table = list(hits)
        for _ in range(fresh):
            b = self._take_free()
            self.refcount[b] = 1
            table.append(b)
        if self.prefix_caching:
            for i in range(len(hits), n // bs):
                key = tuple(tokens[: (i + 1) * bs])
                if key not in self.cached:
                    self.cached[key] = table[i]
                    self.block_key[table[i]] = key
        self.tables[seq_id] = table
        self.num_tokens[seq_id] = n
        return len(hits) * bs

    def free(self, seq_id):
        if not self.prefix_caching:
            return super().free(seq_id)
        for block_id in reversed(self.tables.get(seq_id, [])):
            self.refcount[block_id] -= 1
            if self.refcount[block_id] == 0:
                self.free_blocks.append(block_id)
        self.tables.pop(seq_id, None)
        self.num_tokens.pop(seq_id, None)
