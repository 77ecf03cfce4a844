// pa_allocator.cpp -- libpa's host block allocator.
//
// The block manager of "LLM推理优化：vLLM PagedAttention深度解析与工程实践",
// §3.2 (free pool, per-sequence physical block list, ceil growth, the pool
// checked before any block is taken) with the sharing rules of
// "vLLM 深度拆解：当大模型推理学会「分页注意力」", §3.3 (append_slot into the
// current block or a fresh one, free returns blocks, shared blocks are
// referenced and copied only before a sharer writes into one), and automatic
// prefix caching (the first page, §4.2; the Qwen2.5-7B vLLM 0.6.3 deployment
// page, §3.2): a prompt's full blocks are keyed by their token ids chained to
// the key of the block before them, and a later prompt with the same
// block-aligned token prefix reuses them.
//
// Data structures, sized once at creation:
//   free pool   intrusive doubly linked list over block ids (next/prev
//               arrays): pop at head, push at tail, unlink from the middle
//               (a cached block taken back out of the pool), all O(1)
//   refcount    one int32 per physical block (0 <=> the block is in the pool)
//   sequences   hash map seq_id -> {block ids in logical order, token count}
//   prefix      per block: node id (0: not cached), parent node id, its
//   cache       block_size token ids; a hash index (parent node, tokens) ->
//               block, every hit verified token by token, so a match is
//               exact whatever the hash does
// Every failing call returns before changing anything.
//
// Why node ids and not content hashes: a cached block's key names its parent
// by the node id the parent got when it was cached, so equal keys mean equal
// token prefixes, with no collision possible.  The keys stay valid because
// the cached prefixes are closed under shortening: a block is only ever held
// together with the blocks of its prefix, and frees return a sequence's
// blocks deepest first, so a parent never goes back out of the pool before
// its cached children.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> next, prev;  // free pool links, -1 at the ends
  int32_t head = -1, tail = -1;
  int64_t count = 0;                // ids in the pool
  std::vector<int32_t> refcount;
  int64_t shared = 0;               // blocks with refcount >= 2
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t tokens = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache (arrays sized when caching is first turned on)
  bool caching = false;
  uint64_t next_node = 1;
  std::vector<uint64_t> node;        // node id of a cached block, 0 if not cached
  std::vector<uint64_t> parent;      // node id of the block before it (0: first block)
  std::vector<int32_t> cached_ids;   // [num_blocks][block_size] token ids
  std::unordered_multimap<uint64_t, int32_t> index;

  void unlink(int32_t id) {
    const int32_t p = prev[static_cast<size_t>(id)], n = next[static_cast<size_t>(id)];
    if (p >= 0) next[static_cast<size_t>(p)] = n; else head = n;
    if (n >= 0) prev[static_cast<size_t>(n)] = p; else tail = p;
    --count;
  }
  void push_back(int32_t id) {
    prev[static_cast<size_t>(id)] = tail;
    next[static_cast<size_t>(id)] = -1;
    if (tail >= 0) next[static_cast<size_t>(tail)] = id; else head = id;
    tail = id;
    ++count;
  }
  // take the pool's first block; a cached block leaves the cache as it goes
  int32_t pop_front() {
    const int32_t id = head;
    unlink(id);
    forget(id);
    return id;
  }

  // mixing step of SplitMix64 (Steele, Lea and Flood, "Fast splittable
  // pseudorandom number generators", OOPSLA 2014); only spreads the index
  static uint64_t mix(uint64_t x) {
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ULL;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebULL;
    return x ^ (x >> 31);
  }
  uint64_t key_hash(uint64_t parent_node, const int32_t* ids) const {
    uint64_t h = mix(parent_node + 0x9e3779b97f4a7c15ULL);
    for (int32_t i = 0; i < block_size; ++i) h = mix(h ^ static_cast<uint32_t>(ids[i]));
    return h;
  }
  const int32_t* ids_of(int32_t b) const {
    return cached_ids.data() + static_cast<size_t>(b) * static_cast<size_t>(block_size);
  }
  // the cached block whose prefix is (parent_node's prefix, ids), or -1
  int32_t lookup(uint64_t parent_node, const int32_t* ids) const {
    auto range = index.equal_range(key_hash(parent_node, ids));
    for (auto it = range.first; it != range.second; ++it) {
      const int32_t b = it->second;
      if (parent[static_cast<size_t>(b)] == parent_node &&
          std::memcmp(ids_of(b), ids, sizeof(int32_t) * static_cast<size_t>(block_size)) == 0)
        return b;
    }
    return -1;
  }
  void remember(int32_t b, uint64_t parent_node, const int32_t* ids) {
    node[static_cast<size_t>(b)] = next_node++;
    parent[static_cast<size_t>(b)] = parent_node;
    std::memcpy(cached_ids.data() + static_cast<size_t>(b) * static_cast<size_t>(block_size), ids,
                sizeof(int32_t) * static_cast<size_t>(block_size));
    index.emplace(key_hash(parent_node, ids), b);
  }
  void forget(int32_t b) {
    if (node.empty() || node[static_cast<size_t>(b)] == 0) return;
    auto range = index.equal_range(key_hash(parent[static_cast<size_t>(b)], ids_of(b)));
    for (auto it = range.first; it != range.second; ++it) {
      if (it->second == b) {
        index.erase(it);
        break;
      }
    }
    node[static_cast<size_t>(b)] = 0;
  }
  void forget_all() {
    index.clear();
    std::fill(node.begin(), node.end(), uint64_t{0});
  }

  int64_t capacity_of(const Seq& s) const {
    return static_cast<int64_t>(s.blocks.size()) * block_size;
  }
  // blocks allocate(seq, n) would take
  int64_t blocks_needed(const Seq* s, int64_t n) const {
    const int64_t have = s ? capacity_of(*s) : 0;
    if (have >= n) return 0;
    return (n - have + block_size - 1) / block_size;
  }
  // every refcount change goes through here, keeping `shared` current
  void set_ref(int32_t id, int32_t v) {
    int32_t& rc = refcount[static_cast<size_t>(id)];
    shared += static_cast<int64_t>(v > 1) - static_cast<int64_t>(rc > 1);
    rc = v;
  }
  int32_t ref(int32_t id) const { return refcount[static_cast<size_t>(id)]; }
  // does one more token of s need a block from the pool (new or copy-on-write)?
  bool append_needs_block(const Seq* s) const {
    if (!s) return true;
    const int64_t p = s->tokens;
    const int64_t idx = p / block_size;
    if (idx >= static_cast<int64_t>(s->blocks.size())) return true;
    return refcount[static_cast<size_t>(s->blocks[static_cast<size_t>(idx)])] > 1;
  }
  // append one token; the caller has checked that the pool can serve it
  int64_t append(int64_t seq_id, int32_t* cow_src, int32_t* cow_dst) {
    Seq& s = seqs[seq_id];
    const int64_t p = s.tokens;
    const size_t idx = static_cast<size_t>(p / block_size);
    int32_t src = -1, dst = -1;
    if (idx >= s.blocks.size()) {
      const int32_t id = pop_front();
      set_ref(id, 1);
      s.blocks.push_back(id);
    } else if (refcount[static_cast<size_t>(s.blocks[idx])] > 1) {
      src = s.blocks[idx];
      dst = pop_front();
      set_ref(src, ref(src) - 1);
      set_ref(dst, 1);
      s.blocks[idx] = dst;
    }
    s.tokens = static_cast<int32_t>(p + 1);
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    return static_cast<int64_t>(s.blocks[idx]) * block_size + p % block_size;
  }
};

namespace {

pa_status invalid(const char* msg) { return pa::fail(PA_ERR_INVALID_ARG, msg); }

const pa_allocator::Seq* find(const pa_allocator* a, int64_t seq_id) {
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order,
                          pa_allocator** out) {
  pa::clear_error();
  if (!out) return invalid("pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return invalid("pa_alloc_create: num_blocks and block_size must be positive");
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return pa::fail(PA_ERR_OOM, "pa_alloc_create: host allocation failed");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->next.assign(static_cast<size_t>(num_blocks), -1);
  a->prev.assign(static_cast<size_t>(num_blocks), -1);
  a->refcount.assign(static_cast<size_t>(num_blocks), 0);
  if (initial_free_order) {
    std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t id = initial_free_order[i];
      if (id < 0 || id >= num_blocks || seen[static_cast<size_t>(id)]) {
        delete a;
        return invalid("pa_alloc_create: initial_free_order is not a permutation");
      }
      seen[static_cast<size_t>(id)] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) a->push_back(initial_free_order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->push_back(i);
  }
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

pa_status pa_alloc_allocate(pa_allocator* a, int64_t seq_id, int32_t num_tokens) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_allocate: allocator is NULL");
  if (num_tokens < 0) return invalid("pa_alloc_allocate: num_tokens < 0");
  const pa_allocator::Seq* s = find(a, seq_id);
  const int64_t need = a->blocks_needed(s, num_tokens);
  if (need > a->count) return pa::fail(PA_ERR_OOM, "pa_alloc_allocate: not enough free blocks");
  pa_allocator::Seq& seq = a->seqs[seq_id];
  for (int64_t k = 0; k < need; ++k) {
    const int32_t id = a->pop_front();
    a->set_ref(id, 1);
    seq.blocks.push_back(id);
  }
  if (num_tokens > seq.tokens) seq.tokens = num_tokens;
  return PA_OK;
}

pa_status pa_alloc_append_slot(pa_allocator* a, int64_t seq_id, int64_t* slot_out,
                               int32_t* cow_src, int32_t* cow_dst) {
  pa::clear_error();
  if (!a || !slot_out) return invalid("pa_alloc_append_slot: NULL argument");
  const pa_allocator::Seq* s = find(a, seq_id);
  if (s && s->tokens == INT32_MAX) return invalid("pa_alloc_append_slot: sequence full");
  if (a->append_needs_block(s) && a->count < 1)
    return pa::fail(PA_ERR_OOM, "pa_alloc_append_slot: not enough free blocks");
  *slot_out = a->append(seq_id, cow_src, cow_dst);
  return PA_OK;
}

pa_status pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int64_t* slots_out, int32_t* context_lens_out, int32_t* cow_src,
                                int32_t* cow_dst) {
  pa::clear_error();
  if (!a || n < 0 || (n > 0 && (!seq_ids || !slots_out)))
    return invalid("pa_alloc_append_slots: bad argument");
  std::unordered_set<int64_t> distinct;
  distinct.reserve(static_cast<size_t>(n) * 2);
  int64_t need = 0;
  for (int32_t k = 0; k < n; ++k) {
    if (!distinct.insert(seq_ids[k]).second)
      return invalid("pa_alloc_append_slots: sequence ids must be distinct");
    const pa_allocator::Seq* s = find(a, seq_ids[k]);
    if (s && s->tokens == INT32_MAX) return invalid("pa_alloc_append_slots: sequence full");
    need += a->append_needs_block(s) ? 1 : 0;
  }
  if (need > a->count)
    return pa::fail(PA_ERR_OOM, "pa_alloc_append_slots: not enough free blocks");
  for (int32_t k = 0; k < n; ++k) {
    slots_out[k] = a->append(seq_ids[k], cow_src ? cow_src + k : nullptr,
                             cow_dst ? cow_dst + k : nullptr);
    if (context_lens_out) context_lens_out[k] = a->seqs[seq_ids[k]].tokens;
  }
  return PA_OK;
}

pa_status pa_alloc_share_prefix(pa_allocator* a, int64_t src_seq, int64_t dst_seq,
                                int32_t num_tokens) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_share_prefix: allocator is NULL");
  const pa_allocator::Seq* s = find(a, src_seq);
  if (!s) return invalid("pa_alloc_share_prefix: unknown source sequence");
  if (find(a, dst_seq)) return invalid("pa_alloc_share_prefix: destination exists");
  if (num_tokens <= 0 || num_tokens % a->block_size != 0 || num_tokens > s->tokens)
    return invalid("pa_alloc_share_prefix: prefix must be block-aligned and within the source");
  const size_t nblk = static_cast<size_t>(num_tokens / a->block_size);
  std::vector<int32_t> blocks(s->blocks.begin(), s->blocks.begin() + static_cast<long>(nblk));
  for (int32_t id : blocks) a->set_ref(id, a->ref(id) + 1);
  pa_allocator::Seq& d = a->seqs[dst_seq];
  d.blocks = std::move(blocks);
  d.tokens = num_tokens;
  return PA_OK;
}

pa_status pa_alloc_fork(pa_allocator* a, int64_t src_seq, int64_t dst_seq) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_fork: allocator is NULL");
  const pa_allocator::Seq* s = find(a, src_seq);
  if (!s) return invalid("pa_alloc_fork: unknown source sequence");
  if (find(a, dst_seq)) return invalid("pa_alloc_fork: destination exists");
  pa_allocator::Seq copy = *s;
  for (int32_t id : copy.blocks) a->set_ref(id, a->ref(id) + 1);
  a->seqs[dst_seq] = std::move(copy);
  return PA_OK;
}

pa_status pa_alloc_free(pa_allocator* a, int64_t seq_id) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_free: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_OK;
  const std::vector<int32_t>& blocks = it->second.blocks;
  const size_t nb = blocks.size();
  for (size_t k = 0; k < nb; ++k) {
    // with caching on, deepest block first: a cached prefix leaves the pool end first
    const int32_t id = blocks[a->caching ? nb - 1 - k : k];
    a->set_ref(id, a->ref(id) - 1);
    if (a->ref(id) == 0) a->push_back(id);
  }
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_alloc_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out,
                               int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (!a || !n_out) return invalid("pa_alloc_block_table: NULL argument");
  const pa_allocator::Seq* s = find(a, seq_id);
  if (!s) return invalid("pa_alloc_block_table: unknown sequence");
  const int32_t n = static_cast<int32_t>(s->blocks.size());
  *n_out = n;
  if (n > cap || (n > 0 && !out)) return invalid("pa_alloc_block_table: output too small");
  if (n) std::memcpy(out, s->blocks.data(), sizeof(int32_t) * static_cast<size_t>(n));
  return PA_OK;
}

pa_status pa_alloc_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                                int32_t* out, int32_t max_blocks_per_seq, int32_t pad,
                                int32_t* context_lens_out) {
  pa::clear_error();
  if (!a || n < 0 || max_blocks_per_seq <= 0 || (n > 0 && (!seq_ids || !out)))
    return invalid("pa_alloc_block_tables: bad argument");
  for (int32_t k = 0; k < n; ++k) {
    const pa_allocator::Seq* s = find(a, seq_ids[k]);
    if (!s) return invalid("pa_alloc_block_tables: unknown sequence");
    if (static_cast<int64_t>(s->blocks.size()) > max_blocks_per_seq)
      return invalid("pa_alloc_block_tables: a table is longer than max_blocks_per_seq");
  }
  for (int32_t k = 0; k < n; ++k) {
    const pa_allocator::Seq* s = find(a, seq_ids[k]);
    int32_t* row = out + static_cast<int64_t>(k) * max_blocks_per_seq;
    const size_t nb = s->blocks.size();
    if (nb) std::memcpy(row, s->blocks.data(), sizeof(int32_t) * nb);
    for (size_t j = nb; j < static_cast<size_t>(max_blocks_per_seq); ++j) row[j] = pad;
    if (context_lens_out) context_lens_out[k] = s->tokens;
  }
  return PA_OK;
}

pa_status pa_alloc_slots(const pa_allocator* a, int64_t seq_id, int32_t begin, int32_t end,
                         int64_t* out) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_slots: allocator is NULL");
  const pa_allocator::Seq* s = find(a, seq_id);
  if (!s) return invalid("pa_alloc_slots: unknown sequence");
  if (begin < 0 || end < begin || end > s->tokens || (end > begin && !out))
    return invalid("pa_alloc_slots: range outside the sequence");
  for (int32_t p = begin; p < end; ++p)
    out[p - begin] = static_cast<int64_t>(s->blocks[static_cast<size_t>(p / a->block_size)]) *
                         a->block_size + p % a->block_size;
  return PA_OK;
}

int32_t pa_alloc_num_tokens(const pa_allocator* a, int64_t seq_id) {
  if (!a) return -1;
  const pa_allocator::Seq* s = find(a, seq_id);
  return s ? s->tokens : -1;
}

int32_t pa_alloc_num_free(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->count) : -1;
}

int32_t pa_alloc_num_shared_blocks(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->shared) : -1;
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block_id) {
  if (!a || block_id < 0 || block_id >= a->num_blocks) return -1;
  return a->refcount[static_cast<size_t>(block_id)];
}

pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (!a || !n_out) return invalid("pa_alloc_free_list: NULL argument");
  *n_out = static_cast<int32_t>(a->count);
  if (a->count > cap || (a->count > 0 && !out))
    return invalid("pa_alloc_free_list: output too small");
  int64_t k = 0;
  for (int32_t id = a->head; id >= 0; id = a->next[static_cast<size_t>(id)]) out[k++] = id;
  return PA_OK;
}

pa_status pa_alloc_set_prefix_caching(pa_allocator* a, int32_t enabled) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_set_prefix_caching: allocator is NULL");
  if (enabled && a->node.empty()) {
    const size_t nb = static_cast<size_t>(a->num_blocks);
    const size_t ids = nb * static_cast<size_t>(a->block_size);
    try {
      a->node.assign(nb, 0);
      a->parent.assign(nb, 0);
      a->cached_ids.assign(ids, 0);
    } catch (const std::bad_alloc&) {
      a->node.clear();
      a->parent.clear();
      a->cached_ids.clear();
      return pa::fail(PA_ERR_OOM, "pa_alloc_set_prefix_caching: host allocation failed");
    }
  }
  a->forget_all();
  a->caching = enabled != 0;
  return PA_OK;
}

pa_status pa_alloc_allocate_prompt(pa_allocator* a, int64_t seq_id, const int32_t* tokens,
                                   int32_t num_tokens, int32_t* cached_tokens_out) {
  pa::clear_error();
  if (!a) return invalid("pa_alloc_allocate_prompt: allocator is NULL");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens))
    return invalid("pa_alloc_allocate_prompt: bad token array");
  if (find(a, seq_id)) return invalid("pa_alloc_allocate_prompt: sequence exists");
  const int32_t bs = a->block_size;
  const int64_t nblk = (static_cast<int64_t>(num_tokens) + bs - 1) / bs;
  // longest cached block-aligned prefix, short of the block holding the last token
  std::vector<int32_t> hits;
  uint64_t chain = 0;
  if (a->caching && num_tokens > 0) {
    const int64_t cap = (static_cast<int64_t>(num_tokens) - 1) / bs;
    for (int64_t i = 0; i < cap; ++i) {
      const int32_t b = a->lookup(chain, tokens + i * bs);
      if (b < 0) break;
      hits.push_back(b);
      chain = a->node[static_cast<size_t>(b)];
    }
  }
  int64_t from_pool = nblk - static_cast<int64_t>(hits.size());
  for (int32_t b : hits) from_pool += a->refcount[static_cast<size_t>(b)] == 0 ? 1 : 0;
  if (from_pool > a->count)
    return pa::fail(PA_ERR_OOM, "pa_alloc_allocate_prompt: not enough free blocks");
  pa_allocator::Seq& s = a->seqs[seq_id];
  s.blocks.reserve(static_cast<size_t>(nblk));
  for (int32_t b : hits) {
    if (a->ref(b) == 0) a->unlink(b);
    a->set_ref(b, a->ref(b) + 1);
    s.blocks.push_back(b);
  }
  for (int64_t k = static_cast<int64_t>(hits.size()); k < nblk; ++k) {
    const int32_t id = a->pop_front();
    a->set_ref(id, 1);
    s.blocks.push_back(id);
  }
  // cache the prompt's other full blocks; a prefix cached already keeps its block
  if (a->caching) {
    for (int64_t i = static_cast<int64_t>(hits.size()); i < num_tokens / bs; ++i) {
      const int32_t* ids = tokens + i * bs;
      const int32_t have = a->lookup(chain, ids);
      const int32_t b = have >= 0 ? have : s.blocks[static_cast<size_t>(i)];
      if (have < 0) a->remember(b, chain, ids);
      chain = a->node[static_cast<size_t>(b)];
    }
  }
  s.tokens = num_tokens;
  if (cached_tokens_out) *cached_tokens_out = static_cast<int32_t>(hits.size()) * bs;
  return PA_OK;
}

int32_t pa_alloc_num_cached_blocks(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->index.size()) : -1;
}

pa_status pa_partition_work_items(const int32_t* context_lens, int32_t num_seqs,
                                  int32_t partition_size, int32_t max_parts, int32_t* items_out,
                                  int32_t capacity, int32_t* n_out) {
  pa::clear_error();
  if (!n_out || num_seqs < 0 || partition_size <= 0 || capacity < 0 ||
      (num_seqs > 0 && !context_lens) || (capacity > 0 && !items_out))
    return invalid("pa_partition_work_items: bad argument");
  // The decode's work-list grid runs item i on XCD i % 8 (workgroups go to
  // the XCDs round-robin by id; the KV heads of an item share its XCD).  The
  // partitions are dealt to one queue per XCD in runs of consecutive
  // partitions of one sequence, longest run first, each to the queue holding
  // the fewest tokens so far.  Runs are whole sequences (up to an eighth of
  // all partitions) when that balances the queues to within 1 %; otherwise
  // the run length halves until it does (down to single partitions, where
  // the dealing is as even as partitions allow).  A sequence's partitions
  // thus share one XCD's L2 (its query rows and block-table row) and write
  // one contiguous range of partials there.  Each queue lists its full
  // partitions, then its ragged last partitions longest first, so the
  // shortest work ends the launch.  The queues interleave (queue x at
  // positions 8j + x) while every queue has items left; the rest follow in
  // the same round-robin order, no longer pinned.
  constexpr int kQueues = 8;
  struct Item {
    int32_t seq, part, ntok;
  };
  struct Run {
    int64_t tokens;
    int32_t seq, p0, p1;
  };
  std::vector<int32_t> nparts(static_cast<size_t>(num_seqs), 0);
  int64_t n = 0, total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t L = context_lens[i];
    if (L <= 0) continue;
    int64_t np = (L + partition_size - 1) / partition_size;
    if (max_parts >= 0 && np > max_parts) np = max_parts;
    nparts[static_cast<size_t>(i)] = static_cast<int32_t>(np);
    n += np;
    total += std::min<int64_t>(L, np * partition_size);
  }
  if (n > INT32_MAX) return invalid("pa_partition_work_items: too many items");
  std::vector<Run> runs;
  std::vector<int> queue_of;
  auto deal = [&](int64_t quota) {   // runs of at most `quota` partitions -> queues; max load
    runs.clear();
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int64_t L = context_lens[i];
      for (int64_t p0 = 0; p0 < nparts[static_cast<size_t>(i)]; p0 += quota) {
        const int64_t p1 = std::min<int64_t>(nparts[static_cast<size_t>(i)], p0 + quota);
        runs.push_back({std::min<int64_t>(L, p1 * partition_size) - p0 * partition_size, i,
                        static_cast<int32_t>(p0), static_cast<int32_t>(p1)});
      }
    }
    // longest first; ties keep sequence order
    std::stable_sort(runs.begin(), runs.end(),
                     [](const Run& x, const Run& y) { return x.tokens > y.tokens; });
    queue_of.assign(runs.size(), 0);
    int64_t load[kQueues] = {};
    for (size_t r = 0; r < runs.size(); ++r) {
      int x = 0;
      for (int k = 1; k < kQueues; ++k)
        if (load[k] < load[x]) x = k;
      load[x] += runs[r].tokens;
      queue_of[r] = x;
    }
    return *std::max_element(load, load + kQueues);
  };
  // the longest runs that balance to within 1 %, else the best balance seen
  // (the longer runs on a tie)
  int64_t best_quota = 1, best_max = INT64_MAX;
  for (int64_t quota = std::max<int64_t>(1, (n + kQueues - 1) / kQueues);; quota /= 2) {
    const int64_t mx = deal(quota);
    if (mx < best_max) {
      best_max = mx;
      best_quota = quota;
    }
    if (static_cast<double>(mx) * kQueues <= 1.01 * static_cast<double>(total) || quota == 1)
      break;
  }
  deal(best_quota);
  std::vector<Item> full[kQueues], ragged[kQueues];
  for (size_t r = 0; r < runs.size(); ++r) {
    const Run& run = runs[r];
    const int x = queue_of[r];
    const int64_t L = context_lens[run.seq];
    for (int32_t p = run.p0; p < run.p1; ++p) {
      const int32_t ntok =
          static_cast<int32_t>(std::min<int64_t>(partition_size, L - int64_t{p} * partition_size));
      (ntok == partition_size ? full[x] : ragged[x]).push_back({run.seq, p, ntok});
    }
  }
  size_t longest = 0;
  for (int x = 0; x < kQueues; ++x) {
    std::stable_sort(ragged[x].begin(), ragged[x].end(),
                     [](const Item& a, const Item& b) { return a.ntok > b.ntok; });
    full[x].insert(full[x].end(), ragged[x].begin(), ragged[x].end());
    longest = std::max(longest, full[x].size());
  }
  int64_t k = 0;
  auto emit = [&](const Item& it) {
    if (k < capacity) {
      items_out[2 * k] = it.seq;
      items_out[2 * k + 1] = it.part;
    }
    ++k;
  };
  for (size_t j = 0; j < longest; ++j)   // once a queue runs out, the rest shift
    for (int x = 0; x < kQueues; ++x)
      if (j < full[x].size()) emit(full[x][j]);
  *n_out = static_cast<int32_t>(n);
  if (n > capacity) return invalid("pa_partition_work_items: output too small");
  return PA_OK;
}

}  // extern "C"
