"""A prefix-caching scenario replayed step by step on libpa's allocator and on
the reference model of the block manager with prefix caching.

Prompts (block size bs; SYS is a 4-block system prompt):
  seq 0  A = SYS + 2 full blocks + 8 tokens
  seq 1  B = SYS + bs + 4 tokens              hits SYS (4 blocks in use)
  seq 2  C = 3 blocks + 2 tokens, its own     no hit
  free A                                      A's two full tail blocks wait in the pool, cached
  seq 3  D = SYS + A's two tail blocks + bs + 9 tokens
                                              hits SYS and takes A's two blocks back out of the pool
  free C                                      C's blocks wait in the pool, cached (deepest first)
  seq 4  E = unique tokens, all but one free block
                                              hands out C's blocks 2 and 1: evicted
  free E
  seq 5  F = C again                          hits C's block 0 only (block 1 was evicted)
  seq 6  G = SYS + 5 tokens                   hits SYS (third sharer)
Live at the end: B, D, F, G.  After every operation the cached length and the
tables of both allocators must agree ("LLM推理优化：vLLM PagedAttention深度解析
与工程实践", §4.2 prefix reuse; the Qwen2.5-7B vLLM 0.6.3 deployment page,
§3.2: block-aligned, token-exact prefixes).
"""
import numpy as np

from workloads import prompt_tokens

LIVE = (1, 3, 5, 6)


def prompts(seed, bs):
    cat = lambda *a: np.concatenate(a).astype(np.int32)
    sys_ = prompt_tokens(seed, 0, 4 * bs)
    tail_a = prompt_tokens(seed, 1, 2 * bs + 8)
    c = prompt_tokens(seed, 3, 3 * bs + 2)
    return {
        0: cat(sys_, tail_a),
        1: cat(sys_, prompt_tokens(seed, 2, bs + 4)),
        2: c,
        3: cat(sys_, tail_a[: 2 * bs], prompt_tokens(seed, 4, bs + 9)),
        5: c.copy(),
        6: cat(sys_, prompt_tokens(seed, 6, 5)),
    }


def run(alloc, model, seed, bs, on_prompt=None):
    """Replays the scenario on libpa's allocator `alloc` and the model `model`
    (both with prefix caching on, same pool and initial order).  on_prompt(seq,
    tokens, cached) runs after each allocation, to write the uncached tail.
    Returns (live prompts {seq: tokens}, facts about the run)."""
    P = prompts(seed, bs)
    facts = {}

    def allocate(seq, tokens):
        c1 = alloc.allocate_prompt(seq, tokens)
        c2 = model.allocate_prompt(seq, tokens)
        assert c1 == c2, f"seq {seq}: cached {c1} (library) vs {c2} (model)"
        assert np.array_equal(alloc.block_table(seq), model.block_table(seq)), f"seq {seq}: table"
        assert alloc.num_free() == model.num_free(), f"seq {seq}: free count"
        if on_prompt is not None:
            on_prompt(seq, tokens, c1)
        return c1

    def free(seq):
        alloc.free(seq)
        model.free(seq)
        assert np.array_equal(alloc.free_list(), np.array(model.free_blocks, np.int32))

    facts["A"] = allocate(0, P[0])
    facts["B"] = allocate(1, P[1])
    facts["C"] = allocate(2, P[2])
    a_tail = list(model.block_table(0))[4:6]    # A's two full blocks past SYS
    free(0)
    # both wait in the pool with no reference and their cache entries
    assert all(model.refcount[b] == 0 and b in model.free_blocks and b in model.block_key
               for b in a_tail)
    facts["D"] = allocate(3, P[3])
    facts["hits_taken_from_pool"] = sum(1 for b in model.block_table(3)[: facts["D"] // bs]
                                        if b in a_tail)
    c_table = list(model.block_table(2))
    free(2)
    facts["E"] = allocate(4, prompt_tokens(seed, 5, (model.num_free() - 1) * bs))
    # E took every free block but the last, C's first: C's blocks 1 and 2 left the cache
    facts["evicted"] = sum(1 for b in c_table[1:3] if b not in model.block_key or
                           model.block_key[b] != tuple(P[2][: (c_table.index(b) + 1) * bs]))
    free(4)
    facts["F"] = allocate(5, P[5])
    facts["G"] = allocate(6, P[6])
    return {s: P[s] for s in LIVE}, facts


def expected_facts(bs):
    """What the scenario must show: reuse of blocks in use, reuse of blocks
    taken back out of the pool, and a prefix cut short by eviction."""
    return {"A": 0, "B": 4 * bs, "C": 0, "D": 6 * bs, "hits_taken_from_pool": 2, "E": 0,
            "evicted": 2, "F": bs, "G": 4 * bs}
