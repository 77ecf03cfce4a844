"""Pins of the prefix-caching reference model (oracle/allocator_model.py) to
things other than itself: the pages' printed example and stated behaviours,
closed forms, a brute-force search over earlier prompts, a hand-derived
eviction scenario, and invariants that any correct cache keeps (a reused
block holds the KV of exactly the same token prefix).  CPU only.

PA_ALLOC_MODEL_PATH, when set, loads the model from another file (the planted
mistakes of test_oracle_mutations.py)."""
import importlib.util
import json
import os

import numpy as np
import pytest

from oracle import allocator_model as _default


def _model_module():
    path = os.environ.get("PA_ALLOC_MODEL_PATH")
    if not path:
        return _default
    spec = importlib.util.spec_from_file_location("planted_allocator_model", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


M = _model_module()
Model = M.PrefixCachingBlockManagerModel


def chars(text):
    return [ord(c) for c in text]


# ---------------------------------------------------------------------------
# the pages
# ---------------------------------------------------------------------------

def test_prefix_page_example(golden_dir):
    """Two requests sharing a 9-character beginning ([A] §4.2)."""
    g = json.load(open(os.path.join(golden_dir, "prefix_cache_examples.json")))
    r1, r2 = (chars(t) for t in g["requests"])
    for bs, want in g["cached_tokens"].items():
        bs = int(bs)
        m = Model(64, bs)
        assert m.allocate_prompt("r1", r1) == 0
        assert m.allocate_prompt("r2", r2) == want, (bs, g["cite"])
        k = want // bs
        assert m.block_table("r2")[:k] == m.block_table("r1")[:k]
        assert not set(m.block_table("r2")[k:]) & set(m.block_table("r1"))
        for b in m.block_table("r1")[:k]:
            assert m.refcount[b] == 2


def _system_prompt(rng, n=1536):
    return [int(t) for t in rng.integers(1000, 150000, n)]


def test_prefix_fixed_system_prompt_hits():
    """A fixed system prompt at the front, the varying part at the end: every
    request after the first reuses the system prompt's full blocks (the
    deployment page, §3.2-3.3: ~1.5K-token system prompt)."""
    rng = np.random.default_rng(5)
    bs = 16
    for sys_len in (1536, 1530, 16, 15):
        system = _system_prompt(rng, sys_len)
        m = Model(4096, bs)
        for k in range(8):
            user = [int(t) for t in rng.integers(1000, 150000, int(rng.integers(1, 200)))]
            got = m.allocate_prompt(k, system + user)
            n = sys_len + len(user)
            want = 0 if k == 0 else min((sys_len // bs) * bs, ((n - 1) // bs) * bs)
            assert got == want, (sys_len, k)


def test_prefix_varying_front_loses_everything():
    """A request id or time stamp put before a fixed system prompt changes the
    first block, and with it every later block (the deployment page, §3.2)."""
    rng = np.random.default_rng(6)
    system = _system_prompt(rng)
    m = Model(4096, 16)
    for k in range(6):
        assert m.allocate_prompt(k, [k + 1] + system + [7, 8, 9]) == 0


def test_prefix_changed_message_order_loses_everything():
    """The same messages in another order share no block-aligned prefix (the
    deployment page, §3.2: message structure must stay stable)."""
    rng = np.random.default_rng(8)
    system = _system_prompt(rng, 320)
    user = _system_prompt(rng, 64)
    m = Model(256, 16)
    assert m.allocate_prompt(0, system + user) == 0
    assert m.allocate_prompt(1, user + system) == 0
    assert m.allocate_prompt(2, system + user) == 320 + 48   # the last block is never reused


def test_prefix_hit_is_block_aligned_and_token_exact():
    m = Model(64, 16)
    base = list(range(100, 148))                              # 48 tokens, 3 blocks
    m.allocate_prompt(0, base)
    assert m.allocate_prompt(1, base[:47] + [1, 2]) == 32      # a difference in block 2
    assert m.allocate_prompt(2, base[:15] + [0] + base[16:]) == 0   # a difference in block 0
    assert m.allocate_prompt(3, base[:20]) == 16               # 20 tokens: 1 full block reused
    assert m.allocate_prompt(4, base[:16]) == 0                # the only block holds the last token
    assert m.allocate_prompt(5, base[:17]) == 16
    assert m.allocate_prompt(6, base) == 32                    # aligned repeat: last block computed


def test_prefix_caching_off_reuses_nothing():
    m = Model(64, 4, prefix_caching=False)
    assert m.allocate_prompt(0, list(range(20))) == 0
    assert m.allocate_prompt(1, list(range(20))) == 0
    assert not set(m.block_table(0)) & set(m.block_table(1))
    m.set_prefix_caching(True)
    assert m.allocate_prompt(2, list(range(20))) == 0          # nothing was cached while off
    assert m.allocate_prompt(3, list(range(20))) == 16
    m.set_prefix_caching(False)
    assert m.allocate_prompt(4, list(range(20))) == 0


# ---------------------------------------------------------------------------
# a hand-derived scenario: eviction order, hits taken from the pool, OOM
# ---------------------------------------------------------------------------

def test_prefix_eviction_scenario():
    m = Model(8, 2)
    assert m.allocate_prompt("a", [1, 2, 3, 4, 5, 6, 7]) == 0
    assert m.block_table("a") == [0, 1, 2, 3]                 # (1,2) (1..4) (1..6) cached
    m.free("a")
    assert m.free_blocks == [4, 5, 6, 7, 3, 2, 1, 0]          # deepest block first
    m.allocate("x", 12)                                       # hands out 4 5 6 7 3 2
    assert m.block_table("x") == [4, 5, 6, 7, 3, 2] and m.free_blocks == [1, 0]
    with pytest.raises(M.OOM):                                # hits 0, 1 leave the pool too
        m.allocate_prompt("b", [1, 2, 3, 4, 5, 6, 9])
    assert m.free_blocks == [1, 0] and "b" not in m.tables
    m.free("x")
    assert m.free_blocks == [1, 0, 2, 3, 7, 6, 5, 4]
    assert m.allocate_prompt("b", [1, 2, 3, 4, 5, 6, 9]) == 4  # (1..6) was lost with block 2
    assert m.block_table("b") == [0, 1, 2, 3] and m.free_blocks == [7, 6, 5, 4]
    assert m.allocate_prompt("c", [1, 2, 3, 4, 5, 6, 9, 9, 9]) == 6
    assert m.block_table("c") == [0, 1, 2, 7, 6] and m.free_blocks == [5, 4]
    assert m.allocate_prompt("d", [1, 2, 3, 4]) == 2           # (1..4) exists, not re-registered
    assert m.block_table("d") == [0, 5] and m.free_blocks == [4]
    m.free("d")
    assert m.free_blocks == [4, 5]
    assert m.allocate_prompt("e", [1, 2, 3, 4, 5]) == 4
    assert m.block_table("e") == [0, 1, 4] and m.free_blocks == [5]
    assert [m.refcount[b] for b in range(8)] == [3, 3, 2, 1, 1, 0, 1, 1]


# ---------------------------------------------------------------------------
# brute force and invariants on random prompts
# ---------------------------------------------------------------------------

def _prompts(rng, count, bs):
    """Prompts that share prefixes: a few trunks, cut and extended at random."""
    trunks = [[int(t) for t in rng.integers(0, 3, 6 * bs)] for _ in range(3)]
    out = []
    for _ in range(count):
        t = trunks[int(rng.integers(len(trunks)))]
        cut = int(rng.integers(0, len(t) + 1))
        tail = [int(x) for x in rng.integers(0, 3, int(rng.integers(0, 3 * bs)))]
        p = t[:cut] + tail
        if rng.random() < 0.2 and p:
            p[int(rng.integers(len(p)))] ^= 1                   # a single changed token
        out.append(p)
    return out


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
def test_prefix_brute_force_without_eviction(bs):
    """Nothing is freed and the pool never runs dry: the reuse is the longest
    block-aligned prefix shared with any earlier prompt's full blocks, short
    of the block that holds the last token."""
    rng = np.random.default_rng(20 + bs)
    prompts = _prompts(rng, 120, bs)
    m = Model(sum(-(-len(p) // bs) for p in prompts) + 1, bs)
    for k, p in enumerate(prompts):
        best = 0
        for q in prompts[:k]:
            lcp = 0
            while lcp < min(len(p), len(q)) and p[lcp] == q[lcp]:
                lcp += 1
            best = max(best, min(lcp // bs, len(q) // bs))
        want = 0 if not p else min(best, (len(p) - 1) // bs) * bs
        assert m.allocate_prompt(k, p) == want, k


def test_prefix_random_ops_reuse_only_identical_prefixes():
    """Random allocate / append / fork / share / free / prompt operations on a
    small pool: every reused block holds the KV of exactly the same tokens,
    reference counts equal the tables' holds, and no block is lost."""
    rng = np.random.default_rng(31)
    for bs, nb in ((2, 24), (4, 40), (16, 30)):
        m = Model(nb, bs, rng.permutation(nb))
        content = {}           # block -> token tuple whose KV it holds (None: unknown)
        live, nid = [], 0
        prompts = _prompts(rng, 400, bs)
        hits_seen = 0
        for step in range(1500):
            r = rng.random()
            try:
                if r < 0.35 or not live:
                    p = prompts[int(rng.integers(len(prompts)))]
                    c = m.allocate_prompt(nid, p)
                    t = m.block_table(nid)
                    for i, b in enumerate(t):
                        end = min((i + 1) * bs, len(p))
                        if i < c // bs:
                            assert content.get(b) == tuple(p[:end]), (step, i)
                            hits_seen += 1
                        else:
                            content[b] = tuple(p[:end])
                    live.append(nid)
                    nid += 1
                elif r < 0.55:
                    sid = live[int(rng.integers(len(live)))]
                    pos = m.num_tokens[sid]
                    slot, cow = m.append_slot(sid)
                    content[slot // bs] = None                    # written with unknown tokens
                elif r < 0.6:
                    src = live[int(rng.integers(len(live)))]
                    m.fork(src, nid)
                    live.append(nid)
                    nid += 1
                elif r < 0.65:
                    src = live[int(rng.integers(len(live)))]
                    n = (m.num_tokens[src] // bs) * bs
                    if n:
                        m.share_prefix(src, nid, n)
                        live.append(nid)
                        nid += 1
                elif r < 0.7:
                    sid = live[int(rng.integers(len(live)))]
                    before = len(m.tables[sid])
                    m.allocate(sid, m.num_tokens[sid] + int(rng.integers(0, 3 * bs)))
                    for b in m.tables[sid][before:]:
                        content[b] = None
                else:
                    m.free(live.pop(int(rng.integers(len(live)))))
            except M.OOM:
                pass
            held = [b for t in m.tables.values() for b in t]
            assert len(m.free_blocks) + len(set(held)) == nb
            assert len(set(m.free_blocks)) == len(m.free_blocks)
            for b in range(nb):
                assert m.refcount[b] == held.count(b)
                assert (m.refcount[b] == 0) == (b in m.free_blocks)
            # prefix-closed: a cached prefix's shorter block-aligned prefixes are cached, so
            # the walk may stop at the first miss; a cached block's prefix is held wherever
            # the block is held
            for key, b in m.cached.items():
                assert len(key) % bs == 0 and m.block_key[b] == key
                if len(key) > bs:
                    parent = m.cached.get(key[:-bs])
                    assert parent is not None, (step, key)
                    for t in m.tables.values():
                        assert b not in t or parent in t[: t.index(b)]
        assert hits_seen > 50, bs
