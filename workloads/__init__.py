"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the method's arithmetic: it draws context lengths, the initial
order of the free block list, and N(0,1) query/key/value samples rounded to
16-bit floats, and it lists the allocator operations that build the block
tables.  Each side (the HIP library and the oracle) replays those operations
with its own allocator, computes its own slots and writes its own pools.

Generator: ``numpy.random.default_rng([seed, stream, index])`` with one
stream per quantity, so any sequence's values can be regenerated alone.

Workloads (the ``full`` variants are the benchmark shapes; the ``small``
variants keep the head/dim/block structure with fewer and shorter sequences):

1. tiny: 4 seqs, lens {1,15,16,37}, 4 q = 4 kv heads, D 64, bs 16, 64 blocks,
   fp16.
2. LLaMA-13B-shaped MHA layer: 32 seqs, 40 heads, D 128, fp16, bs 16,
   lens ~ U{128..2048}, single-pass kernel.
3. Qwen2.5-7B-shaped GQA layer: 64 seqs, 28 q / 4 kv heads, D 128, bf16,
   bs 16, lens log-uniform in [256, 32768], partitioned (512) + merge.
4. 7B GQA long context: 16 seqs x 32768, 32 q / 8 kv heads, D 128, bf16,
   bs 16, partitioned (512) + merge.
5. continuous-batching step: 256 seqs, 32 q / 8 kv heads, D 128, bf16;
   the first 64 share a 1024-token prefix (the same physical blocks),
   tails ~ U{16..4096}; bs 16 or 32; partitioned (512) + merge.

Context lengths count every cached token including the new one, whose K/V
comes through the cache write at position L-1; positions before it are
history written straight into the pools.  Pools hold 1.25x the unique blocks
the lengths need (64 for the tiny case), and the initial free list is a
seeded permutation of all block ids, so tables are scattered.
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np

STREAM_LEN = 1
STREAM_PERM = 2
STREAM_Q = 3
STREAM_K = 4
STREAM_V = 5
STREAM_K_NEW = 6
STREAM_V_NEW = 7
STREAM_K_PREFIX = 8
STREAM_V_PREFIX = 9

POISON = {"f16": 0x7E00, "bf16": 0x7FC0}   # quiet NaN patterns for unused slots


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 samples -> 16-bit patterns, rounded to nearest even.

    Input preparation only (the samples are finite)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


@dataclass(frozen=True)
class Spec:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                    # "f16" | "bf16"
    kernel: str                   # "single" | "partitioned"
    partition_size: int = 512
    lengths: str = "fixed"        # fixed | uniform | loguniform | prefix_tails
    len_lo: int = 0
    len_hi: int = 0
    fixed_lengths: tuple = ()
    prefix_len: int = 0           # shared prefix tokens
    prefix_seqs: int = 0          # sequences 0..prefix_seqs-1 share it
    num_blocks: int = 0           # 0 -> 1.25x the unique blocks needed
    pool_factor: float = 1.25
    seed: int = 0
    # Start every sequence this many tokens short of its drawn length (not
    # below 1, nor below the shared prefix + 1): a decode benchmark that
    # appends one token per step then spends its timed steps around the drawn
    # lengths.  The pool size and the block order follow the drawn lengths.
    length_shift: int = 0


SPECS = {
    1: Spec("tiny paged decode: 4 seqs, lens {1,15,16,37}, 4q=4kv heads, D64, bs16, fp16",
            4, 4, 4, 64, 16, "f16", "single", lengths="fixed",
            fixed_lengths=(1, 15, 16, 37), num_blocks=64, seed=1),
    2: Spec("LLaMA-13B-shaped MHA layer: 32 seqs, 40 heads, D128, fp16, bs16, lens U{128..2048}",
            32, 40, 40, 128, 16, "f16", "single", lengths="uniform", len_lo=128,
            len_hi=2048, seed=2),
    3: Spec("Qwen2.5-7B-shaped GQA layer: 64 seqs, 28q/4kv heads, D128, bf16, bs16, "
            "lens log-uniform 256..32768, partition 512",
            64, 28, 4, 128, 16, "bf16", "partitioned", lengths="loguniform", len_lo=256,
            len_hi=32768, seed=3),
    4: Spec("7B GQA long-context layer: 16 seqs x 32768, 32q/8kv heads, D128, bf16, bs16, "
            "partition 512",
            16, 32, 8, 128, 16, "bf16", "partitioned", lengths="fixed",
            fixed_lengths=(32768,) * 16, seed=4),
    5: Spec("continuous-batching step: 256 seqs, 32q/8kv heads, D128, bf16, 64 seqs share a "
            "1024-token prefix, tails U{16..4096}, partition 512",
            256, 32, 8, 128, 16, "bf16", "partitioned", lengths="prefix_tails", len_lo=16,
            len_hi=4096, prefix_len=1024, prefix_seqs=64, seed=5),
}

# Smaller variants with the same head / dim / block structure: several
# partitions and ragged tails, sized so the oracle finishes in seconds.
SMALL = {
    1: {},
    2: dict(num_seqs=4, len_lo=128, len_hi=700),
    3: dict(num_seqs=6, len_lo=256, len_hi=2100),
    4: dict(num_seqs=2, fixed_lengths=(2100, 1537)),
    5: dict(num_seqs=24, prefix_len=64, prefix_seqs=8, len_lo=16, len_hi=600),
}


def spec(cfg_id: int, variant: str = "full", **overrides) -> Spec:
    s = SPECS[cfg_id]
    if variant == "small":
        s = replace(s, **SMALL[cfg_id])
    elif variant != "full":
        raise ValueError(variant)
    if overrides:
        s = replace(s, **overrides)
    return s


def _rng(seed, stream, index=0):
    return np.random.default_rng([seed, stream, index])


@dataclass
class Workload:
    spec: Spec
    lengths: np.ndarray                     # int32 [S], including the new token
    num_blocks: int
    initial_free_order: np.ndarray          # int32 [num_blocks]
    alloc_ops: list = field(default_factory=list)

    # shape shortcuts
    @property
    def S(self): return self.spec.num_seqs
    @property
    def Hq(self): return self.spec.num_q_heads
    @property
    def Hkv(self): return self.spec.num_kv_heads
    @property
    def D(self): return self.spec.head_dim
    @property
    def bs(self): return self.spec.block_size
    @property
    def dtype(self): return self.spec.dtype
    @property
    def scale(self): return float(np.float32(1.0 / math.sqrt(self.spec.head_dim)))
    @property
    def elem_bytes(self): return 2

    def prefix_of(self, i: int) -> int:
        """Tokens of sequence i that live in the shared prefix blocks."""
        return self.spec.prefix_len if i < self.spec.prefix_seqs else 0

    def max_blocks_per_seq(self, extra_tokens: int = 0) -> int:
        return int(-(-(int(self.lengths.max()) + extra_tokens) // self.bs))

    # -- values ---------------------------------------------------------------
    def _normal(self, stream, index, shape):
        return to_bits(_rng(self.spec.seed, stream, index).standard_normal(shape, dtype=np.float32),
                       self.dtype)

    def query(self) -> np.ndarray:
        return self._normal(STREAM_Q, 0, (self.S, self.Hq, self.D))

    def new_tokens(self, which: str) -> np.ndarray:
        stream = STREAM_K_NEW if which == "k" else STREAM_V_NEW
        return self._normal(stream, 0, (self.S, self.Hkv, self.D))

    def prefix_tokens(self, which: str) -> np.ndarray:
        stream = STREAM_K_PREFIX if which == "k" else STREAM_V_PREFIX
        return self._normal(stream, 0, (self.spec.prefix_len, self.Hkv, self.D))

    def private_history(self, i: int, which: str) -> np.ndarray:
        """Tokens prefix_of(i) .. L_i-2 of sequence i: [n][Hkv][D]."""
        stream = STREAM_K if which == "k" else STREAM_V
        n = int(self.lengths[i]) - 1 - self.prefix_of(i)
        return self._normal(stream, i, (max(n, 0), self.Hkv, self.D))

    def sequence_tokens(self, i: int, which: str, new=None) -> np.ndarray:
        """All L_i tokens of sequence i in logical order: [L_i][Hkv][D]."""
        parts = []
        if self.prefix_of(i):
            parts.append(self.prefix_tokens(which))
        parts.append(self.private_history(i, which))
        nt = self.new_tokens(which) if new is None else new
        parts.append(nt[i:i + 1])
        return np.concatenate(parts, axis=0)

    def kv_bytes(self, unique: bool = True) -> int:
        """Algorithmic K+V bytes one decode call reads (shared prefix once if unique)."""
        per_tok = 2 * self.Hkv * self.D * self.elem_bytes
        toks = int(self.lengths.astype(np.int64).sum())
        if unique and self.spec.prefix_seqs > 1:
            toks -= (self.spec.prefix_seqs - 1) * self.spec.prefix_len
        return toks * per_tok


def _lengths(s: Spec) -> np.ndarray:
    r = _rng(s.seed, STREAM_LEN)
    if s.lengths == "fixed":
        L = np.array(s.fixed_lengths[: s.num_seqs], dtype=np.int64)
        if L.size != s.num_seqs:
            raise ValueError("fixed_lengths shorter than num_seqs")
    elif s.lengths == "uniform":
        L = r.integers(s.len_lo, s.len_hi + 1, s.num_seqs)
    elif s.lengths == "loguniform":
        L = np.round(np.exp(r.uniform(math.log(s.len_lo), math.log(s.len_hi), s.num_seqs)))
        L = np.clip(L, s.len_lo, s.len_hi)
    elif s.lengths == "prefix_tails":
        L = r.integers(s.len_lo, s.len_hi + 1, s.num_seqs)
        L[: s.prefix_seqs] += s.prefix_len
    else:
        raise ValueError(s.lengths)
    return L.astype(np.int32)


def make_workload(s: Spec) -> Workload:
    L = _lengths(s)
    bs = s.block_size
    if s.prefix_seqs:
        if s.prefix_len % bs:
            raise ValueError("shared prefix must be block-aligned")
        if np.any(L[: s.prefix_seqs] <= s.prefix_len):
            raise ValueError("sharing sequences must extend past the prefix")
    blocks = int(sum(-(-int(x) // bs) for x in L))
    if s.prefix_seqs > 1:
        blocks -= (s.prefix_seqs - 1) * (s.prefix_len // bs)
    nb = s.num_blocks or int(math.ceil(s.pool_factor * blocks))
    if nb < blocks:
        raise ValueError("pool smaller than the blocks the lengths need")
    perm = _rng(s.seed, STREAM_PERM).permutation(nb).astype(np.int32)
    if s.length_shift:
        floor = np.ones_like(L)
        floor[: s.prefix_seqs] = s.prefix_len + 1
        L = np.maximum(L - s.length_shift, floor).astype(np.int32)

    ops = []
    if s.prefix_seqs:
        ops.append(("allocate", 0, s.prefix_len))
        for i in range(1, s.prefix_seqs):
            ops.append(("share_prefix", 0, i, s.prefix_len))
    for i in range(s.num_seqs):
        ops.append(("allocate", i, int(L[i]) - 1))
    for i in range(s.num_seqs):
        ops.append(("append_slot", i))
    return Workload(spec=s, lengths=L, num_blocks=nb, initial_free_order=perm, alloc_ops=ops)


def workload(cfg_id: int, variant: str = "full", **overrides) -> Workload:
    return make_workload(spec(cfg_id, variant, **overrides))


# ---------------------------------------------------------------------------
# multi-token (chunked-prefill) attention inputs
# ---------------------------------------------------------------------------
# Each sequence holds L_i tokens in the cache, the last n_i of which are its
# query chunk (their K/V written with the rest).  Full variant: a
# Qwen2.5-7B-shaped layer (28 q / 4 kv heads, D 128, bf16, bs 16) with 8
# sequences, each running a 512-token prefill chunk after 0 .. 8192 tokens of
# earlier chunks; small variants keep the head structure at sizes the oracle
# finishes in seconds, with whole prompts, one-token chunks and ragged tails.

STREAM_PF_Q = 20
STREAM_PF_K = 21
STREAM_PF_V = 22


@dataclass(frozen=True)
class PrefillSpec:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    contexts: tuple               # L_i, tokens in the cache including the chunk
    chunks: tuple                 # n_i <= L_i
    seed: int = 40
    pool_factor: float = 1.25


PREFILL_SPECS = {
    "full": PrefillSpec(
        "Qwen2.5-7B-shaped chunked prefill: 8 seqs x 512-token chunks after 0..8192 cached "
        "tokens, 28q/4kv heads, D128, bf16, bs16",
        28, 4, 128, 16, "bf16",
        contexts=tuple(h + 512 for h in (0, 512, 1024, 2048, 3072, 4096, 6144, 8192)),
        chunks=(512,) * 8),
    "small": PrefillSpec(
        "small chunked prefill, 28q/4kv, D128, bf16, bs16", 28, 4, 128, 16, "bf16",
        contexts=(1, 17, 100, 530, 64, 33), chunks=(1, 17, 37, 512, 1, 32)),
}


@dataclass
class PrefillWorkload:
    spec: PrefillSpec
    lengths: np.ndarray           # int32 [S]
    chunks: np.ndarray            # int32 [S]
    query_start: np.ndarray       # int32 [S + 1]
    num_blocks: int
    initial_free_order: np.ndarray

    @property
    def S(self): return len(self.spec.contexts)
    @property
    def Hq(self): return self.spec.num_q_heads
    @property
    def Hkv(self): return self.spec.num_kv_heads
    @property
    def D(self): return self.spec.head_dim
    @property
    def bs(self): return self.spec.block_size
    @property
    def dtype(self): return self.spec.dtype
    @property
    def T(self): return int(self.query_start[-1])
    @property
    def scale(self): return float(np.float32(1.0 / math.sqrt(self.spec.head_dim)))

    def max_blocks_per_seq(self) -> int:
        return int(-(-int(self.lengths.max()) // self.bs))

    def tokens(self, i: int, which: str) -> np.ndarray:
        """All L_i cached tokens of sequence i (the chunk last): [L_i][Hkv][D]."""
        stream = STREAM_PF_K if which == "k" else STREAM_PF_V
        x = _rng(self.spec.seed, stream, i).standard_normal(
            (int(self.lengths[i]), self.Hkv, self.D), dtype=np.float32)
        return to_bits(x, self.dtype)

    def query(self) -> np.ndarray:
        x = _rng(self.spec.seed, STREAM_PF_Q).standard_normal((self.T, self.Hq, self.D),
                                                              dtype=np.float32)
        return to_bits(x, self.dtype)

    def flops(self) -> int:
        """Causal attention FLOPs: 4 D per (query row, head, visible key)."""
        keys = sum(int(n) * (int(L) - int(n)) + int(n) * (int(n) + 1) // 2
                   for L, n in zip(self.lengths, self.chunks))
        return 4 * self.D * self.Hq * keys

    def kv_bytes(self) -> int:
        """K+V bytes of the cached tokens the chunks read (each once)."""
        return int(self.lengths.astype(np.int64).sum()) * 2 * self.Hkv * self.D * 2


def prefill_workload(variant: str = "small", **overrides) -> PrefillWorkload:
    s = PREFILL_SPECS[variant]
    if overrides:
        s = replace(s, **overrides)
    L = np.array(s.contexts, np.int32)
    n = np.array(s.chunks, np.int32)
    if L.shape != n.shape or np.any(n < 0) or np.any(n > L):
        raise ValueError("chunks must satisfy 0 <= n_i <= L_i")
    blocks = int(sum(-(-int(x) // s.block_size) for x in L))
    nb = max(int(math.ceil(s.pool_factor * blocks)), 1)
    perm = _rng(s.seed, STREAM_PERM).permutation(nb).astype(np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return PrefillWorkload(spec=s, lengths=L, chunks=n, query_start=qs, num_blocks=nb,
                           initial_free_order=perm)


# -- prompts for the prefix cache -------------------------------------------------------
# A token's K/V depends on every token before it in a real model, so the rows
# drawn here for position j of a prompt come from a generator seeded by a
# digest of the prompt's tokens 0..j: two prompts get bit-identical rows
# exactly where they share a prefix, and different rows after the first token
# where they differ.  (Input preparation only; the digest is blake2b.)

STREAM_PC_K = 30
STREAM_PC_V = 31
STREAM_PC_Q = 32
STREAM_PC_TOKENS = 33


def prompt_tokens(seed: int, index: int, n: int, vocab: int = 32000) -> np.ndarray:
    """n seeded token ids in [0, vocab) (int32)."""
    return _rng(seed, STREAM_PC_TOKENS, index).integers(0, vocab, n).astype(np.int32)


def prefix_keyed_kv(seed: int, tokens, num_kv_heads: int, head_dim: int, dtype: str):
    """(keys, values), each [n][num_kv_heads][head_dim] 16-bit patterns, row j
    drawn from N(0,1) with a generator keyed by (seed, digest of tokens[:j+1])."""
    import hashlib
    toks = np.ascontiguousarray(tokens, dtype=np.int32).reshape(-1)
    n = toks.shape[0]
    k = np.empty((n, num_kv_heads, head_dim), np.float32)
    v = np.empty_like(k)
    h = hashlib.blake2b(digest_size=16)
    for j in range(n):
        h.update(toks[j:j + 1].tobytes())
        d = np.frombuffer(h.digest(), np.uint32)
        key = [seed] + [int(x) for x in d]
        k[j] = np.random.default_rng([STREAM_PC_K] + key).standard_normal(
            (num_kv_heads, head_dim), dtype=np.float32)
        v[j] = np.random.default_rng([STREAM_PC_V] + key).standard_normal(
            (num_kv_heads, head_dim), dtype=np.float32)
    return to_bits(k, dtype), to_bits(v, dtype)


def prompt_queries(seed: int, num_seqs: int, num_q_heads: int, head_dim: int,
                   dtype: str) -> np.ndarray:
    """[num_seqs][num_q_heads][head_dim] N(0,1) queries, 16-bit patterns."""
    x = _rng(seed, STREAM_PC_Q).standard_normal((num_seqs, num_q_heads, head_dim),
                                                dtype=np.float32)
    return to_bits(x, dtype)
