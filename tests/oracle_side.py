"""Builds the oracle's own copy of a workload's state: the allocator model
replays the workload's operations, the oracle's cache write fills NaN-poisoned
pools.  Used by the oracle pin tests and by the GPU parity tests (as the
expected side).  Nothing here touches the HIP library."""
from dataclasses import dataclass

import numpy as np

import oracle
from oracle.allocator_model import BlockManagerModel
from workloads import POISON, Workload


@dataclass
class OracleState:
    model: BlockManagerModel
    key_cache: np.ndarray
    value_cache: np.ndarray
    block_tables: np.ndarray      # int32 [S][MB]
    context_lens: np.ndarray      # int32 [S]
    new_slots: np.ndarray         # int64 [S]
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray


def replay(w: Workload) -> tuple:
    model = BlockManagerModel(w.num_blocks, w.bs, w.initial_free_order)
    new_slots = np.full(w.S, -1, np.int64)
    for op in w.alloc_ops:
        if op[0] == "allocate":
            model.allocate(op[1], op[2])
        elif op[0] == "share_prefix":
            model.share_prefix(op[1], op[2], op[3])
        elif op[0] == "append_slot":
            slot, cow = model.append_slot(op[1])
            assert cow is None
            new_slots[op[1]] = slot
        else:
            raise ValueError(op)
    return model, new_slots


def tables_of(model: BlockManagerModel, S: int, mb: int) -> np.ndarray:
    bt = np.zeros((S, mb), np.int32)
    for i in range(S):
        t = model.block_table(i)
        bt[i, : len(t)] = t
    return bt


def build(w: Workload, poison: bool = True, write_new: bool = True) -> OracleState:
    model, new_slots = replay(w)
    shape = (w.num_blocks, w.bs, w.Hkv, w.D)
    fill = POISON[w.dtype] if poison else 0
    kc = np.full(shape, fill, np.uint16)
    vc = np.full(shape, fill, np.uint16)
    if w.spec.prefix_seqs:
        P = w.spec.prefix_len
        slots = np.array(model.slots(0, 0, P), np.int64)
        oracle.cache_write(w.prefix_tokens("k"), w.prefix_tokens("v"), kc, vc, slots)
    for i in range(w.S):
        b, e = w.prefix_of(i), int(w.lengths[i]) - 1
        if e > b:
            slots = np.array(model.slots(i, b, e), np.int64)
            oracle.cache_write(w.private_history(i, "k"), w.private_history(i, "v"), kc, vc, slots)
    k_new, v_new = w.new_tokens("k"), w.new_tokens("v")
    if write_new:
        oracle.cache_write(k_new, v_new, kc, vc, new_slots)
    mb = w.max_blocks_per_seq()
    return OracleState(model=model, key_cache=kc, value_cache=vc,
                       block_tables=tables_of(model, w.S, mb),
                       context_lens=w.lengths.copy(), new_slots=new_slots,
                       q=w.query(), k_new=k_new, v_new=v_new)


@dataclass
class OracleInt8State:
    key_cache: np.ndarray         # int8 [NB][bs][Hkv][D]
    value_cache: np.ndarray
    key_scale: np.ndarray         # float32 [NB][Hkv][bs]
    value_scale: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    q: np.ndarray


def build_int8(w: Workload, poison: bool = True) -> OracleInt8State:
    """The workload's state over INT8 pools: the same replay and slots, every
    row quantised by the oracle's INT8 cache write; unused codes -128, unused
    scales NaN."""
    model, new_slots = replay(w)
    shape = (w.num_blocks, w.bs, w.Hkv, w.D)
    kc = np.full(shape, -128 if poison else 0, np.int8)
    vc = kc.copy()
    ks = np.full((w.num_blocks, w.Hkv, w.bs), np.nan if poison else 0.0, np.float32)
    vs = ks.copy()
    if w.spec.prefix_seqs:
        P = w.spec.prefix_len
        slots = np.array(model.slots(0, 0, P), np.int64)
        oracle.cache_write_int8(w.prefix_tokens("k"), w.prefix_tokens("v"), kc, vc, ks, vs, slots,
                                w.dtype)
    for i in range(w.S):
        b, e = w.prefix_of(i), int(w.lengths[i]) - 1
        if e > b:
            slots = np.array(model.slots(i, b, e), np.int64)
            oracle.cache_write_int8(w.private_history(i, "k"), w.private_history(i, "v"), kc, vc,
                                    ks, vs, slots, w.dtype)
    oracle.cache_write_int8(w.new_tokens("k"), w.new_tokens("v"), kc, vc, ks, vs, new_slots,
                            w.dtype)
    return OracleInt8State(key_cache=kc, value_cache=vc, key_scale=ks, value_scale=vs,
                           block_tables=tables_of(model, w.S, w.max_blocks_per_seq()),
                           context_lens=w.lengths.copy(), q=w.query())
