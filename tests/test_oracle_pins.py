"""Pins of the CPU oracle to things other than itself: library conversions,
brute-force fp64 contiguous attention, the pages' worked examples and closed
forms, and invariances that the paged layout must not break.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.allocator_model import BlockManagerModel
from workloads import POISON, to_bits, workload
from tests import oracle_side

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------
# references written independently of the oracle
# ---------------------------------------------------------------------------

def ref_widen64(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def brute_force(q_bits, K_bits, V_bits, scale, dtype):
    """Contiguous attention in fp64.  q [Hq][D]; K, V [L][Hkv][D] logical order."""
    q = ref_widen64(q_bits, dtype)
    K = ref_widen64(K_bits, dtype)
    V = ref_widen64(V_bits, dtype)
    Hq, D = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, D))
    for h in range(Hq):
        g = h // G
        s = scale * (K[:, g, :] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


def tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype, nb=None, perm=None):
    """Random tokens scattered over a poisoned pool by numpy indexing (not by
    the oracle's cache write), plus the matching tables."""
    nblk = [-(-L // bs) for L in lens]
    nb = nb or sum(nblk) + 3
    perm = rng.permutation(nb) if perm is None else perm
    kc = np.full((nb, bs, Hkv, D), POISON[dtype], np.uint16)
    vc = kc.copy()
    mb = max(nblk)
    bt = np.zeros((S, mb), np.int32)
    seqs_k, seqs_v = [], []
    nxt = 0
    for i, L in enumerate(lens):
        K = to_bits(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype)
        V = to_bits(rng.standard_normal((L, Hkv, D)).astype(np.float32), dtype)
        for j in range(nblk[i]):
            bt[i, j] = perm[nxt]
            nxt += 1
        for j in range(L):
            kc[bt[i, j // bs], j % bs] = K[j]
            vc[bt[i, j // bs], j % bs] = V[j]
        seqs_k.append(K)
        seqs_v.append(V)
    q = to_bits(rng.standard_normal((S, Hq, D)).astype(np.float32), dtype)
    return q, kc, vc, bt, np.array(lens, np.int32), seqs_k, seqs_v


# ---------------------------------------------------------------------------
# conversions (pinned to numpy's float16 and torch's bfloat16 casts)
# ---------------------------------------------------------------------------

def edge_floats():
    rng = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.0, 65519.996, 65520.0, 65536.0, 1e30, -1e30,
            6.1035156e-05, 5.9604645e-08, 2.9802322e-08, 2.9802326e-08, 1e-10,
            3.3895314e38, 3.4028235e38, 1.1754944e-38, 9.2e-41, 1.4e-45]
    mant = rng.integers(0, 1 << 23, 4000)
    expo = rng.integers(1, 255, 4000)
    sign = rng.integers(0, 2, 4000)
    bits = (sign.astype(np.uint32) << 31) | (expo.astype(np.uint32) << 23) | mant.astype(np.uint32)
    r = list(bits.view(np.float32))
    # exact ties for both targets: patterns with a one followed by zeros
    for e in range(100, 150):
        for tail in (0x1000, 0x3000, 0x8000, 0x18000):
            r.append(np.uint32((e << 23) | tail).view(np.float32))
    # subnormal float32 inputs
    r += list((rng.integers(1, 1 << 23, 200).astype(np.uint32)).view(np.float32))
    return np.array(vals + [float(x) for x in r], np.float32)


def test_f16_widen_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "f16")
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_widen_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_narrow_matches_numpy():
    x = edge_floats()
    x = np.concatenate([x, np.float32([np.nan, np.inf, -np.inf])])
    ours = oracle.narrow(x, "f16")
    ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all(ours[nan] & 0x3FF)


def test_bf16_narrow_matches_torch():
    x = edge_floats()
    x = np.concatenate([x, np.float32([np.nan, np.inf, -np.inf])])
    ours = oracle.narrow(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all(ours[nan] & 0x7F)


def test_scalar_conversions_agree_with_array_forms():
    for x in (0.1, -2.5, 65520.0, 1e-6, 3.0e38):
        assert oracle.f32_to_f16(x) == int(oracle.narrow(np.float32([x]), "f16")[0])
        assert oracle.f32_to_bf16(x) == int(oracle.narrow(np.float32([x]), "bf16")[0])
    assert oracle.f16_to_f32(0x3C00) == 1.0 and oracle.bf16_to_f32(0x3F80) == 1.0


# ---------------------------------------------------------------------------
# byte closed forms and the GQA ratio (golden, from the pages)
# ---------------------------------------------------------------------------

def test_kv_bytes_closed_forms(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes.json")))
    for row in g["per_token"]:
        assert oracle.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                         row["elem_bytes"]) == row["bytes"], row["cite"]
    for row in g["per_sequence"]:
        per_tok = oracle.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                            row["elem_bytes"])
        assert per_tok * row["tokens"] == row["bytes"], row["cite"]
    for row in g["per_batch"]:
        per_tok = oracle.kv_bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                            row["elem_bytes"])
        assert per_tok * row["tokens"] * row["batch"] == row["bytes"], row["cite"]
    for row in g["gqa_ratio"]:
        gqa = oracle.kv_bytes_per_token(1, row["kv_heads"], 128, 2)
        mha = oracle.kv_bytes_per_token(1, row["q_heads"], 128, 2)
        assert gqa / mha == row["ratio"], row["cite"]


def test_kv_bytes_gathered():
    lens = np.array([1, 15, 16, 37], np.int32)
    assert oracle.kv_bytes_gathered(lens, 4, 64, 2) == 69 * 2 * 4 * 64 * 2


# ---------------------------------------------------------------------------
# allocator model: the pages' worked examples and the invariants
# ---------------------------------------------------------------------------

def test_worked_block_tables(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "block_table_examples.json")))
    for ex in g["examples"]:
        nb = 128
        head = ex["free_order_head"]
        order = head + [b for b in range(nb) if b not in head]
        m = BlockManagerModel(nb, ex["block_size"], order)
        m.allocate("seq", ex["num_tokens"])
        assert m.block_table("seq") == ex["table"], ex["cite"]
        bs = ex["block_size"]
        fills = [min(bs, ex["num_tokens"] - k * bs) for k in range(len(ex["table"]))]
        assert fills == ex["fills"], ex["cite"]
        row = np.array(ex["table"], np.int32)
        for pos, slot in ex["slot_checks"]:
            assert m.slot("seq", pos) == slot
            assert oracle.slot(row, pos, bs) == slot


def test_fifo_and_ceil_growth():
    m = BlockManagerModel(8, 4, [5, 2, 7, 0, 1, 3, 6, 4])
    m.allocate("a", 5)                       # ceil(5/4) = 2 blocks
    assert m.block_table("a") == [5, 2]
    m.allocate("a", 8)                       # still covered
    assert m.block_table("a") == [5, 2]
    m.allocate("b", 1)
    assert m.block_table("b") == [7]
    m.free("a")                              # returned to the tail, in table order
    assert m.free_blocks == [0, 1, 3, 6, 4, 5, 2]
    m.allocate("c", 12)
    assert m.block_table("c") == [0, 1, 3]


def test_oom_leaves_state_unchanged():
    m = BlockManagerModel(4, 16, [3, 1, 0, 2])
    m.allocate("a", 40)
    snap = (list(m.free_blocks), {k: list(v) for k, v in m.tables.items()}, list(m.refcount))
    with pytest.raises(Exception):
        m.allocate("b", 17)                  # needs 2, only 1 free
    assert snap == (list(m.free_blocks), {k: list(v) for k, v in m.tables.items()},
                    list(m.refcount))
    m.allocate("b", 16)
    m.allocate("a", 48)                      # covered by the 3 blocks it holds
    with pytest.raises(Exception):
        m.append_slot("b")                   # b's block is full, pool empty
    assert m.num_tokens["b"] == 16


def test_append_slot_and_cow():
    m = BlockManagerModel(6, 4, [4, 0, 5, 1, 2, 3])
    m.allocate("a", 6)                       # [4, 0], 6 tokens
    assert m.append_slot("a") == (0 * 4 + 2, None)       # position 6
    m.fork("a", "b")                         # shares [4, 0] incl. partial block 0
    assert m.refcount[4] == 2 and m.refcount[0] == 2
    slot, cow = m.append_slot("b")           # position 7 lands in shared block 0
    assert cow == (0, 5) and slot == 5 * 4 + 3
    assert m.block_table("b") == [4, 5] and m.block_table("a") == [4, 0]
    assert m.refcount[0] == 1 and m.refcount[5] == 1 and m.refcount[4] == 2
    m.free("a")
    assert m.free_blocks == [1, 2, 3, 0]     # block 4 still held by b
    m.free("b")
    assert m.free_blocks == [1, 2, 3, 0, 4, 5]


def test_model_invariants_random_ops():
    rng = np.random.default_rng(11)
    nb, bs = 48, 8
    m = BlockManagerModel(nb, bs, rng.permutation(nb))
    live = []
    for step in range(3000):
        r = rng.random()
        try:
            if r < 0.3 or not live:
                sid = step
                m.allocate(sid, int(rng.integers(0, 40)))
                live.append(sid)
            elif r < 0.65:
                m.append_slot(live[rng.integers(len(live))])
            elif r < 0.75:
                src = live[rng.integers(len(live))]
                n = (m.num_tokens[src] // bs) * bs
                if n:
                    m.share_prefix(src, step, n)
                    live.append(step)
            elif r < 0.82:
                m.fork(live[rng.integers(len(live))], step)
                live.append(step)
            else:
                m.free(live.pop(rng.integers(len(live))))
        except Exception as e:
            assert "free blocks" in str(e)
        held = [b for t in m.tables.values() for b in t]
        assert len(m.free_blocks) + len(set(held)) == nb               # conservation
        assert len(set(m.free_blocks)) == len(m.free_blocks)
        for b in range(nb):
            assert m.refcount[b] == held.count(b)                       # refcount
            assert (m.refcount[b] == 0) == (b in m.free_blocks)
        for sid, t in m.tables.items():
            waste = len(t) * bs - m.num_tokens[sid]
            assert 0 <= waste < bs or (m.num_tokens[sid] == 0 and not t)  # < one block


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_cache_write_scatter_readback(dtype):
    rng = np.random.default_rng(3)
    nb, bs, hkv, d, n = 20, 16, 3, 8, 57
    kc = np.full((nb, bs, hkv, d), POISON[dtype], np.uint16)
    vc = kc.copy()
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    slots[5] = -1                                                      # padding token
    k = rng.integers(0, 65536, (n, hkv, d)).astype(np.uint16)
    v = rng.integers(0, 65536, (n, hkv, d)).astype(np.uint16)
    oracle.cache_write(k, v, kc, vc, slots)
    touched = np.zeros((nb, bs), bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc[s // bs, s % bs], k[t]) and np.array_equal(vc[s // bs, s % bs], v[t])
        touched[s // bs, s % bs] = True
    assert np.all(kc[~touched] == POISON[dtype]) and np.all(vc[~touched] == POISON[dtype])


def test_cache_write_rejects_bad_slots():
    kc = np.zeros((4, 16, 1, 8), np.uint16)
    vc = kc.copy()
    k = np.ones((2, 1, 8), np.uint16)
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.cache_write(k, k, kc, vc, np.array([3, 3], np.int64))
    with pytest.raises(oracle.OracleError, match="range"):
        oracle.cache_write(k, k, kc, vc, np.array([3, 64], np.int64))
    assert not kc.any()


# ---------------------------------------------------------------------------
# decode vs brute-force contiguous attention in fp64
# ---------------------------------------------------------------------------

CASES = [
    # S, Hq, Hkv, D, bs, lens, dtype
    (3, 4, 4, 4, 16, [1, 17, 40], "f16"),        # MHA, G = 1
    (2, 8, 2, 64, 16, [33, 64], "bf16"),         # G = 4
    (2, 7, 1, 64, 16, [50, 5], "bf16"),          # MQA, G = 7
    (4, 14, 2, 64, 32, [1, 31, 32, 63], "f16"),  # G = 7, bs 32
    (2, 4, 2, 4, 16, [64, 3], "bf16"),           # G = 2
]


@pytest.mark.parametrize("case", CASES)
def test_decode_matches_fp64_brute_force(case):
    S, Hq, Hkv, D, bs, lens, dtype = case
    rng = np.random.default_rng(hash(str(case)) % (1 << 32))
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype)
    scale = 1.0 / math.sqrt(D)
    out32, outT = oracle.decode(q, kc, vc, bt, cl, scale, dtype)
    for i in range(S):
        ref = brute_force(q[i], Ks[i], Vs[i], np.float32(scale), dtype)
        err = np.abs(out32[i] - ref).max()
        assert err <= 1e-5 * max(1.0, np.abs(ref).max()), (i, err)
        # the 16-bit output is the fp32 result rounded to nearest even
        assert np.array_equal(outT[i], oracle.narrow(out32[i], dtype))


def test_decode_uses_contiguous_head_groups():
    """q head h reads kv head h // G: swapping two kv heads' contents must move
    exactly the outputs of their query-head groups."""
    rng = np.random.default_rng(5)
    S, Hq, Hkv, D, bs = 1, 6, 3, 16, 16
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, S, Hq, Hkv, D, bs, [20], "bf16")
    a, _ = oracle.decode(q, kc, vc, bt, cl, 0.25, "bf16")
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, [0, 1]] = kc[:, :, [1, 0]]
    vc2[:, :, [0, 1]] = vc[:, :, [1, 0]]
    q2 = q.copy()
    q2[:, [0, 1, 2, 3]] = q[:, [2, 3, 0, 1]]
    b, _ = oracle.decode(q2, kc2, vc2, bt, cl, 0.25, "bf16")
    assert np.array_equal(b[:, [2, 3, 0, 1, 4, 5]], a)


def test_decode_special_cases():
    rng = np.random.default_rng(9)
    # L = 1: the only weight is 1, output is v itself, exactly
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 2, 4, 2, 64, 16, [1, 1], "bf16")
    _, outT = oracle.decode(q, kc, vc, bt, cl, 0.125, "bf16")
    for i in range(2):
        for h in range(4):
            assert np.array_equal(outT[i, h], Vs[i][0, h // 2])
    # all keys equal: uniform weights, output is the mean of V
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 1, 2, 1, 64, 16, [45], "f16")
    for j in range(45):
        kc[bt[0, j // 16], j % 16] = kc[bt[0, 0], 0]
    out32, _ = oracle.decode(q, kc, vc, bt, cl, 0.125, "f16")
    mean = ref_widen64(Vs[0][:, 0], "f16").mean(axis=0)
    assert np.abs(out32[0] - mean).max() < 1e-5


def test_decode_ignores_poison_beyond_length():
    """Unused tail slots hold NaN; they must not reach the result."""
    rng = np.random.default_rng(2)
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 2, 4, 4, 64, 16, [17, 30], "f16")
    out32, _ = oracle.decode(q, kc, vc, bt, cl, 0.125, "f16")
    assert np.isfinite(out32).all()


def test_physical_permutation_invariance():
    """Moving blocks to other physical ids (tables updated) changes nothing, bit for bit."""
    rng = np.random.default_rng(4)
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 3, 8, 2, 64, 16, [40, 7, 33], "bf16")
    a32, aT = oracle.decode(q, kc, vc, bt, cl, 0.125, "bf16")
    nb = kc.shape[0]
    perm = rng.permutation(nb)                 # block b moves to perm[b]
    kc2 = np.empty_like(kc); vc2 = np.empty_like(vc)
    kc2[perm] = kc; vc2[perm] = vc
    bt2 = perm[bt].astype(np.int32)
    b32, bT = oracle.decode(q, kc2, vc2, bt2, cl, 0.125, "bf16")
    assert np.array_equal(a32.view(np.uint32), b32.view(np.uint32))
    assert np.array_equal(aT, bT)


def test_block_size_invariance():
    """The same tokens laid out with bs 16 and bs 32 give identical results."""
    rng = np.random.default_rng(6)
    lens = [50, 1, 33]
    q, kc16, vc16, bt16, cl, Ks, Vs = tiny_case(rng, 3, 4, 2, 64, 16, lens, "f16")
    nb32 = sum(-(-L // 32) for L in lens) + 2
    kc32 = np.full((nb32, 32, 2, 64), POISON["f16"], np.uint16); vc32 = kc32.copy()
    bt32 = np.zeros((3, 2), np.int32)
    ids = rng.permutation(nb32)
    n = 0
    for i, L in enumerate(lens):
        for j in range(-(-L // 32)):
            bt32[i, j] = ids[n]; n += 1
        for j in range(L):
            kc32[bt32[i, j // 32], j % 32] = Ks[i][j]
            vc32[bt32[i, j // 32], j % 32] = Vs[i][j]
    a32, _ = oracle.decode(q, kc16, vc16, bt16, cl, 0.125, "f16")
    b32, _ = oracle.decode(q, kc32, vc32, bt32, cl, 0.125, "f16")
    assert np.array_equal(a32.view(np.uint32), b32.view(np.uint32))


@pytest.mark.parametrize("P", [16, 32, 48, 512])
def test_partitioned_form_equals_single_pass(P):
    rng = np.random.default_rng(8)
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 4, 8, 2, 64, 16, [1, 16, 95, 130], "bf16")
    a, _ = oracle.decode(q, kc, vc, bt, cl, 0.125, "bf16")
    b, _ = oracle.decode_partitioned(q, kc, vc, bt, cl, 0.125, "bf16", P)
    vmax = max(np.abs(ref_widen64(V, "bf16")).max() for V in Vs)
    assert np.abs(a - b).max() <= 1e-5 * vmax
    for i in range(4):
        ref = brute_force(q[i], Ks[i], Vs[i], np.float32(0.125), "bf16")
        assert np.abs(b[i] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


def test_decode_pairs_matches_full_and_threads():
    rng = np.random.default_rng(12)
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 3, 8, 4, 64, 16, [70, 9, 16], "f16")
    full, fullT = oracle.decode(q, kc, vc, bt, cl, 0.125, "f16", nthreads=1)
    pairs = np.array([[2, 7], [0, 0], [1, 3]], np.int32)
    sub, subT = oracle.decode_pairs(q, kc, vc, bt, cl, 0.125, "f16", pairs, nthreads=3)
    for n, (i, h) in enumerate(pairs):
        assert np.array_equal(sub[n], full[i, h]) and np.array_equal(subT[n], fullT[i, h])
    mt, _ = oracle.decode(q, kc, vc, bt, cl, 0.125, "f16", nthreads=4)
    assert np.array_equal(mt, full)


def test_decode_rejects_bad_metadata():
    rng = np.random.default_rng(1)
    q, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 2, 4, 4, 64, 16, [5, 9], "f16")
    cl0 = cl.copy(); cl0[1] = 0
    with pytest.raises(oracle.OracleError, match="length"):
        oracle.decode(q, kc, vc, bt, cl0, 0.125, "f16")
    bt2 = bt.copy(); bt2[0, 0] = kc.shape[0]
    with pytest.raises(oracle.OracleError, match="block"):
        oracle.decode(q, kc, vc, bt2, cl, 0.125, "f16")


# ---------------------------------------------------------------------------
# workload replay on the oracle side: paged result = contiguous brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_small_paged_equals_contiguous(cfg):
    w = workload(cfg, "small")
    st = oracle_side.build(w)
    n_shared = w.spec.prefix_seqs
    for i in range(w.S):
        # every token of sequence i sits at the slot the model reports
        for j in (0, int(w.lengths[i]) - 1):
            s = st.model.slot(i, j)
            assert s == oracle.slot(st.block_tables[i], j, w.bs)
        if i < n_shared:
            P = w.spec.prefix_len // w.bs
            assert np.array_equal(st.block_tables[i, :P], st.block_tables[0, :P])
    picks = list(range(min(w.S, 3)))
    pairs = np.array([[i, h] for i in picks for h in range(w.Hq)], np.int32)
    out32, _ = oracle.decode_pairs(st.q, st.key_cache, st.value_cache, st.block_tables,
                                   st.context_lens, w.scale, w.dtype, pairs)
    for i in picks:
        K = w.sequence_tokens(i, "k", st.k_new)
        V = w.sequence_tokens(i, "v", st.v_new)
        ref = brute_force(st.q[i], K, V, np.float32(w.scale), w.dtype)
        got = out32[[n for n, (a, _) in enumerate(pairs) if a == i]]
        assert np.abs(got - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


# ---------------------------------------------------------------------------
# INT8 KV cache: quantisation properties, scatter, decode vs fp64 brute force
# ---------------------------------------------------------------------------

def _rows(rng, n, d, dtype, mags=(1e-3, 1.0, 30.0, 4000.0)):
    x = np.concatenate([rng.standard_normal((n, d)) * m for m in mags]).astype(np.float32)
    return to_bits(x, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_int8_quantize_properties(dtype):
    """Round-to-nearest bound: with q = fl(x / s) = (x / s)(1 + d), |d| <= 2^-24
    and |x / s| <= 127, |x - s c| <= s (1/2 + 127 * 2^-24); the largest
    magnitude maps to +-127, s * 127 is the row's largest magnitude, and
    negation commutes."""
    rng = np.random.default_rng(21)
    bits = _rows(rng, 64, 128, dtype)
    x = ref_widen64(bits, dtype)
    codes, scales = oracle.quantize_rows(bits, dtype)
    s = scales.astype(np.float64)[:, None]
    amax = np.abs(x).max(axis=1)
    assert np.all(np.abs(x - s * codes) <= s * (0.5 + 128 * 2.0 ** -24))
    assert np.all(np.abs(s[:, 0] * 127 - amax) <= amax * 2 ** -23)
    top = np.abs(x).argmax(axis=1)
    assert np.array_equal(np.abs(codes[np.arange(len(x)), top]), np.full(len(x), 127))
    assert np.abs(codes).max() <= 127
    neg = bits ^ np.uint16(0x8000)
    c2, s2 = oracle.quantize_rows(neg, dtype)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_int8_quantize_exact_on_scaled_integers(dtype):
    """Rows of integers times 2^k whose largest magnitude is 127 * 2^k quantise
    losslessly: scale exactly 2^k, codes equal to the integers."""
    rng = np.random.default_rng(22)
    for k in range(-8, 9):
        ints = rng.integers(-127, 128, (16, 64))
        ints[:, 5] = 127 * rng.choice([-1, 1], 16)
        bits = to_bits((ints * 2.0 ** k).astype(np.float32), dtype)
        codes, scales = oracle.quantize_rows(bits, dtype)
        assert np.all(scales == np.float32(2.0 ** k))
        assert np.array_equal(codes, ints)


def test_int8_quantize_ties_to_even_zero_and_nonfinite():
    row = np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5], np.float32)
    codes, scales = oracle.quantize_rows(to_bits(row, "bf16")[None], "bf16")
    assert scales[0] == 1.0
    assert codes[0].tolist() == [127, 2, 4, -2, 0, 0, 2, -2]
    codes, scales = oracle.quantize_rows(np.zeros((1, 8), np.uint16), "bf16")
    assert scales[0] == 0.0 and not codes.any()
    inf_row = to_bits(np.array([1.0, np.inf, 2.0, 3.0], np.float32), "f16")[None]
    codes, scales = oracle.quantize_rows(inf_row, "f16")
    assert np.isnan(scales[0]) and not codes.any()


def test_int8_cache_write_scatter_readback():
    rng = np.random.default_rng(23)
    nb, bs, hkv, d, n, dtype = 12, 16, 3, 32, 41, "bf16"
    kc = np.full((nb, bs, hkv, d), -128, np.int8)
    vc = kc.copy()
    ks = np.full((nb, hkv, bs), np.nan, np.float32)
    vs = ks.copy()
    slots = rng.choice(nb * bs, n, replace=False).astype(np.int64)
    slots[3] = -1
    k = _rows(rng, n * hkv, d, dtype, (1.0,)).reshape(n, hkv, d)
    v = _rows(rng, n * hkv, d, dtype, (1.0,)).reshape(n, hkv, d)
    oracle.cache_write_int8(k, v, kc, vc, ks, vs, slots, dtype)
    kq, ksc = oracle.quantize_rows(k, dtype)
    vq, vsc = oracle.quantize_rows(v, dtype)
    touched = np.zeros((nb, bs), bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = s // bs, s % bs
        assert np.array_equal(kc[b, o], kq[t]) and np.array_equal(vc[b, o], vq[t])
        for g in range(hkv):              # scales are [block][kv head][offset]
            assert ks[b, g, o] == ksc[t, g] and vs[b, g, o] == vsc[t, g]
        touched[b, o] = True
    assert np.all(kc[~touched] == -128) and np.all(vc[~touched] == -128)
    assert np.isnan(ks.transpose(0, 2, 1)[~touched]).all()


def int8_tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype):
    """An INT8 pool filled by the oracle's own cache write; the test reads it
    back with its own index arithmetic for the brute force."""
    q, kc16, vc16, bt, cl, Ks, Vs = tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype)
    nb = kc16.shape[0]
    kc = np.full((nb, bs, Hkv, D), -128, np.int8)
    vc = kc.copy()
    ks = np.full((nb, Hkv, bs), np.nan, np.float32)
    vs = ks.copy()
    for i, L in enumerate(lens):
        slots = np.array([bt[i, j // bs] * bs + j % bs for j in range(L)], np.int64)
        oracle.cache_write_int8(Ks[i], Vs[i], kc, vc, ks, vs, slots, dtype)
    return q, kc, vc, ks, vs, bt, cl


def dequant64(codes, scales, bt_row, L, bs):
    """[L][Hkv][D] fp64 rows scale x code, read back from the pools."""
    return np.stack([codes[bt_row[j // bs], j % bs].astype(np.float64) *
                     scales[bt_row[j // bs], :, j % bs].astype(np.float64)[:, None]
                     for j in range(L)])


@pytest.mark.parametrize("case", CASES)
def test_int8_decode_matches_fp64_brute_force(case):
    S, Hq, Hkv, D, bs, lens, dtype = case
    rng = np.random.default_rng(hash(str(case)) % (1 << 31) + 5)
    q, kc, vc, ks, vs, bt, cl = int8_tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype)
    scale = 1.0 / math.sqrt(D)
    out32, outT = oracle.decode_int8(q, kc, vc, ks, vs, bt, cl, scale, dtype)
    G = Hq // Hkv
    for i in range(S):
        K = dequant64(kc, ks, bt[i], lens[i], bs)
        V = dequant64(vc, vs, bt[i], lens[i], bs)
        qq = ref_widen64(q[i], dtype)
        for h in range(Hq):
            s = np.float64(np.float32(scale)) * (K[:, h // G] @ qq[h])
            p = np.exp(s - s.max())
            ref = (p @ V[:, h // G]) / p.sum()
            assert np.abs(out32[i, h] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        assert np.array_equal(outT[i], oracle.narrow(out32[i], dtype))


def test_int8_lossless_rows_equal_16bit_decode():
    """Rows whose values are integers with largest magnitude 127 dequantise to
    themselves, so the INT8 decode equals the 16-bit decode bit for bit."""
    rng = np.random.default_rng(24)
    S, Hq, Hkv, D, bs, lens = 3, 8, 2, 64, 16, [20, 1, 47]
    q, kc16, vc16, bt, cl, _, _ = tiny_case(rng, S, Hq, Hkv, D, bs, lens, "bf16")
    nb = kc16.shape[0]
    kc = np.full((nb, bs, Hkv, D), -128, np.int8); vc = kc.copy()
    ks = np.full((nb, Hkv, bs), np.nan, np.float32); vs = ks.copy()
    for i, L in enumerate(lens):
        K = rng.integers(-127, 128, (L, Hkv, D)); K[:, :, 0] = 127
        V = rng.integers(-127, 128, (L, Hkv, D)); V[:, :, 3] = -127
        Kb, Vb = to_bits(K.astype(np.float32), "bf16"), to_bits(V.astype(np.float32), "bf16")
        slots = np.array([bt[i, j // bs] * bs + j % bs for j in range(L)], np.int64)
        oracle.cache_write(Kb, Vb, kc16, vc16, slots)
        oracle.cache_write_int8(Kb, Vb, kc, vc, ks, vs, slots, "bf16")
    a32, aT = oracle.decode(q, kc16, vc16, bt, cl, 0.01, "bf16")
    b32, bT = oracle.decode_int8(q, kc, vc, ks, vs, bt, cl, 0.01, "bf16")
    assert np.array_equal(a32.view(np.uint32), b32.view(np.uint32)) and np.array_equal(aT, bT)


def test_int8_decode_pairs_and_poison():
    rng = np.random.default_rng(25)
    q, kc, vc, ks, vs, bt, cl = int8_tiny_case(rng, 3, 8, 2, 64, 16, [17, 5, 33], "f16")
    full, fullT = oracle.decode_int8(q, kc, vc, ks, vs, bt, cl, 0.125, "f16")
    assert np.isfinite(full).all()                      # NaN scales of unused slots stay out
    pairs = np.array([[2, 7], [0, 1]], np.int32)
    sub, subT = oracle.decode_int8(q, kc, vc, ks, vs, bt, cl, 0.125, "f16", pairs=pairs,
                                   nthreads=2)
    for n, (i, h) in enumerate(pairs):
        assert np.array_equal(sub[n], full[i, h]) and np.array_equal(subT[n], fullT[i, h])


# ---------------------------------------------------------------------------
# multi-token (chunked-prefill) attention
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # Hq, Hkv, D, bs, lens, chunk sizes, dtype
    (4, 4, 8, 16, [1, 17, 40], [1, 5, 40], "f16"),          # MHA; a whole 40-token prompt
    (8, 2, 64, 16, [33, 64, 20], [33, 16, 1], "bf16"),      # G = 4; first chunk of a prompt
    (7, 1, 64, 32, [50, 9], [17, 9], "bf16"),              # MQA, G = 7, bs 32
]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_prefill_matches_fp64_causal_brute_force(case):
    Hq, Hkv, D, bs, lens, chunks, dtype = case
    rng = np.random.default_rng(hash(str(case)) % (1 << 31) + 11)
    S = len(lens)
    _, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, S, Hq, Hkv, D, bs, lens, dtype)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = to_bits(rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float32), dtype)
    scale = 1.0 / math.sqrt(D)
    out32, outT = oracle.prefill(q, kc, vc, bt, cl, qs, scale, dtype, nthreads=2)
    G = Hq // Hkv
    for i in range(S):
        K, V = ref_widen64(Ks[i], dtype), ref_widen64(Vs[i], dtype)
        for k in range(chunks[i]):
            pos = lens[i] - chunks[i] + k
            row = qs[i] + k
            qq = ref_widen64(q[row], dtype)
            for h in range(Hq):
                sc = np.float64(np.float32(scale)) * (K[: pos + 1, h // G] @ qq[h])
                p = np.exp(sc - sc.max())
                ref = (p @ V[: pos + 1, h // G]) / p.sum()
                assert np.abs(out32[row, h] - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max()), \
                    (i, k, h)
    assert np.array_equal(outT, oracle.narrow(out32, dtype))


def test_prefill_first_row_and_single_token_chunks():
    """A whole prompt's first row sees only key 0 (its output is V[0]
    exactly); chunks of one token are decode steps, bit for bit."""
    rng = np.random.default_rng(13)
    lens = [30, 7, 16]
    qd, kc, vc, bt, cl, Ks, Vs = tiny_case(rng, 3, 4, 2, 64, 16, lens, "bf16")
    qs = np.array([0, 30, 31, 32], np.int32)          # whole first prompt, then 1-token chunks
    q = np.concatenate([to_bits(rng.standard_normal((30, 4, 64)).astype(np.float32), "bf16"),
                        qd[1:]])
    out32, outT = oracle.prefill(q, kc, vc, bt, cl, qs, 0.125, "bf16")
    for h in range(4):
        assert np.array_equal(outT[0, h], Vs[0][0, h // 2])
    dec32, _ = oracle.decode(qd, kc, vc, bt, cl, 0.125, "bf16")
    assert np.array_equal(out32[30:32].view(np.uint32), dec32[1:3].view(np.uint32))


def test_prefill_rejects_bad_chunks():
    rng = np.random.default_rng(14)
    qd, kc, vc, bt, cl, _, _ = tiny_case(rng, 2, 4, 2, 64, 16, [5, 9], "f16")
    q = np.zeros((12, 4, 64), np.uint16)
    with pytest.raises(oracle.OracleError):                # a chunk longer than its sequence
        oracle.prefill(q, kc, vc, bt, cl, np.array([0, 6, 12], np.int32), 0.125, "f16")
