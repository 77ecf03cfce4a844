"""The no-allocation split-context decode (pa_decode_partitioned_noalloc,
for callers that cannot allocate device memory) against pa_decode_partitioned
with a caller workspace: two calls in a row through the C ABI, the second on
a smaller input, outputs bit-identical to the existing entry point's (the
same kernels) and within the decode bars of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_106_amd as pa
from workloads import workload
from tests import gpu_side, oracle_side
from tests.test_gpu_parity import ORACLE_THREADS, check_outputs, free_gpu

pytestmark = pytest.mark.gpu


def _call_noalloc(g, w, P, items, out):
    """pa_decode_partitioned_noalloc through the C ABI (ctypes), on the
    current stream."""
    c, st = g.cache, g.step
    L = pa.lib()
    n = 0 if items is None else items.shape[0]
    rc = L.pa_decode_partitioned_noalloc(
        out.data_ptr(), g.q.data_ptr(), c.key_cache.data_ptr(), c.value_cache.data_ptr(),
        st.block_tables.data_ptr(), st.block_tables.shape[1], st.context_lens.data_ptr(), w.S,
        w.Hq, w.Hkv, w.D, w.bs, w.num_blocks, int(w.lengths.max()), ctypes.c_float(w.scale),
        pa.PA_BF16 if w.dtype == "bf16" else pa.PA_F16, P,
        None if items is None else items.data_ptr(), n,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None, None)
    assert rc == 0, L.pa_last_error()


def _with_workspace(g, w, P, items):
    out = torch.full((w.S, w.Hq, w.D), 0x7FFF, dtype=torch.int16, device="cuda")
    mcl = int(w.lengths.max())
    ws = torch.empty(max(pa.pa_decode_partitioned_workspace_size(w.S, w.Hq, w.D, mcl, P), 16),
                     dtype=torch.uint8, device="cuda")
    c, st = g.cache, g.step
    pa.pa_decode_partitioned(out, g.q, c.key_cache, c.value_cache, st.block_tables,
                             st.context_lens, mcl, w.scale, w.dtype, P, ws, items)
    torch.cuda.synchronize()
    return gpu_side.to_host16(out)


@pytest.mark.parametrize("listed", [False, True], ids=["dense", "list"])
def test_noalloc_matches_caller_workspace_twice(listed):
    # first the Qwen2.5-7B-shaped small workload, then a smaller one (fewer,
    # shorter sequences, another head grouping): the second call's partials
    # land in the array the first one filled
    cases = [(workload(3, "small"), 512), (workload(1, "full"), 16)]
    assert cases[1][0].S * cases[1][0].Hq < cases[0][0].S * cases[0][0].Hq
    for w, P in cases:
        label = f"no-alloc {w.spec.name[:40]} P={P} {'list' if listed else 'dense'}"
        need = pa.pa_decode_partitioned_workspace_size(w.S, w.Hq, w.D, int(w.lengths.max()), P)
        assert need <= pa.pa_decode_partitioned_noalloc_max_workspace()
        g = gpu_side.build(w)
        o = oracle_side.build(w)
        items = torch.from_numpy(pa.partition_work_items(w.lengths, P)).cuda() if listed else None
        out = torch.full((w.S, w.Hq, w.D), 0x7FFF, dtype=torch.int16, device="cuda")
        _call_noalloc(g, w, P, items, out)
        torch.cuda.synchronize()
        got = gpu_side.to_host16(out)
        ref = _with_workspace(g, w, P, items)
        assert np.array_equal(got, ref), f"{label}: differs from pa_decode_partitioned"
        ref32, refT = oracle.decode(o.q, o.key_cache, o.value_cache, o.block_tables,
                                    o.context_lens, w.scale, w.dtype, nthreads=ORACLE_THREADS)
        check_outputs(got, ref32, refT, w.dtype, label)
        del g
        free_gpu()
