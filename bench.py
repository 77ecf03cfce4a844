"""Paged decode attention benchmark on one MI355X.

One step = the whole decode path for one batch: host block allocation and
slot assignment (a1), the metadata copy to the GPU (a2), the cache write of
the new tokens (a3) and the decode (split-context partitions + merge, or
single pass, by workload).  Inputs are synthetic and seeded (workloads/),
resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--config 3] [--block-size 16] [--kv-dtype int8]
    python bench.py --prefill [--steps K] [--warmup W]     (chunked-prefill attention)

Prints one JSON line on stdout.  value = algorithmic K/V bytes read by the
timed steps' decodes / wall time of the timed steps (GB/s); the decode call
alone is also timed with HIP events that its own launches record, on the
step's stream: every timed step's decode up to 20 steps, then every k-th with
at least 20 timed (roofline.achieved).  Before the warm-up, the decode of the
prepared state runs back to back for --settle-ms so the clocks have settled.
"""
import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read GB/s (% of HBM peak); seqs/s per layer"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD's published figure
MIN_TIMED_DECODES = 20  # decodes timed with HIP events: every step up to this many steps,
                        # then every k-th step with at least this many timed


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(o, w, budget_s, threads, int8):
    """Oracle decodes of whole sequences (all q heads; a seeded order, cycling)
    on `threads` host threads until about budget_s seconds of work: (bytes/s,
    sequences/s, sequences, tokens, seconds)."""
    import oracle

    per_tok = 2 * w.Hkv * (w.D + 4) if int8 else 2 * w.Hkv * w.D * w.elem_bytes
    spent, done_bytes, nseq, ntok = 0.0, 0, 0, 0
    order = np.random.default_rng(1234).permutation(w.S)
    k = 0
    batch_n = 4 if threads > 1 else 1
    while spent < budget_s:
        batch = [int(order[(k + j) % w.S]) for j in range(batch_n)]
        k += batch_n
        pairs = np.array([[i, h] for i in batch for h in range(w.Hq)], np.int32)
        t0 = time.perf_counter()
        if int8:
            oracle.decode_int8(o.q, o.key_cache, o.value_cache, o.key_scale, o.value_scale,
                               o.block_tables, o.context_lens, w.scale, w.dtype, pairs=pairs,
                               nthreads=threads)
        else:
            oracle.decode_pairs(o.q, o.key_cache, o.value_cache, o.block_tables, o.context_lens,
                                w.scale, w.dtype, pairs, nthreads=threads)
        spent += time.perf_counter() - t0
        toks = int(sum(int(w.lengths[i]) for i in batch))
        done_bytes += toks * per_tok
        ntok += toks
        nseq += len(batch)
    return done_bytes / spent, nseq / spent, nseq, ntok, spent


def cpu_baseline(w, budget_s, int8=False):
    """The oracle as it stands, timed on the host cores over whole sequences of
    the same workload: on every core the process may use (about budget_s
    seconds of work), then on one thread (about half that)."""
    from tests import oracle_side

    o = oracle_side.build_int8(w) if int8 else oracle_side.build(w)
    threads = len(os.sched_getaffinity(0))
    bps, sps, nseq, ntok, spent = _oracle_rate(o, w, budget_s, threads, int8)
    bps1, sps1, nseq1, ntok1, spent1 = _oracle_rate(o, w, budget_s / 2, 1, int8)
    what = "stored K/V bytes (codes + scales)" if int8 else "logical K/V bytes"
    return {
        "value": bps / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{nseq} sequence decodes drawn cyclically from the workload's {w.S} "
                   f"(all {w.Hq} q heads each, {ntok} tokens) on {threads} threads, "
                   f"{spent:.1f} s of oracle time; {what} of the sample / oracle decode time"),
        "seqs_per_s": sps,
        "single_thread": {
            "value": bps1 / 1e9, "unit": "GB/s", "cores": 1, "seqs_per_s": sps1,
            "sample": f"{nseq1} sequence decodes ({ntok1} tokens), {spent1:.1f} s on one thread"},
        "cpu_model": cpu_model(),
        "nproc": os.cpu_count(),
    }


PREFILL_METRIC = "chunked-prefill attention TFLOP/s (causal, % of bf16 MFMA peak)"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak, AMD's published figure


def prefill_cpu_baseline(w, budget_s):
    """The oracle's prefill on the last r query rows of every chunk (the same
    positions as in the workload), r doubling until about budget_s seconds."""
    import oracle
    from tests.test_gpu_parity_prefill import build_oracle
    from workloads import prefill_workload

    kc, vc, bt = build_oracle(w)
    threads = len(os.sched_getaffinity(0))
    r = 1
    while True:
        sub = prefill_workload("full", chunks=tuple(min(r, int(n)) for n in w.chunks))
        q = sub.query()
        t0 = time.perf_counter()
        oracle.prefill(q, kc, vc, bt, w.lengths, sub.query_start, w.scale, w.dtype,
                       nthreads=threads)
        spent = time.perf_counter() - t0
        if spent > budget_s / 3 or r >= int(w.chunks.max()):
            break
        r *= 2
    return {"value": sub.flops() / spent / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"the last {r} query rows of each of the {w.S} chunks (all {w.Hq} heads, "
                       f"{sub.T} rows), {spent:.1f} s of oracle time; causal FLOPs of the sample / "
                       "oracle time")}


def run_prefill(args):
    import torch
    from paged_kv_cache_106_amd import pa_prefill
    from paged_kv_cache_106_amd._hip import Event
    from tests.test_gpu_parity_prefill import build_gpu, dev
    from workloads import prefill_workload

    w = prefill_workload("full")
    log(f"[bench] {w.spec.name}; rows={w.T}; {w.flops() / 1e9:.1f} GFLOP per call")
    kc, vc, bt, lens, qs, _ = build_gpu(w)
    q = dev(w.query())
    out = torch.empty((w.T, w.Hq, w.D), dtype=torch.int16, device="cuda")
    mql = int(w.chunks.max())
    # longest context first (host-side order, like the decode's work list)
    order = dev(np.argsort(-w.lengths, kind="stable").astype(np.int32))
    for _ in range(args.warmup):
        pa_prefill(out, q, kc, vc, bt, lens, qs, mql, w.scale, w.dtype, seq_order=order)
    torch.cuda.synchronize()
    ev = [(Event(timing=True), Event(timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        pa_prefill(out, q, kc, vc, bt, lens, qs, mql, w.scale, w.dtype, seq_order=order,
                   start_event=a, stop_event=b)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    fl = w.flops()
    value = fl * args.steps / elapsed / 1e12
    achieved = fl / float(t.mean()) / 1e12
    result = {
        "metric": PREFILL_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, seeded block scatter)",
        "config": {"workload": w.spec.name, "num_seqs": w.S, "query_rows": w.T,
                   "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
                   "block_size": w.bs, "flops_per_call": fl,
                   "flops_counting": "4 x head_dim per (query row, head, visible key)"},
        "prefill_us": round(float(t.mean()) * 1e6, 2),
        "prefill_us_p10_p90": [round(float(np.percentile(t, 10)) * 1e6, 2),
                               round(float(np.percentile(t, 90)) * 1e6, 2)],
        "query_tokens_per_s": round(w.T / float(t.mean()), 1),
        "roofline": {"bound": "mfma", "kernel": "pa_prefill: prefill_kernel",
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile("prefill_qwen25_7b_gqa_8x512_profile.md",
                                                     "prefill"),
                     "traffic_unit": "bytes per call (FETCH_SIZE x2 + WRITE_SIZE, copy-calibrated)"},
    }
    del kc, vc
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


KERNEL_SOURCES = {
    # the sources each kernel family is built and launched from (for the
    # decode also the work-list builder, which orders its workgroups)
    "decode": ("pa_attn*", "pa_internal.h", "pa_api.hip", "pa_allocator.cpp"),
    "prefill": ("pa_prefill.hip", "pa_mfma.h", "pa_internal.h"),
}


def input_digests(w):
    """sha256 (first 16 hex digits) of the workload's small host inputs: the
    drawn lengths, the initial order of the block pool and the queries, so a
    run can be matched to its inputs."""
    import hashlib
    d = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
    return {"lengths": d(w.lengths), "free_order": d(w.initial_free_order), "q": d(w.query())}


def kernel_source_sha256(kind="decode"):
    """sha256 over the sources one kernel family is built and launched from."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_106_amd", "csrc")
    files = set()
    for pat in KERNEL_SOURCES[kind]:
        files.update(glob.glob(os.path.join(csrc, pat)))
    for f in sorted(files):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(name, kind):
    """HBM bytes per call from a committed PMC summary under profiles/, or
    None if there is none or the kernel sources changed since it was taken."""
    import re
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^kernel_source_sha256: (\w+)", text, re.M)
    tr = re.search(r"^traffic_bytes_per_call: (\d+)", text, re.M)
    if not sha or not tr or sha.group(1) != kernel_source_sha256(kind):
        return None
    return int(tr.group(1))


def recorded_traffic(config_id, block_size, int8=False):
    """HBM bytes per decode call of a workload from its PMC summary (or None)."""
    names = {(2, False): "decode_llama13b_mha_32seq_pmc.md",
             (3, False): "decode_qwen25_7b_gqa_64seq_pmc.md",
             (3, True): "decode_qwen25_7b_gqa_64seq_int8_pmc.md",
             (4, False): "decode_7b_gqa_longctx_16seq_pmc.md",
             (5, False): "decode_continuous_batch_256seq_pmc.md"}
    name = names.get((config_id, int8)) if block_size in (None, 16) else None
    return traffic_from_profile(name, "decode") if name else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--block-size", type=int, default=None, choices=[16, 32])
    ap.add_argument("--kv-dtype", default=None, choices=["int8"],
                    help="INT8 KV pools (codes + fp32 row scales) instead of 16-bit ones")
    ap.add_argument("--prefill", action="store_true",
                    help="time the chunked-prefill attention (pa_prefill) instead of a decode step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up, decode calls back to back (the same inputs, "
                         "no step state changes) for this long, so the GPU clocks have "
                         "settled when the steps start")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gc", dest="no_gc", action="store_false",
                    help="keep Python's garbage collector on during the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libpa has no multi-GPU path "
              "(decode attention would shard by sequence or by KV head)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tests import gpu_side
    from workloads import workload

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.int32, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "bytes_written": 1 << 30,
                          "launches": 5}), flush=True)
        return
    if args.prefill:
        return run_prefill(args)
    overrides = {"block_size": args.block_size} if args.block_size else {}
    # each step appends a token to every sequence: the cache starts short by
    # the warm-up plus half the timed steps, so the timed steps centre on the
    # workload's lengths
    w = workload(args.config, "full", length_shift=args.warmup + args.steps // 2, **overrides)
    # a pool the configuration fixes (the tiny workload's 64 blocks) may not
    # hold the tokens the steps append: it then grows to what they need
    grown = args.warmup + args.steps + 1
    need = sum(-(-(int(x) + grown) // w.bs) for x in w.lengths)
    if w.spec.prefix_seqs > 1:
        need -= (w.spec.prefix_seqs - 1) * (w.spec.prefix_len // w.bs)
    pool_grown = need > w.num_blocks
    if pool_grown:
        w = workload(args.config, "full", length_shift=args.warmup + args.steps // 2,
                     num_blocks=need, **overrides)
    log(f"[bench] {w.spec.name}; bs={w.bs}; S={w.S}; KV bytes/step ~{w.kv_bytes()/1e6:.1f} MB")
    t0 = time.perf_counter()
    int8 = args.kv_dtype == "int8"
    g = gpu_side.build(w, extra_tokens=args.warmup + args.steps + 1, kv_dtype=args.kv_dtype)
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    step = g.step
    stream = step.stream
    per_tok = g.cache.kv_bytes_per_token()
    shared = (w.spec.prefix_seqs - 1) * w.spec.prefix_len if w.spec.prefix_seqs > 1 else 0

    # HIP events recorded by the decode's launches themselves (hipExtLaunchKernel):
    # start of its first kernel, end of its last, on the step's stream, with no
    # marker packet in the stream (a marker costs a few microseconds of GPU time)
    # (each event still costs the stream a few microseconds: every step's decode
    # is timed up to MIN_TIMED_DECODES steps, then every k-th with at least
    # MIN_TIMED_DECODES of them)
    from paged_kv_cache_106_amd._hip import Event
    time_every = max(1, args.steps // MIN_TIMED_DECODES)
    ev = {k: (Event(timing=True), Event(timing=True)) for k in range(0, args.steps, time_every)}
    kv_bytes, len_sum = 0, 0.0
    host = np.zeros((args.steps, 4))                            # host seconds per phase
    # the collector is run and paused before the warm-up, so nothing but the
    # synchronisation separates the warm-up from the timed steps (an idle GPU
    # between them changes its clocks for the first timed steps)
    gc.collect()
    gc_was_enabled = gc.isenabled()
    if args.no_gc:
        gc.disable()       # a collection pass over this large heap stalls the host for ~30 ms
    settle_calls = 0
    if args.settle_ms > 0:
        # the decode of the current state, repeated: no token is appended
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
            for _ in range(10):
                step.attend(g.q)
            settle_calls += 10
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(g.q, g.k_new, g.v_new)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        h0 = time.perf_counter()
        b = step.prepare()                                      # a1
        h1 = time.perf_counter()
        step.upload(b)                                          # a2 (copy-on-write pairs only)
        h2 = time.perf_counter()
        step.write_new(g.k_new, g.v_new)                        # a2 + a3: one launch
        h3 = time.perf_counter()
        step.attend(g.q, *ev.get(k, (None, None)))              # a4 | a5 + a6
        host[k] = (h1 - h0, h2 - h1, h3 - h2, time.perf_counter() - h3)
        kv_bytes += (int(step.host_context_lens.astype(np.int64).sum()) - shared) * per_tok
        len_sum += float(step.host_context_lens.mean())
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if gc_was_enabled:
        gc.enable()
    log(f"[bench] {args.warmup} warmup and {args.steps} timed steps done")

    t_decode = np.array([a.elapsed_time(b) for a, b in ev.values()]) * 1e-3   # s
    kv_per_call = kv_bytes / args.steps
    value = kv_bytes / elapsed / 1e9
    dec_avg = float(t_decode.mean())
    achieved = kv_per_call / dec_avg / 1e9
    kernel_name = ("pa_decode_partitioned: partition kernel + merge kernel"
                   if w.spec.kernel == "partitioned" else "pa_decode: single-pass kernel")
    if int8:
        kernel_name = kernel_name.replace("pa_decode", "pa_decode_int8").replace(
            "pa_decode_int8_partitioned", "pa_decode_partitioned_int8")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) q/k/v, seeded lengths and block scatter)",
        "config": {
            "workload": w.spec.name,
            "num_seqs": w.S, "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
            "block_size": w.bs, "kernel": w.spec.kernel,
            "partition_size": w.spec.partition_size if w.spec.kernel == "partitioned" else None,
            "partition_grid": g.step.last_grid,
            "seed": w.spec.seed,
            "inputs_sha256": input_digests(w),
            "mean_context_len": round(len_sum / args.steps, 2),      # over the timed steps
            "num_blocks": w.num_blocks,
            "pool_grown_for_steps": pool_grown,
            "kv_dtype": "int8 codes + fp32 row scales" if int8 else w.dtype,
            "kv_bytes_per_step": int(kv_per_call),
            "kv_bytes_counting": ("unique (a shared prefix once)" if shared else "logical") +
                                 (", codes + scales as stored" if int8 else ""),
        },
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s_per_layer": round(w.S * args.steps / elapsed, 1),
        "decode_us": round(dec_avg * 1e6, 2),
        "decode_us_p50": round(float(np.median(t_decode)) * 1e6, 2),
        "decode_timed_steps": len(t_decode),
        "decode_timed_every": time_every,
        "clock_settle_decodes": settle_calls,
        "decode_us_p10_p90": [round(float(np.percentile(t_decode, 10)) * 1e6, 2),
                              round(float(np.percentile(t_decode, 90)) * 1e6, 2)],
        "decode_seqs_per_s": round(w.S / dec_avg, 1),
        "host_us_per_step": dict(zip(("prepare", "upload", "write", "attend"),
                                     (round(float(x) * 1e6, 1) for x in host.mean(axis=0)))),
        "host_prepare_us_p50_max": [round(float(np.median(host[:, 0])) * 1e6, 1),
                                    round(float(host[:, 0].max()) * 1e6, 1)],
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(args.config, args.block_size, int8),
            "traffic_unit": "bytes per decode call (FETCH_SIZE x2 + WRITE_SIZE, copy-calibrated)",
        },
    }
    del g
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        # the oracle on the workload's own lengths
        result["cpu_baseline"] = cpu_baseline(workload(args.config, "full", **overrides),
                                              args.cpu_seconds, int8)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
