"""Benchmark of one decode step of paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole hot path over one batch: the cache write of
each sequence's newest token followed by decode attention of every
sequence's query over its paged history (one pa_decode_append call; with
--unfused, reshape_and_cache then pa_paged_attention_decode).  The default workload is the
Qwen-7B-shaped GQA batch (64 sequences, 28 query / 4 KV heads, head_dim 128,
block size 16, context lengths ~ U[512, 4096], bf16).  Inputs are seeded
synthetic tensors already resident in HBM.  Steps rotate over R copies of the
KV pool so that no step finds its KV bytes in the 256 MB last-level cache left
there by the previous one.

The K timed steps are captured once in a HIP graph (as a serving loop would
launch a decode step) and the timed region is one replay, bracketed by a
device synchronisation on both sides; --eager launches them one by one.

Prints ONE JSON line: throughput (decode tokens/s = sequences per second of
steps); the decode call's achieved KV bandwidth against the 8 TB/s HBM peak
(HIP events on the stream the kernels run on, around replays of a graph of
200 decode calls whatever K is, so that the replay's own start-up is spread
thin: partition kernel + merge kernel); the same figures for every seeded
workload; and the float64 CPU oracle timed on bounded samples of the same
workloads.
"""

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
METRIC = "decode attention tokens/s and achieved KV HBM GB/s (% of peak), 1 MI355X"
# committed rocprofv3 summaries of `bench.py --config NAME --decode-only`
TRAFFIC_FILE = os.path.join(HERE, "profiles", "decode_%s_traffic.json")
TRACE_FILE = os.path.join(HERE, "profiles", "decode_%s_kernel_trace.json")
# decode calls per graph replay behind the call-duration figures (any --steps):
# a replay's start-up costs tens of microseconds, which a short replay would
# spread over too few calls
DECODE_CALLS = 200
# the seeded workloads, timed one after another in the "workloads" figure
WORKLOADS = ("tiny_fp32", "qwen7b_gqa_bf16", "llama7b_mha_fp16", "long_ctx_bf16",
             "mixed_shared_bf16")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen7b_gqa_bf16")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--kernel", choices=["auto", "generic", "mfma"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=8.0,
                    help="wall-time budget of the oracle sample")
    ap.add_argument("--decode-only", action="store_true",
                    help="time decode calls only, on cold pool replicas (for counter and "
                         "trace runs): no hot-cache, single-call, other-operation or "
                         "workload figures")
    ap.add_argument("--decode-calls", type=int, default=DECODE_CALLS,
                    help="decode calls per graph replay behind the call-duration figures")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the figures of the other seeded workloads")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a graph")
    ap.add_argument("--unfused", action="store_true",
                    help="cache write and decode as two calls instead of pa_decode_append")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run the plain copy kernel of this size, 5 times")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the block-size x head-dim sweep (one JSON line per shape)")
    ap.add_argument("--sweep-out", default=None,
                    help="with --sweep or --sweep-lengths: also write the table as markdown to this file")
    ap.add_argument("--sweep-head-dims", default="64,128,256",
                    help="with --sweep: comma-separated head dims")
    ap.add_argument("--sweep-block-sizes", default="8,16,32,64",
                    help="with --sweep: comma-separated block sizes")
    ap.add_argument("--sweep-lengths", action="store_true",
                    help="only run the context-length x batch sweep (one JSON line per point)")
    ap.add_argument("--sweep-lens", default="64,256,1024,4096,16384,65536,131072",
                    help="with --sweep-lengths: comma-separated history lengths")
    ap.add_argument("--sweep-seqs", default="1,4,16,64,256,1024,2048",
                    help="with --sweep-lengths: comma-separated batch sizes")
    ap.add_argument("--sweep-kv", default="bf16,fp8",
                    help="with --sweep-lengths: KV formats (bf16, fp8)")
    ap.add_argument("--sweep-max-tokens", type=int, default=1 << 23,
                    help="with --sweep-lengths: largest batch history (tokens) swept")
    return ap.parse_args()


def kernel_source_hash():
    from paged_kv_decode_attention_amd.build import decode_source_hash
    return decode_source_hash()


def load_traffic(config_name, per_launch_alg_bytes):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; else None."""
    path = TRAFFIC_FILE % config_name
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def load_kernel_only(config_name, alg_bytes):
    """rocprofv3 kernel-only durations of the bench call's two kernels (the
    16-bit matrix-core decode kernel and its merge kernel) from the committed
    kernel trace of `bench.py --decode-only` (every dispatch reads a cold pool
    replica), if it was taken on the current kernel sources; else None."""
    path = TRACE_FILE % config_name
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_source_hash():
        return None
    ks = t.get("kernels", {})
    # the run's decode and merge kernels: the most-called of each
    most = lambda key: max(((k, v) for k, v in ks.items() if key in k),
                           key=lambda kv: kv[1]["calls"], default=(None, None))[1]
    dec = most("decode_")
    mrg = most("merge_")
    if not dec or not mrg:
        return None
    pick = lambda k: {x: k[x] for x in ("calls", "avg_us", "median_us", "min_us", "max_us")}
    return {"source": os.path.relpath(path, HERE),
            "decode_kernel": pick(dec), "merge_kernel": pick(mrg),
            "decode_kernel_gbps": alg_bytes / (dec["median_us"] * 1e-6) / 1e9,
            "decode_kernel_frac": alg_bytes / (dec["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def _oracle_arrays(inp):
    """The oracle's inputs: exactly the values the GPU reads, as float32
    (upcast to float64 inside the oracle), tables as int64."""
    import numpy as np
    return (inp.query.float().numpy(), inp.key_cache.float().numpy(),
            inp.value_cache.float().numpy(), inp.block_tables.numpy().astype(np.int64),
            inp.context_lens.numpy().astype(np.int64))


def oracle_rate(arrays, scale, budget_s):
    """The oracle (float64 gather + softmax) on one host thread: passes over
    the batch's sequences, one sequence (all heads) at a time, until the
    wall-time budget is spent (at least one sequence).  Returns (sequence
    steps, history tokens, seconds)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    import oracle

    q, kc, vc, bt, cl = arrays
    S, H = q.shape[0], q.shape[1]
    done, tokens, elapsed = 0, 0, 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        while elapsed < budget_s or done == 0:
            b = done % S
            t0 = time.perf_counter()
            oracle.decode_contiguous(q, kc, vc, bt, cl, scale, pairs=[(b, h) for h in range(H)])
            elapsed += time.perf_counter() - t0
            done += 1
            tokens += int(cl[b])
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return done, tokens, elapsed


def cpu_baseline(inp, budget_s):
    """The oracle on the host: one thread (the reported value), and every
    core of the process's affinity set as a pool of worker processes over
    sequences (all_cores), each for about budget_s of wall time on a bounded
    sample of the workload."""
    arrays = _oracle_arrays(inp)
    q, kc = arrays[0], arrays[1]
    S, H = q.shape[0], q.shape[1]
    # float64 K and V bytes of one history token (all KV heads): the gathered
    # rows the oracle reduces
    kv_row_bytes = 2 * kc.shape[1] * kc.shape[3] * 8
    done, tokens, elapsed = oracle_rate(arrays, inp.cfg.scale, budget_s)
    return {
        "value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": "float64 oracle (contiguous gather + softmax), %d sequence-steps "
                  "(%.2f passes over the %d sequences, all %d heads, %d history tokens), "
                  "%.1f s, 1 BLAS thread" % (done, done / S, S, H, tokens, elapsed),
        "seconds": elapsed,
        "fp64_gbps": tokens * kv_row_bytes / elapsed / 1e9,
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "all_cores": cpu_baseline_pool(arrays, inp.cfg.scale, budget_s),
    }


_POOL = {}


def _pool_init(d):
    """Worker start-up: map the oracle's inputs read-only from files (shared
    page cache, nothing pickled) and hold BLAS to one thread."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass
    for k in ("q", "kc", "vc", "bt", "cl"):
        _POOL[k] = np.load(os.path.join(d, k + ".npy"), mmap_mode="r")
    with open(os.path.join(d, "scale")) as f:
        _POOL["scale"] = float(f.read())


def _pool_seq(b):
    """One sequence (all heads) through the oracle in a worker process."""
    import oracle
    P = _POOL
    H = P["q"].shape[1]
    oracle.decode_contiguous(P["q"], P["kc"], P["vc"], P["bt"], P["cl"], P["scale"],
                             pairs=[(b, h) for h in range(H)])
    return int(P["cl"][b])


def cpu_baseline_pool(arrays, scale, budget_s, max_workers=16):
    """The oracle on a pool of worker processes (one per core of the affinity
    set, at most max_workers, each with one BLAS thread), fed whole passes
    over the batch's sequences for about budget_s of wall time.  Workers are
    started fresh (spawn: no GPU state inherited) and map the inputs from
    temporary files."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile
    import numpy as np

    q, kc, vc, bt, cl = arrays
    S = q.shape[0]
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    d = tempfile.mkdtemp(prefix="pa_oracle_")
    try:
        for k, v in zip(("q", "kc", "vc", "bt", "cl"), arrays):
            np.save(os.path.join(d, k + ".npy"), v)
        with open(os.path.join(d, "scale"), "w") as f:
            f.write(repr(float(scale)))
        with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                    initializer=_pool_init, initargs=(d,)) as ex:
            list(ex.map(_pool_seq, [b % S for b in range(workers)]))     # workers up
            done, tokens = 0, 0
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < budget_s:
                tokens += sum(ex.map(_pool_seq, range(S)))              # one pass
                done += S
            elapsed = time.perf_counter() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    kv_row_bytes = 2 * kc.shape[1] * kc.shape[3] * 8
    return {"value": done / elapsed, "unit": "tokens/s", "cores": workers,
            "fp64_gbps": tokens * kv_row_bytes / elapsed / 1e9,
            "sample": "%d sequence-steps (whole passes over the batch) on %d worker processes "
                      "in %.1f s" % (done, workers, elapsed)}


def unique_kv_bytes(cfg, block_tables, context_lens):
    """K+V bytes of the distinct (physical block, slot) token rows a decode
    call reads: a block shared by several sequences' tables (the shared
    prefixes of the mixed workload) counts once."""
    import numpy as np
    from paged_kv_decode_attention_amd.inputs import ELEM_BYTES
    bt = np.asarray(block_tables, dtype=np.int64)
    cl = np.asarray(context_lens, dtype=np.int64)
    BS = cfg.block_size
    rows = [bt[b, np.arange(int(cl[b])) // BS] * BS + np.arange(int(cl[b])) % BS
            for b in range(bt.shape[0])]
    n = np.unique(np.concatenate(rows)).size if rows else 0
    return int(n) * cfg.num_kv_heads * cfg.head_dim * ELEM_BYTES[cfg.dtype] * 2


def kernel_label(S, H_kv, G, D, BS, max_ctx, dtype):
    """The kernel family and schedule a decode call of this shape takes: calls
    small enough for one fixed partition per history (the library's
    pa_decode_partition_size) run one launch, float32 ones on the vector ALU."""
    import torch
    from paged_kv_decode_attention_amd import ops

    fam = ops.decode_kernel(D, BS, G, dtype)
    P = ops.decode_partition_size(S, H_kv, G, D, BS, max_ctx, dtype)
    if P >= max_ctx:
        mfma = fam == ops.KERNEL_MFMA and dtype != torch.float32
        return ("matrix-core" if mfma else "vector-ALU") + ", one partition per history"
    return "matrix-core, balanced" if fam == ops.KERNEL_MFMA else "vector-ALU, partitions"


def graph_call_us(capture, timed_replay, call, n_calls, reps=3):
    """Mean, min and max duration (us) of one call over `reps` replays of a
    graph of n_calls calls (an untimed replay first)."""
    import numpy as np
    import torch
    for k in range(min(10, n_calls)):
        call(k)
    torch.cuda.synchronize()
    g = capture(lambda: [call(k) for k in range(n_calls)])
    g.replay()
    us = np.array([timed_replay(g)[1] / n_calls * 1e6 for _ in range(reps)])
    del g
    return float(us.mean()), float(us.min()), float(us.max())


def workload_rates(dev, capture, timed_replay, oracle_budget_s):
    """Decode-call figures of every seeded workload (decode calls only, pool
    replicas rotated so that at least 1.5 GB of K/V pass between two reads of
    the same bytes), and the oracle on one host thread on a bounded sample
    of each (none when oracle_budget_s is None)."""
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import inputs as I
    from paged_kv_decode_attention_amd import ops

    res = {}
    for name in WORKLOADS:
        cfg = I.CONFIGS[name]
        inp = I.generate(cfg)
        lens = inp.context_lens.numpy()
        alg = I.kv_bytes_read(cfg, lens)
        q = inp.query.to(dev)
        bt = inp.block_tables.to(dev)
        cl = inp.context_lens.to(dev)
        S, H, D = q.shape
        N, H_kv, BS, _ = inp.key_cache.shape
        W = bt.shape[1]
        pool = 2 * inp.key_cache.numel() * inp.key_cache.element_size()
        R = int(min(8, max(2, np.ceil(1.5e9 / pool))))
        kcs = [inp.key_cache.to(dev) for _ in range(R)]
        vcs = [inp.value_cache.to(dev) for _ in range(R)]
        out = torch.empty_like(q)
        max_ctx = W * BS
        ws = torch.zeros(max(ops.decode_workspace_size(S, H, H_kv, D, BS, max_ctx, 0, q.dtype),
                             256), dtype=torch.uint8, device=dev)

        def call(k):
            ops.paged_attention_decode(q, kcs[k % R], vcs[k % R], bt, cl, cfg.scale,
                                       max_context_len=max_ctx, out=out, workspace=ws)
        # about 20 ms of calls per replay (at about 6 TB/s)
        n_calls = int(min(DECODE_CALLS, max(20, 2e7 // max(1, alg // 6000))))
        mean, lo, hi = graph_call_us(capture, timed_replay, call, n_calls)
        t = mean * 1e-6
        row = {"call_us_mean": mean, "call_us_min": lo, "call_us_max": hi,
               "calls_per_replay": n_calls, "pool_replicas": R,
               "decode_tokens_per_s": S / t, "alg_bytes_per_call": alg,
               "achieved_gbps": alg / t / 1e9, "frac": alg / t / 1e9 / HBM_PEAK_GBPS,
               "kernel": kernel_label(S, H_kv, H // H_kv, D, BS, max_ctx, q.dtype),
               "dtype": cfg.dtype}
        if name == "tiny_fp32":
            row["note"] = "launch-bound (%.0f KB of K/V): no roofline claim" % (alg / 1e3)
        if name == "mixed_shared_bf16":
            u = unique_kv_bytes(cfg, inp.block_tables.numpy(), lens)
            row["unique_bytes_per_call"] = u
            row["unique_gbps"] = u / t / 1e9
            row["note"] = ("frac counts logical bytes (every sequence's history, shared "
                           "prefix blocks once per sequence); unique_gbps counts each "
                           "distinct token row once")
        del kcs, vcs, q, bt, cl, out, ws
        torch.cuda.empty_cache()
        if oracle_budget_s is not None:
            arrays = _oracle_arrays(inp)
            done, tokens, el = oracle_rate(arrays, cfg.scale, oracle_budget_s)
            row["oracle_1core"] = {"tokens_per_s": done / el, "sequence_steps": done,
                                   "history_tokens": tokens, "seconds": el}
            del arrays
        res[name] = row
        del inp
    return res


def q8_decode_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes, capture,
                   timed_replay, fmt="fp8"):
    """The same decode calls on 8-bit caches: OCP FP8 E4M3 codes
    (pa_paged_attention_decode_fp8) or INT8 codes (pa_paged_attention_decode_i8).
    Each pool replica is quantised once by the library's own 8-bit cache write
    (every slot written as one token, per-cache scales), then K decode calls
    are replayed from a HIP graph.  Algorithmic bytes are half the 16-bit ones."""
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import ops

    fp8 = fmt == "fp8"
    # unit-variance pools: E4M3 spans +-448 * 1/64 = +-7, INT8 +-127 * 1/24 = +-5.3
    k_scale = v_scale = 1.0 / 64 if fp8 else 1.0 / 24
    write = ops.reshape_and_cache_fp8 if fp8 else ops.reshape_and_cache_i8
    decode = ops.paged_attention_decode_fp8 if fp8 else ops.paged_attention_decode_i8
    N, H_kv, BS, D = kcs[0].shape
    slots = torch.arange(N * BS, dtype=torch.int64, device=dev)
    k8s, v8s = [], []
    for kc, vc in zip(kcs, vcs):
        k8 = torch.empty(N, H_kv, BS, D, dtype=torch.uint8 if fp8 else torch.int8, device=dev)
        v8 = torch.empty_like(k8)
        # pool rows as tokens: [N, BS, H_kv, D] -> [N*BS, H_kv, D], slot = row
        write(kc.permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous(),
              vc.permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous(),
              k8, v8, slots, k_scale, v_scale)
        k8s.append(k8)
        v8s.append(v8)
    out = torch.empty_like(q)
    S, H = q.shape[0], q.shape[1]
    ws = torch.zeros(max(ops.decode_workspace_size(S, H, H_kv, D, BS, max_ctx, 0, q.dtype), 256),
                     dtype=torch.uint8, device=dev)

    def call(k):
        r = k % len(k8s)
        decode(q, k8s[r], v8s[r], bt, cl, k_scale, v_scale, cfg.scale,
               max_context_len=max_ctx, out=out, workspace=ws)
    for k in range(10):
        call(k)
    torch.cuda.synchronize()
    g = capture(lambda: [call(k) for k in range(args.decode_calls)])
    g.replay()
    us = np.array([timed_replay(g)[1] / args.decode_calls * 1e6 for _ in range(3)])
    t = float(us.mean()) * 1e-6
    alg8 = alg_bytes // 2
    del k8s, v8s
    return {"kv_format": ("OCP FP8 E4M3" if fp8 else "INT8 symmetric") + ", per-cache scales",
            "decode_us_mean": t * 1e6,
            "decode_tokens_per_s": S / t, "alg_bytes_per_launch": alg8,
            "achieved_gbps": alg8 / t / 1e9, "frac": alg8 / t / 1e9 / HBM_PEAK_GBPS,
            "bound": "hbm"}


def verify_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes, capture,
                timed_replay, q_len=4):
    """Verify step (pa_paged_attention_verify) on the same workload: q_len new
    query tokens per sequence, K calls replayed from a HIP graph.  The
    matrix-core kernel serves 16 // G query tokens of a sequence per pass over
    its K/V (their (token, head) pairs are its 16 columns), or 32 // G with
    two column tiles when q_len * G > 16 (head_dim 64 and 128), so a call
    reads the histories ceil(q_len / tokens per pass) times."""
    import math
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import ops

    S, H, D = q.shape
    N, H_kv, BS, _ = kcs[0].shape
    qv = q.repeat_interleave(q_len, dim=0).contiguous()
    qs = torch.arange(0, S * q_len + 1, q_len, dtype=torch.int32, device=dev)
    out = torch.empty_like(qv)
    ws = torch.zeros(max(ops.load_library().pa_verify_workspace_size(
        S * q_len, H, H_kv, D, BS, max_ctx, 0, ops.dtype_code(q.dtype)), 256),
        dtype=torch.uint8, device=dev)

    def call(k):
        r = k % len(kcs)
        ops.paged_attention_verify(qv, kcs[r], vcs[r], bt, cl, qs, q_len, cfg.scale,
                                   max_context_len=max_ctx, out=out, workspace=ws)
    for k in range(10):
        call(k)
    torch.cuda.synchronize()
    g = capture(lambda: [call(k) for k in range(args.decode_calls)])
    g.replay()
    us = np.array([timed_replay(g)[1] / args.decode_calls * 1e6 for _ in range(3)])
    del g
    t = float(us.mean()) * 1e-6
    G = H // H_kv
    cols = 32 if q_len * G > 16 and D <= 128 else 16
    per_pass = max(1, cols // G)
    passes = math.ceil(q_len / per_pass)
    read = alg_bytes * passes       # histories read once per pass (to first order)
    return {"query_tokens_per_seq": q_len, "call_us_mean": t * 1e6,
            "verified_tokens_per_s": S * q_len / t, "alg_bytes_per_launch": alg_bytes,
            "kv_passes": passes, "kv_bytes_read_approx": read, "read_gbps": read / t / 1e9,
            "note": "%d query tokens of a sequence share a pass over its K/V "
                    "(%d (token, head) columns of %d)" % (per_pass, per_pass * G, cols)}


def graph_time_s(call, K):
    """Seconds per call(j): K calls captured in one HIP graph (after 5 eager
    warm-up calls), HIP events around each of 3 replays, the mean."""
    import numpy as np
    import torch
    for j in range(5):
        call(j)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(gr, stream=st):
            for j in range(K):
                call(j)
    torch.cuda.current_stream().wait_stream(st)
    gr.replay()
    torch.cuda.synchronize()
    us = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / K)
    del gr
    return float(np.mean(us)) * 1e-6


def shape_sweep(args, dev):
    """Decode-call rate over block sizes 8/16/32/64 and head dims 64/128/256,
    on 16-bit caches and on FP8 E4M3 and INT8 caches: the bench batch (64
    sequences, 28 query / 4 KV heads, the same seeded context lengths), bf16
    queries, shuffled tables, random pools on the GPU (the 8-bit ones quantised
    by the library's cache writes), pool replicas rotated so the last-level cache
    cannot hold the working set; K calls replayed from a HIP graph, HIP
    events around each replay.  Then the shapes the vector-ALU kernel serves
    (the same batch): fp32 at each head dim; and bf16 with more query heads
    per KV head than one matrix-core pass takes, which run as several passes
    (64 on one KV head at head_dim 128, 32 at 256, and 37 per KV head, two
    unequal passes, at 128)."""
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import inputs as I
    from paged_kv_decode_attention_amd import ops

    base = I.CONFIGS["qwen7b_gqa_bf16"]
    lens = I.draw_context_lens(base).astype(np.int64)
    S = base.num_seqs
    K = min(args.steps, 100)
    scales = {"fp8": 1.0 / 64, "int8": 1.0 / 24}
    rows = []

    def timed(call):
        return graph_time_s(call, K)

    def run(D, BS, H, H_kv, dt, kvs):
        G = H // H_kv
        rng = np.random.default_rng(7)
        nblk = -(-lens // BS)
        N = int(nblk.sum()) + 64
        W = -(-4096 // BS)
        perm = rng.permutation(N).astype(np.int32)
        bt = np.full((S, W), -1, dtype=np.int32)
        k = 0
        for b in range(S):
            bt[b, :nblk[b]] = perm[k:k + nblk[b]]
            k += nblk[b]
        g = torch.Generator(device=dev).manual_seed(11)
        q = torch.randn(S, H, D, generator=g, device=dev).to(dt)
        btd = torch.from_numpy(bt).to(dev)
        cld = torch.from_numpy(lens.astype(np.int32)).to(dev)
        out = torch.empty_like(q)
        max_ctx = W * BS
        ws = torch.zeros(max(ops.decode_workspace_size(S, H, H_kv, D, BS, max_ctx, 0, q.dtype),
                             256), dtype=torch.uint8, device=dev)
        mfma = ops.decode_kernel(D, BS, G, q.dtype) == ops.KERNEL_MFMA
        for kv in kvs:
            if kv in ("fp8", "int8") and not mfma:
                continue
            k_scale = v_scale = scales.get(kv, 1.0)
            e = {"fp8": 1, "int8": 1}.get(kv, q.element_size())
            pool = N * H_kv * BS * D * e
            # replicas cycled through: 1.2 GB or more of K/V between two
            # reads of the same bytes, well beyond the 256 MB last-level
            # cache
            R = max(2, int(np.ceil(1.2e9 / (2 * pool))))
            kcs, vcs = [], []
            for _ in range(2 * R):
                x = torch.randn(N, H_kv, BS, D, generator=g, device=dev).to(dt)
                if kv in ("fp8", "int8"):
                    # pool rows as tokens: slot pb * BS + off holds row (pb, :, off)
                    c = torch.empty(N, H_kv, BS, D, device=dev,
                                    dtype=torch.uint8 if kv == "fp8" else torch.int8)
                    rows_ = x.permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous()
                    slots = torch.arange(N * BS, dtype=torch.int64, device=dev)
                    write = (ops.reshape_and_cache_fp8 if kv == "fp8"
                             else ops.reshape_and_cache_i8)
                    write(rows_, rows_, c, torch.empty_like(c), slots, k_scale, v_scale)
                    x = c
                (kcs if len(kcs) < R else vcs).append(x)
            torch.cuda.synchronize()

            if kv in ("fp8", "int8"):
                dec = (ops.paged_attention_decode_fp8 if kv == "fp8"
                       else ops.paged_attention_decode_i8)

                def call(j):
                    dec(q, kcs[j % R], vcs[j % R], btd, cld, k_scale, v_scale,
                        max_context_len=max_ctx, out=out, workspace=ws)
            else:
                def call(j):
                    ops.paged_attention_decode(q, kcs[j % R], vcs[j % R], btd, cld,
                                               max_context_len=max_ctx, out=out, workspace=ws)
            t = timed(call)
            alg = int(lens.sum()) * H_kv * D * e * 2
            cap = 16 if D == 256 else 32
            passes = -(-G // cap) if mfma else 1     # the matrix-core kernel's passes
            heads = "%d/%d" % (H, H_kv) + (" (%d passes)" % passes if passes > 1 else "")
            row = {"head_dim": D, "block_size": BS, "heads": heads, "kv_passes": passes,
                   "kv": {"fp8": "fp8 e4m3", "int8": "int8"}.get(kv, kv),
                   "kernel": "matrix-core, balanced" if mfma else "vector-ALU, partitions",
                   "decode_us": t * 1e6, "alg_bytes": alg, "achieved_gbps": alg / t / 1e9,
                   "frac": alg / t / 1e9 / HBM_PEAK_GBPS, "decode_tokens_per_s": S / t,
                   "pool_replicas": R}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del kcs, vcs
            torch.cuda.empty_cache()

    H, H_kv = base.num_heads, base.num_kv_heads
    for D in [int(x) for x in args.sweep_head_dims.split(",")]:
        for BS in [int(x) for x in args.sweep_block_sizes.split(",")]:
            run(D, BS, H, H_kv, torch.bfloat16, ("bf16", "fp8", "int8"))
    for D in [int(x) for x in args.sweep_head_dims.split(",")]:
        run(D, 16, H, H_kv, torch.float32, ("fp32",))
    if "128" in args.sweep_head_dims.split(","):
        run(128, 16, 64, 1, torch.bfloat16, ("bf16",))
    if "256" in args.sweep_head_dims.split(","):
        run(256, 16, 32, 1, torch.bfloat16, ("bf16",))
    if "128" in args.sweep_head_dims.split(","):
        run(128, 16, 148, 4, torch.bfloat16, ("bf16", "fp8"))
    if args.sweep_out:
        L = ["# Decode shape sweep: block size x head dim x KV format (64 sequences, "
             "L~U[512,4096] seed 2; 28/4 heads unless the row says otherwise)", "",
             "Command (repository root, one MI355X):", "",
             "    python bench.py --sweep --sweep-out <file>", "",
             "| head_dim | block_size | heads (query/KV) | KV | kernel | decode call us | "
             "KV TB/s | % of 8 TB/s | decode tokens/s |", "|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            L.append("| %d | %d | %s | %s | %s | %.1f | %.2f | %.1f | %.0f |" % (
                r["head_dim"], r["block_size"], r["heads"], r["kv"], r["kernel"],
                r["decode_us"], r["achieved_gbps"] / 1e3, 100 * r["frac"],
                r["decode_tokens_per_s"]))
        L += ["", "Algorithmic bytes: sum_b L_b x KV heads x head_dim x element bytes (4 for "
              "fp32, 2 for bf16, 1 for FP8 E4M3 and INT8) x 2 (K and V), read once; a "
              "group run in several passes reads them once per pass.  "
              "Timing: K decode calls replayed from a HIP graph, HIP events around each "
              "replay, mean of 3."]
        with open(args.sweep_out, "w") as fh:
            fh.write("\n".join(L) + "\n")


LENGTH_MIXES = {"U[32,255]": (32, 255), "U[256,1023]": (256, 1023)}


def length_sweep(args, dev):
    """Decode-call rate over context length x batch: every history of the
    batch L tokens long (L from the --sweep-lens list), S sequences (from
    --sweep-seqs), or L drawn uniformly from a short range (the LENGTH_MIXES
    rows), at 28 query / 4 KV heads, head_dim 128, block size 16, bf16
    queries, on bf16 and FP8 E4M3 caches.  Points with more than
    --sweep-max-tokens history tokens are left out.  Shuffled tables, random
    pools on the GPU (FP8 quantised by the library's cache write), replicas
    rotated so that 1.2 GB or more of K/V lies between two reads of the same
    bytes; K calls replayed from a HIP graph, HIP events around each
    replay."""
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import ops

    H, H_kv, D, BS = 28, 4, 128, 16
    G = H // H_kv
    scale8 = 1.0 / 64
    kvs = args.sweep_kv.split(",")
    points = []
    for L in [int(x) for x in args.sweep_lens.split(",")]:
        for S in [int(x) for x in args.sweep_seqs.split(",")]:
            if S * L <= args.sweep_max_tokens:
                points.append((str(L), S, np.full(S, L, dtype=np.int64)))
    for name, (lo, hi) in LENGTH_MIXES.items():
        for S in (1024, 2048):
            lens = np.random.default_rng(5).integers(lo, hi + 1, size=S).astype(np.int64)
            points.append((name, S, lens))
    rows = []
    for label, S, lens in points:
        rng = np.random.default_rng(7)
        nblk = -(-lens // BS)
        N = int(nblk.sum()) + 16
        W = int(nblk.max())
        perm = rng.permutation(N).astype(np.int32)
        bt = np.full((S, W), -1, dtype=np.int32)
        k = 0
        for b in range(S):
            bt[b, :nblk[b]] = perm[k:k + nblk[b]]
            k += nblk[b]
        g = torch.Generator(device=dev).manual_seed(11)
        q = torch.randn(S, H, D, generator=g, device=dev).to(torch.bfloat16)
        btd = torch.from_numpy(bt).to(dev)
        cld = torch.from_numpy(lens.astype(np.int32)).to(dev)
        out = torch.empty_like(q)
        max_ctx = W * BS
        ws = torch.zeros(max(ops.decode_workspace_size(S, H, H_kv, D, BS, max_ctx, 0, q.dtype),
                             256), dtype=torch.uint8, device=dev)
        for kv in kvs:
            e = 2 if kv == "bf16" else 1
            pool = N * H_kv * BS * D * e
            R = max(1, int(np.ceil(1.2e9 / (2 * pool))))
            kcs, vcs = [], []
            for _ in range(2 * R):
                x = torch.randn(N, H_kv, BS, D, generator=g, device=dev).to(torch.bfloat16)
                if kv != "bf16":
                    c = torch.empty(N, H_kv, BS, D, device=dev, dtype=torch.uint8)
                    rows_ = x.permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous()
                    ops.reshape_and_cache_fp8(rows_, rows_, c, torch.empty_like(c),
                                              torch.arange(N * BS, dtype=torch.int64, device=dev),
                                              scale8, scale8)
                    del rows_
                    x = c
                (kcs if len(kcs) < R else vcs).append(x)
            torch.cuda.synchronize()
            if kv == "bf16":
                def call(j):
                    ops.paged_attention_decode(q, kcs[j % R], vcs[j % R], btd, cld,
                                               max_context_len=max_ctx, out=out, workspace=ws)
            else:
                def call(j):
                    ops.paged_attention_decode_fp8(q, kcs[j % R], vcs[j % R], btd, cld, scale8,
                                                   scale8, max_context_len=max_ctx, out=out,
                                                   workspace=ws)
            alg = int(lens.sum()) * H_kv * D * e * 2
            # about 0.2 s of calls per point, at least 20, at most 200
            est = max(alg / 6e12, 8e-6)
            K = int(min(200, max(20, 0.2 / est)))
            t = graph_time_s(call, K)
            row = {"context": label, "seqs": S, "kv": "bf16" if kv == "bf16" else "fp8 e4m3",
                   "history_tokens": int(lens.sum()), "decode_us": t * 1e6, "alg_bytes": alg,
                   "achieved_gbps": alg / t / 1e9, "frac": alg / t / 1e9 / HBM_PEAK_GBPS,
                   "decode_tokens_per_s": S / t, "calls": K, "pool_replicas": R,
                   "kernel": kernel_label(S, H_kv, G, D, BS, max_ctx, q.dtype)}
            rows.append(row)
            print(json.dumps(row), flush=True)
            del kcs, vcs, x
            torch.cuda.empty_cache()
    if args.sweep_out:
        L = ["# Decode call over context length x batch (28/4 heads, head_dim 128, block "
             "size 16, bf16 queries)", "",
             "Command (repository root, one MI355X):", "",
             "    python bench.py --sweep-lengths --sweep-out <file>", "",
             "Each cell: decode-call time in us, and algorithmic KV bytes per second as % of "
             "8 TB/s.  Histories of L tokens each (rows), S sequences (columns); the last rows "
             "draw each history's length uniformly from the range named.", ""]
        seqs = sorted({r["seqs"] for r in rows})
        for kv in sorted({r["kv"] for r in rows}):
            L += ["## KV cache: %s" % kv, "",
                  "| L \\ S | " + " | ".join(str(x) for x in seqs) + " |",
                  "|---|" + "---|" * len(seqs)]
            labels = []
            for r in rows:
                if r["kv"] == kv and r["context"] not in labels:
                    labels.append(r["context"])
            for lab in labels:
                cells = []
                for sq in seqs:
                    m = [r for r in rows if r["kv"] == kv and r["context"] == lab and
                         r["seqs"] == sq]
                    cells.append("%.1f us, %.1f %%" % (m[0]["decode_us"], 100 * m[0]["frac"])
                                 if m else "")
                L.append("| %s | " % lab + " | ".join(cells) + " |")
            L.append("")
        L += ["Algorithmic bytes: history tokens x 4 KV heads x 128 x element bytes (2 for "
              "bf16, 1 for FP8) x 2 (K and V).  Timing: K decode calls replayed from a HIP "
              "graph (K = 20..200, about 0.2 s per point), HIP events around each replay, "
              "mean of 3.  Small calls are launch-bound: there the percentage says little."]
        with open(args.sweep_out, "w") as fh:
            fh.write("\n".join(L) + "\n")


def copy_blocks_rate(kcs, vcs, dev, pairs=2048, calls=8):
    """The copy-on-write block copy (pa_copy_blocks) on the same pools:
    `pairs` distinct (src, dst) blocks per call, a fresh set each call and
    the pool replicas in turn, so no call finds its blocks in the last-level
    cache.  Bytes moved = blocks read + blocks written, both caches."""
    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import ops

    N = kcs[0].shape[0]
    rng = np.random.default_rng(99)
    sets = []
    for _ in range(calls):
        perm = rng.permutation(N)[:2 * pairs].astype(np.int32)
        sets.append(torch.from_numpy(perm.reshape(2, pairs).T.copy()).to(dev))
    ops.copy_blocks(kcs[0], vcs[0], sets[0])                 # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(calls):
        ops.copy_blocks(kcs[k % len(kcs)], vcs[k % len(vcs)], sets[k])
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / calls
    block_bytes = kcs[0][0].numel() * kcs[0].element_size()
    moved = 2 * 2 * pairs * block_bytes
    return {"pairs_per_call": pairs, "bytes_moved_per_call": moved, "us_per_call": t * 1e6,
            "achieved_gbps": moved / t / 1e9, "frac": moved / t / 1e9 / HBM_PEAK_GBPS,
            "bound": "hbm"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_kv_decode_attention_amd import inputs as I
    from paged_kv_decode_attention_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.load_library()
    dev = torch.device("cuda:0")

    if args.sweep:
        shape_sweep(args, dev)
        return
    if args.sweep_lengths:
        length_sweep(args, dev)
        return

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            ops.copy_bytes(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    cfg = I.CONFIGS[args.config]
    inp = I.generate(cfg, new_tokens_at="last")
    S, H, D = inp.query.shape
    N, H_kv, BS, _ = inp.key_cache.shape
    W = inp.block_tables.shape[1]
    lens = inp.context_lens.numpy()
    alg_bytes = I.kv_bytes_read(cfg, lens)

    q = inp.query.to(dev)
    bt = inp.block_tables.to(dev)
    cl = inp.context_lens.to(dev)
    nk, nv = inp.new_key.to(dev), inp.new_value.to(dev)
    slots = inp.slot_mapping.to(dev)
    R = max(1, args.replicas)
    kcs = [inp.key_cache.to(dev) for _ in range(R)]
    vcs = [inp.value_cache.to(dev) for _ in range(R)]
    out = torch.empty_like(q)
    max_ctx = W * BS
    ws_bytes = ops.decode_workspace_size(S, H, H_kv, D, BS, max_ctx, args.partition_size,
                                         q.dtype)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    kind = {"auto": ops.KERNEL_AUTO, "generic": ops.KERNEL_GENERIC, "mfma": ops.KERNEL_MFMA}
    ops.select_kernel(kind[args.kernel])
    P = args.partition_size or ops.decode_partition_size(S, H_kv, H // H_kv, D, BS, max_ctx,
                                                         q.dtype)

    def step(k, ev=None, decode_only=args.decode_only):
        r = k % R
        if not decode_only and args.unfused:
            ops.reshape_and_cache(nk, nv, kcs[r], vcs[r], slots)
        if ev is not None:
            ev[0].record()
        if not decode_only and not args.unfused:
            # the cache write of each sequence's newest token, fused
            ops.decode_append(q, nk, nv, kcs[r], vcs[r], bt, cl, cfg.scale,
                              max_context_len=max_ctx, partition_size=args.partition_size,
                              out=out, workspace=ws)
        else:
            ops.paged_attention_decode(q, kcs[r], vcs[r], bt, cl, cfg.scale,
                                       max_context_len=max_ctx,
                                       partition_size=args.partition_size, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    def capture(body):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                body()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return g

    def timed_replay(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) * 1e-3

    if args.eager:
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(k, events[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dec_ms = np.array([s.elapsed_time(e) for s, e in events])
    else:
        g_step = capture(lambda: [step(k) for k in range(args.steps)])
        g_step.replay()          # untimed replay: first-launch costs out of the way
        wall, _ = timed_replay(g_step)
        del g_step
        # decode call duration: DECODE_CALLS back-to-back decode calls, HIP
        # events around each of 3 replays
        g_dec = capture(lambda: [step(k, decode_only=True) for k in range(args.decode_calls)])
        g_dec.replay()
        dec_ms = np.array([timed_replay(g_dec)[1] / args.decode_calls * 1e3 for _ in range(3)])
        del g_dec
    hot_us = None
    one_us = None
    if not args.decode_only:
        # hot-cache figure, labelled as such: every call reads the same pool
        # replica, so whatever of it the 256 MB last-level cache keeps is reused
        g_hot = capture(lambda: [step(k * R, decode_only=True) for k in range(args.decode_calls)])
        g_hot.replay()
        hot_us = timed_replay(g_hot)[1] / args.decode_calls * 1e6
        del g_hot
        # distribution of single decode calls: HIP events around each of 100
        # calls launched one by one (launch gaps excluded, each call timed alone)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(100)]
        for k in range(100):
            step(k, ev[k], decode_only=True)
        torch.cuda.synchronize()
        one_us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3

    # practical streaming-read ceiling of this GPU (hand-written kernel)
    rd = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(16 * 65536, dtype=torch.uint8, device=dev)
    ops.stream_read(rd, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        ops.stream_read(rd, sink)
    e1.record()
    torch.cuda.synchronize()
    ceiling_gbps = 5 * rd.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del rd

    # the other operations' figures (not in --decode-only runs, which the
    # hardware-counter passes profile)
    copy = fp8_kv = int8_kv = verify = None
    if not args.decode_only:
        copy = copy_blocks_rate(kcs, vcs, dev)
        verify = verify_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes, capture,
                             timed_replay)
        verify["q_len_2"] = verify_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes,
                                        capture, timed_replay, q_len=2)
        if cfg.dtype in ("bf16", "f16"):
            fp8_kv = q8_decode_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes,
                                    capture, timed_replay, "fp8")
            int8_kv = q8_decode_rate(args, cfg, q, bt, cl, kcs, vcs, max_ctx, dev, alg_bytes,
                                     capture, timed_replay, "int8")

    dec_s = float(dec_ms.mean()) * 1e-3
    achieved = alg_bytes / dec_s / 1e9
    traffic = load_traffic(args.config, alg_bytes)
    result = {
        "metric": METRIC,
        "value": S * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": "%s: Qwen-7B-shaped GQA decode" % cfg.name
                        if cfg.name == "qwen7b_gqa_bf16" else cfg.name,
            "num_seqs": S, "num_heads": H, "num_kv_heads": H_kv, "head_dim": D,
            "block_size": BS, "num_blocks": N, "max_blocks_per_seq": W,
            "context_lens": "%s %s, seed %d (min %d, mean %.1f, max %d)" % (
                cfg.lens_kind, list(cfg.lens_args), cfg.seed, lens.min(), lens.mean(),
                lens.max()),
            "partition_size": P if args.partition_size else "balanced schedule",
            "kernel": args.kernel, "kv_pool_replicas": R,
            "step": "decode only" if args.decode_only else (
                "reshape_and_cache + decode" if args.unfused
                else "decode_append (cache write of the newest token + decode)"),
            "launch": "eager" if args.eager else "hip graph of the K steps",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            # counter HBM bytes (the traffic figure) over the same duration
            "counter_gbps": traffic / dec_s / 1e9 if traffic else None,
            "kernel": "paged_attention_decode call (partition kernel + lse merge kernel)",
            "alg_bytes_per_launch": alg_bytes,
            "decode_us_mean": float(dec_ms.mean()) * 1e3,
            "decode_us_min": float(dec_ms.min()) * 1e3,
            "decode_us_max": float(dec_ms.max()) * 1e3,
            "decode_calls_per_replay": args.decode_calls,
            "single_call_us_p10_p50_p90": None if one_us is None else
                [float(np.percentile(one_us, p)) for p in (10, 50, 90)],
            "hot_cache_decode_us": hot_us,
            # rocprofv3 kernel-only durations (committed trace of this
            # command, current sources only), beside the event timings
            "rocprof_kernel_only": load_kernel_only(args.config, alg_bytes),
        },
        "decode_tokens_per_s": S / dec_s,
        "hbm_read_ceiling_gbps": ceiling_gbps,
        "frac_of_read_ceiling": achieved / ceiling_gbps,
        "copy_blocks": copy,
        "fp8_kv": fp8_kv,
        "int8_kv": int8_kv,
        "verify": verify,
        "kernel_src_sha": kernel_source_hash(),
    }
    if not args.decode_only and not args.no_workloads:
        del kcs, vcs
        torch.cuda.empty_cache()
        result["workloads"] = workload_rates(dev, capture, timed_replay,
                                             None if args.no_cpu_baseline else 1.5)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
