#!/usr/bin/env python3
"""Benchmark of the LSA decode hot path on one MI355X.

A step is one pass of the whole path over one batch: at t = 0 (mod 64) the
memory-indexer scan and the top-k re-selection, then the gathered-chunk GQA
decode attention; every step runs the attention.  The default workload is the
128K-context one: batch 16, 64 query / 8 KV heads, head dim 128, 131,072
tokens = 2,048 chunks of 64, 276 chunks (13.5%) retained, tau = 64.  Inputs
are seeded synthetic data (synth/), resident in HBM before timing starts.

Prints one JSON line (rank 0, N = 1):
  value        decode steps/s over exactly --steps steps (hipGraph replay)
  roofline     the attention kernel: algorithmic bytes per launch / its mean
               launch time, timed with HIP events on its own stream, against
               the 8 TB/s HBM peak
  cpu_baseline the CPU oracle (tests only otherwise) on a bounded sample of
               the same workload, on this host's cores

Other modes (used for profiling): --kernel-only (just the attention
launches), --copy-calibration (a plain device copy of known size, to scale
hardware byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
METRIC = "LSA decode steps/s + achieved HBM GB/s (fraction of peak), 128K ctx batch 16"


def metric_for(w) -> str:
    """The headline metric for the 128K workload; the same measure, named
    for its own context and batch, for the others."""
    if w.name == "128k":
        return METRIC
    return f"LSA decode steps/s + achieved HBM GB/s (fraction of peak), {w.name.upper()} ctx batch {w.B}"
KERNEL_SRC = os.path.join(ROOT, "lookahead_chunk_sparse_amd", "csrc", "gather_attend.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_128k_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attend_bytes_per_launch(w, seg: int = 0, k_eff: float | None = None) -> int:
    """Algorithmic HBM bytes of one attention launch: the retained K and V
    tiles of every (request, KV head) (k_eff chunks per request on average
    when selections vary in size, else k), the K and V rows of a resident
    segment of `seg` tokens per request if any, the bf16 queries, the fp32
    outputs and the chunk ids."""
    kv = int(w.B * w.Hkv * (w.k if k_eff is None else k_eff) * 2 * w.T * w.d * 2)
    sk = w.B * w.Hkv * seg * 2 * w.d * 2
    q = w.B * w.Hq * w.d * 2
    out = w.B * w.Hq * w.d * 4
    ids = w.B * w.k * 4
    return kv + sk + q + out + ids


def step_bytes(w, layers: int = 1, seg: int = 0, k_eff: float | None = None) -> int:
    """Algorithmic bytes of one decode step: one attention launch per layer
    plus the indexer scan (every key byte once, one scan shared by all
    layers) amortised over tau steps."""
    return layers * attend_bytes_per_launch(w, seg, k_eff) + (w.B * w.C * w.d_idx) // w.tau


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for_current_kernel(w):
    """HBM bytes per launch from the committed counter runs, if they were taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_sha() or t.get("workload") != w.name:
        return None
    return t.get("hbm_bytes_per_launch")


def setup(w, n_split: int, layers: int = 1, selection: str = "topk"):
    import torch

    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    dev = torch.device("cuda:0")
    t0 = time.time()
    K = torch.from_numpy(W.indexer_keys(w)).to(dev)
    ctx = torch.from_numpy(W.ctx_lens(w)).to(dev)
    kv = W.device_kv_store(w, dev)
    if layers > 1:  # further layers: the same synthetic recipe, each its own store
        stores = [kv] + [W.device_kv_store(w.replace(seed=w.seed + 1000 * l), dev) for l in range(1, layers)]
        dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=stores, n_split=n_split,
                         selection=selection, device=dev)
    else:
        dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, kv=kv, n_split=n_split,
                         selection=selection, device=dev)
    log(f"[bench] inputs placed in HBM in {time.time() - t0:.1f}s (K/V {layers * kv.numel() * 2 / 1e9:.2f} GB, "
        f"{layers} layer(s))")
    return dec


def make_queries(w, n_steps: int):
    import torch

    from synth import workloads as W
    dev = torch.device("cuda:0")
    q_all = torch.empty((n_steps, w.B, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    for t in range(n_steps):
        q_all[t].view(torch.int16).copy_(torch.from_numpy(W.attn_query(w, t).view("int16")))
    n_int = (n_steps + w.tau - 1) // w.tau
    qidx = [torch.from_numpy(W.indexer_query(w, i)).to(dev) for i in range(n_int)]
    return q_all, qidx


def enqueue_steps(dec, w, q_all, qidx, n_steps, out):
    L = len(dec.layers) if dec.layers is not None else 1
    for i in range((n_steps + w.tau - 1) // w.tau):
        ts = range(i * w.tau, min((i + 1) * w.tau, n_steps))
        if L == 1:
            dec.run_interval(i, qidx[i], [q_all[t] for t in ts], [out] * len(ts))
        else:  # layer l at step t uses query (t + 7 l) of the generated set: distinct per layer
            n_q = q_all.shape[0]
            dec.run_interval(i, qidx[i], [[q_all[(t + 7 * l) % n_q] for l in range(L)] for t in ts],
                             [[out] * L for _ in ts])


def capture(dec, w, q_all, qidx, n_steps, out):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        enqueue_steps(dec, w, q_all, qidx, min(n_steps, w.tau), out)  # eager warm-up of every call
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        enqueue_steps(dec, w, q_all, qidx, n_steps, out)
    return g


def graph_timed(fn, n: int, reps: int = 3):
    """Mean duration of one call fn(j) on the current stream: n calls captured
    in one hipGraph, replayed back to back, with HIP events on the replay
    stream around each of `reps` timed replays (after one untimed replay, so
    the stream is busy when each timed pair is recorded).  Returns (the
    median over the replays of replay time / n, every replay's per-call
    mean), in ms.  The GPU runs the captured calls one after the other, so
    the host's time to issue a call never enters, and one disturbed replay
    does not move the median."""
    import torch
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn(0)  # eager first call (library set-up outside the capture)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            fn(j)
    g.replay()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = [a.elapsed_time(b) / n for a, b in evs]
    return statistics.median(per_call), per_call


def time_attention_launches(dec, w, q_all, n_launches: int):
    """Mean duration of one attention call (split kernel + combine) on the
    stream it runs on, over n_launches calls replayed as one graph
    (graph_timed).  Returns (mean ms, min and max of the replays' means)."""
    import torch
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda:0")
    mean_ms, per = graph_timed(lambda j: dec.attend(q_all[j % q_all.shape[0]], 0, out), n_launches)
    return mean_ms, min(per), max(per)


def host_cores() -> int:
    """The host threads this process may use: OMP_NUM_THREADS where it is set
    (the machine's CPU share for this GPU), else the affinity mask's size."""
    return int(os.environ.get("OMP_NUM_THREADS", 0) or 0) or len(os.sched_getaffinity(0))


def _omp_threads(n: int | None):
    """Set the OpenMP thread count of the oracle's runtime (the libgomp the
    oracle library links); None restores host_cores()."""
    import ctypes
    gomp = ctypes.CDLL("libgomp.so.1")
    gomp.omp_set_num_threads(int(n) if n else host_cores())


def cpu_baseline(w, budget_s: float, threads: int | None = None):
    """The oracle on a bounded sample of the same workload: one re-selection
    (scan + top-k over every request) and full attention steps (all heads)
    over the first nb requests, nb chosen so a step fits the budget, repeated
    while the budget lasts.  steps/s is scaled to the whole batch
    (attention time x B/nb).  threads: OpenMP threads (None: every core of
    this process's affinity)."""
    import numpy as np

    import oracle
    from synth import workloads as W

    n_thr = threads or host_cores()
    oracle.lib()
    _omp_threads(n_thr)
    try:
        K = W.indexer_keys(w)
        q_idx = W.indexer_query(w, 0)
        t0 = time.perf_counter()
        _, _, ids = oracle.select(q_idx, K, w.k, w.alpha)
        t_sel = time.perf_counter() - t0
        ctx = W.ctx_lens(w)
        slots = np.tile(np.arange(w.k, dtype=np.int32), (w.B, 1))
        # one request first, to size the sample
        nb = 1
        kv_sel = np.stack([W.kv_chunks(w, b, ids[b]) for b in range(nb)])  # not timed: input placement
        q = W.attn_query(w, 0)
        t0 = time.perf_counter()
        oracle.gather_attend(q[:nb], kv_sel, ids[:nb], ctx[:nb], w.Hkv, w.sm_scale, slots=slots[:nb])
        t_one = time.perf_counter() - t0
        nb = int(max(1, min(w.B, (0.5 * budget_s) // max(t_one, 1e-6))))
        kv_sel = np.stack([W.kv_chunks(w, b, ids[b]) for b in range(nb)])
        t_att, n = 0.0, 0
        while n < 64 and (n == 0 or t_sel + t_att < budget_s):
            q = W.attn_query(w, n)
            t0 = time.perf_counter()
            oracle.gather_attend(q[:nb], kv_sel, ids[:nb], ctx[:nb], w.Hkv, w.sm_scale, slots=slots[:nb])
            t_att += time.perf_counter() - t0
            n += 1
    finally:
        _omp_threads(None)
    per_step = (t_att / n) * (w.B / nb) + t_sel / w.tau
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": n_thr, "kind": "oracle",
            "sample": (f"{w.name}: 1 re-selection (B={w.B}, C={w.C}) in {t_sel:.2f}s + {n} attention steps over "
                       f"{nb} of {w.B} requests (Hq={w.Hq}, k={w.k} chunks) in {t_att:.2f}s on {n_thr} thread(s); "
                       f"steps/s = 1/(attention s/step x {w.B}/{nb} + re-selection s/{w.tau})")}


def timed_runs(run, reps: int, stream=None):
    """Milliseconds of each of `reps` runs of run() (each one exactly the
    timed steps), HIP events on the stream the work goes to, with a full
    synchronisation before and after every run."""
    import torch
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def spread(ms: list) -> dict:
    """Median, min and max of repeated timings, and the spread max/min - 1."""
    return {"repeats": len(ms), "median_ms": round(statistics.median(ms), 5), "min_ms": round(min(ms), 5),
            "max_ms": round(max(ms), 5), "spread": round(max(ms) / min(ms) - 1.0, 4)}


def host_tier_bench(w, steps: int, warmup: int, fetch: str, fetch_grid: int, n_split: int = 0, delta=None,
                    stage_chunks: int = 1024):
    """The host-tier workload: the whole K/V in pinned host memory, selected
    chunks fetched into an HBM pool on a side stream every tau steps (lag 1,
    two pool buffers), attention on the pool.  Eager launches.  The timed
    steps continue after the warm-up intervals, so they show the steady state
    where each interval's fetch overlaps the previous selection's attention.
    Also reports each fetch method alone (HIP events on the side stream): the
    host-to-HBM bandwidth, PCIe-inclusive."""
    import torch

    from lookahead_chunk_sparse_amd import (alloc_fetch_staging, lsa_fetch_chunks, lsa_fetch_chunks_pull,
                                            lsa_fetch_chunks_staged)
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    dev = torch.device("cuda:0")
    t0 = time.time()
    K = torch.from_numpy(W.indexer_keys(w)).to(dev)
    ctx = torch.from_numpy(W.ctx_lens(w)).to(dev)
    host_kv = W.pinned_kv_store(w)
    dec = LsaDecoder(k_idx=K, ctx_len=ctx, Hq=w.Hq, k=w.k, alpha=w.alpha, host_kv=host_kv, fetch=fetch,
                     fetch_grid=fetch_grid, n_split=n_split, delta=delta, stage_chunks=stage_chunks, device=dev)
    log(f"[bench] pinned host K/V {host_kv.numel() * 2 / 1e9:.2f} GB placed in {time.time() - t0:.1f}s")
    n_warm_int = max(1, (warmup + w.tau - 1) // w.tau)
    n_time_int = max(1, steps // w.tau)
    q_all, qidx = make_queries(w, (n_warm_int + n_time_int) * w.tau)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)

    # each fetch method alone
    dec.reselect(qidx[0], 0)
    ids_d = dec.sel_ids[0]
    ids_h = ids_d.cpu()
    if dec.delta:  # selection 0 needs its pool slots before attention reads through them
        from lookahead_chunk_sparse_amd import lsa_pool_assign
        lsa_pool_assign(None, None, ids_d, 2 * w.k, new_slots=dec.sel_slots[0], fetch_slots=dec.fetch_slots[0])
    pool0 = dec.pool[0][:, :w.k]
    fetch_bytes = w.B * w.k * w.chunk_bytes

    def timed(fn, reps=3):
        ms = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(dec.side)
            fn()
            b.record(dec.side)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return statistics.median(ms[1:])

    pool0 = pool0.contiguous() if not pool0.is_contiguous() else pool0
    alone = {"memcpy": timed(lambda: lsa_fetch_chunks(host_kv, ids_h, pool0, stream=dec.side))}
    staging = dec.staging if dec.staging is not None else alloc_fetch_staging(host_kv, stage_chunks, device=dev)
    alone["staged"] = timed(lambda: lsa_fetch_chunks_staged(host_kv, ids_h, pool0, *staging, stream=dec.side))
    del staging
    for g in (8, 16, 64):
        alone[f"pull_grid{g}"] = timed(lambda: lsa_fetch_chunks_pull(host_kv, ids_d, pool0, grid=g,
                                                                     stream=dec.side))
    fetch_alone = {k: {"ms": round(v, 2), "GBs": round(fetch_bytes / (v * 1e-3) / 1e9, 1)} for k, v in alone.items()}
    mean_att, _, _ = time_attention_launches(dec, w, q_all, 50)

    def run(i0, n):
        for i in range(i0, i0 + n):
            ts = range(i * w.tau, (i + 1) * w.tau)
            dec.run_interval(i, qidx[i], [q_all[t] for t in ts], [out] * len(ts))

    run(0, n_warm_int)
    torch.cuda.synchronize()
    dec.fetch_events = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run(n_warm_int, n_time_int)
    end.record()
    dec.join()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    n_steps = n_time_int * w.tau
    # each timed interval's fetch, timed on the side stream while attention runs
    fetch_ms = [a.elapsed_time(b) for i, a, b in dec.fetch_events]
    dec.fetch_events = None
    # the chunks each interval's selection adds to the previous one (outside
    # the timed region): what a delta fetch moves over the host link
    sels = []
    for i in range(n_warm_int + n_time_int):
        dec.reselect(qidx[i], i)
        sels.append(dec.sel_ids[i % 2].cpu().numpy().copy())
    new_frac = [sum(len(set(sels[i][b].tolist()) - set(sels[i - 1][b].tolist())) for b in range(w.B)) / (w.B * w.k)
                for i in range(n_warm_int, n_warm_int + n_time_int)]
    moved = [(f if dec.delta else 1.0) * fetch_bytes for f in new_frac]
    link = [m / (t * 1e-3) / 1e9 for m, t in zip(moved, fetch_ms)] if len(fetch_ms) == len(moved) else []
    fetched = round(statistics.mean(new_frac), 4) if dec.delta else 1.0
    res = {
        "metric": "LSA host-tier decode steps/s, 1M ctx batch 4 (selected chunks fetched from pinned host memory)"
                  + (f", {round(100 * w.churn)}% new chunks per interval" if w.churn else ""),
        "value": round(1000.0 * n_steps / ms_total, 2), "unit": "steps/s", "n_gpus": 1, "steps": n_steps,
        "warmup": n_warm_int * w.tau, "ms_per_step": round(ms_total / n_steps, 5), "higher_is_better": True,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: batch {w.B}, {w.C} chunks of {w.T}, top-{w.k} fetched every {w.tau} "
                               f"steps into a two-buffer HBM pool (lag 1), steady state after the warm-up",
                   "fetch": fetch, "fetch_grid": fetch_grid or 16, "n_split": dec.n_split or "library default",
                   "delta_fetch": dec.delta, "churn_target": w.churn or None,
                   "fetched_fraction_per_interval": fetched,
                   "fetch_bytes_per_reselect_full": fetch_bytes,
                   "fetch_ms_under_overlap": round(statistics.mean(fetch_ms), 3) if fetch_ms else None,
                   "link_GBs_under_overlap": round(statistics.mean(link), 1) if link else None,
                   "fetch_alone": fetch_alone,
                   "attention_us_per_step_alone": round(mean_att * 1e3, 2),
                   "attention_GBs_alone": round(attend_bytes_per_launch(w) / (mean_att * 1e-3) / 1e9, 1),
                   "interval_ms": round(ms_total / n_time_int, 2)},
    }
    print(json.dumps(res), flush=True)


def gating_stats(dec, w, qidx) -> dict:
    """Sigmoid gating (sigma > 0.5, i.e. logit > 0) on this workload's
    indexer, outside any timed region: per interval and request, how many
    chunks pass before the cap, how many are kept (at most k), and how often
    the cap binds."""
    import torch

    from lookahead_chunk_sparse_amd import lsa_index_score, lsa_threshold_chunks
    passing, kept = [], []
    for i, q in enumerate(qidx):
        logits, _ = lsa_index_score(q, dec.k_idx, w.alpha, want_scores=False)
        _, n_all = lsa_threshold_chunks(logits.view(w.B, w.C), w.C, dec.logit_threshold)
        _, n_cap = lsa_threshold_chunks(logits.view(w.B, w.C), w.k, dec.logit_threshold)
        passing.append(n_all.cpu())
        kept.append(n_cap.cpu())
    passing, kept = torch.stack(passing).double(), torch.stack(kept).double()
    q = torch.tensor([0.0, 0.5, 1.0], dtype=torch.float64)
    return {"intervals": len(qidx), "requests": w.B, "cap": w.k, "chunks": w.C,
            "passing_min_median_max": [round(float(x), 1) for x in torch.quantile(passing.flatten(), q)],
            "passing_frac_of_chunks_mean": round(float(passing.mean()) / w.C, 4),
            "kept_min_median_max": [round(float(x), 1) for x in torch.quantile(kept.flatten(), q)],
            "kept_mean": round(float(kept.mean()), 2), "kept_mean_first_interval": round(float(kept[0].mean()), 2),
            "cap_binds_frac": round(float((passing > w.k).double().mean()), 4)}


def token_attend_bytes(w, k_tok: int) -> int:
    """Algorithmic HBM bytes of one token-list attention launch: the K and V
    rows of the k_tok listed tokens of every (request, KV head), the bf16
    queries, the fp32 outputs, the token list and the chunk ids."""
    kv = w.B * w.Hkv * k_tok * 2 * w.d * 2
    return kv + w.B * w.Hq * w.d * (2 + 4) + w.B * k_tok * 4 + w.B * w.k * 4


def token_stage_bench(w, steps: int, warmup: int, k_tok: int, n_split: int, repeats: int = 5):
    """Two-stage selection: chunks by the memory indexer every tau steps,
    then at every step the k_tok best tokens of the recalled chunks by a
    per-step token score (synthetic, bf16-rounded normals; the model's own
    token scorer is not on the path), attended over.  hipGraph replay of
    exactly `steps` steps after `warmup` steps."""
    import torch

    import synth
    from lookahead_chunk_sparse_amd import lsa_gather_attend_default_splits, lsa_topk_tokens
    from lookahead_chunk_sparse_amd.decode import LsaDecoder
    from synth import workloads as W

    dev = torch.device("cuda:0")
    t0 = time.time()
    dec = LsaDecoder(k_idx=torch.from_numpy(W.indexer_keys(w)).to(dev), ctx_len=torch.from_numpy(W.ctx_lens(w)).to(dev),
                     Hq=w.Hq, k=w.k, alpha=w.alpha, kv=W.device_kv_store(w, dev), n_split=n_split, token_topk=k_tok,
                     device=dev)
    n_pool = 16  # distinct per-step token-score tensors, used in turn
    pool = [torch.from_numpy(synth.bf16_bits_to_f32(synth.normal_bf16((w.B, w.k * 64), w.seed,
                                                                      synth.stream(synth.TAG_MISC, 5000 + i))))
            .to(dev) for i in range(n_pool)]
    log(f"[bench] inputs placed in HBM in {time.time() - t0:.1f}s")
    n_q = max(steps, warmup, w.tau)
    q_all, qidx = make_queries(w, n_q)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)

    def enqueue(n):
        for i in range((n + w.tau - 1) // w.tau):
            ts = range(i * w.tau, min((i + 1) * w.tau, n))
            dec.run_interval(i, qidx[i], [q_all[t] for t in ts], [out] * len(ts),
                             token_scores=[pool[t % n_pool] for t in ts])

    def graph(n):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            enqueue(min(n, w.tau))
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            enqueue(n)
        return g

    if warmup:
        graph(warmup).replay()
    g = graph(steps)
    ms_runs = timed_runs(g.replay, repeats)
    ms_per_step = statistics.median(ms_runs) / steps
    steps_s = 1000.0 / ms_per_step

    # the two per-step calls, each timed as 100 calls replayed in one graph
    dec.reselect(qidx[0], 0)
    ids = dec.sel_ids[0]

    def timed(fn, n=100):
        return graph_timed(fn, n)[0]

    topk_ms = timed(lambda j: lsa_topk_tokens(pool[j % n_pool], ids, dec.ctx_len, k_tok, tok=dec.tok,
                                              tok_counts=dec.tok_counts, workspace=dec.tok_workspace))
    lsa_topk_tokens(pool[0], ids, dec.ctx_len, k_tok, tok=dec.tok, tok_counts=dec.tok_counts,
                    workspace=dec.tok_workspace)
    from lookahead_chunk_sparse_amd import lsa_gather_attend
    att_ms = timed(lambda j: lsa_gather_attend(q_all[j % n_q], dec.kv, ids, dec.ctx_len, dec.sm_scale,
                                               workspace=dec.workspace, n_split=dec.n_split, out=out, tok=dec.tok,
                                               tok_counts=dec.tok_counts))
    a_bytes = token_attend_bytes(w, k_tok)
    achieved = a_bytes / (att_ms * 1e-3) / 1e9
    entries = (k_tok + 63) // 64
    splits = dec.n_split or lsa_gather_attend_default_splits(w.B, w.Hkv, entries)
    step_b = a_bytes + w.B * w.k * 64 * 4 + (w.B * w.C * w.d_idx) // w.tau  # + token scores read by the top-k
    print(json.dumps({
        "metric": metric_for(w), "value": round(steps_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": (f"{w.name} context decode, two-stage selection: batch {w.B}, {w.Hq} query / {w.Hkv} KV "
                         f"heads, head dim {w.d}, top-{w.k} of {w.C} chunks every {w.tau} steps, then the top "
                         f"{k_tok} of their {w.k * 64} tokens by a per-step token score"),
            "global_batch": w.B, "seq_len": w.N, "retained_chunks": w.k, "retained_tokens": k_tok,
            "n_split": splits, "tokens_per_s": round(steps_s * w.B, 1),
            "timing": f"hipGraph replay of all steps; value from the median of {repeats} timed runs of exactly "
                      f"{steps} steps", "timed_runs": spread(ms_runs),
            "step_bytes": step_b, "step_GBs": round(step_b * steps_s / 1e9, 1),
            "token_topk_us": round(topk_ms * 1e3, 2), "token_attend_us": round(att_ms * 1e3, 2),
        },
        "roofline": {"bound": "hbm", "kernel": "gather-attend over listed tokens (split kernel + combine)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": a_bytes,
                     "mean_launch_us": round(att_ms * 1e3, 2),
                     "launch_timing": "HIP events on the launch stream around replays of one graph of 100 "
                                      "attention calls; median of 3 replays' per-call means"},
    }), flush=True)


def copy_bandwidth(n_bytes: int = 1 << 30, reps: int = 20) -> float:
    """GB/s of a plain device copy (torch's copy kernel) of n_bytes, counting
    the bytes read and the bytes written, event-timed over reps copies."""
    import torch
    a = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        b.copy_(a)
    end.record()
    torch.cuda.synchronize()
    gbs = 2 * n_bytes * reps / (start.elapsed_time(end) * 1e-3) / 1e9
    del a, b
    return gbs


def read_ceiling(kv, tile_bytes: int = 16384, n_read: int = 1 << 30) -> dict:
    """Best read bandwidth of randomly placed whole tiles of `kv` (the K/V
    store itself, tiles of one (chunk, K|V, head)): the attention's access
    pattern without its arithmetic, with the measurement-only kernel of
    libtileread.so, over a few grid / unroll shapes."""
    import ctypes

    import torch

    from lookahead_chunk_sparse_amd import build as B
    if not os.path.exists(B.MEASURE_LIB_PATH):
        raise ImportError(f"{B.MEASURE_LIB_PATH} is not built")
    L = ctypes.CDLL(B.MEASURE_LIB_PATH)
    L.lsa_measure_tile_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_all = kv.numel() * kv.element_size() // tile_bytes
    n_tiles = min(n_all, n_read // tile_bytes)
    g = torch.Generator().manual_seed(0)
    off = (torch.randperm(n_all, generator=g)[:n_tiles].to(torch.int64) * (tile_bytes // 16)).to(kv.device)
    assert int(off.max()) + tile_bytes // 16 <= kv.numel() * kv.element_size() // 16  # every tile inside the store
    stream = torch.cuda.current_stream()
    best = (0.0, None)
    for grid in (512, 1024, 2048):
        sink = torch.empty(grid * 256, dtype=torch.int32, device=kv.device)
        for unroll in (2, 4):
            args = (kv.data_ptr(), off.data_ptr(), n_tiles, tile_bytes // 16, sink.data_ptr(), grid, unroll,
                    stream.cuda_stream)
            if L.lsa_measure_tile_read(*args) != 0:
                raise RuntimeError("tile-read launch failed")
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(10):
                L.lsa_measure_tile_read(*args)
            end.record(stream)
            torch.cuda.synchronize()
            gbs = n_tiles * tile_bytes * 10 / (start.elapsed_time(end) * 1e-3) / 1e9
            if gbs > best[0]:
                best = (gbs, (grid, unroll))
    return {"GBs": round(best[0], 1), "tile_bytes": tile_bytes, "grid": best[1][0], "unroll": best[1][1]}


def copy_calibration(n_bytes: int, reps: int):
    """A plain device-to-device copy of known size (for counter scaling)."""
    import torch
    a = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n_bytes, "copy_calibration_bytes_written": n_bytes,
                      "reps": reps}))


def score_sweep(nqs, C: int, d_idx: int, launches: int):
    """Batched indexer scoring: nq query rows sharing one key set of C chunks.
    Times the int8-MFMA kernel and the GEMV kernel on the same shapes
    (selected through the library's dispatch threshold), and torch's fill of
    the same output bytes as the write rate they are held to."""
    import torch

    import lookahead_chunk_sparse_amd as lsa
    from synth import TAG_MISC, stream, uniform_i8
    dev = torch.device("cuda:0")
    K = torch.from_numpy(uniform_i8((1, C, d_idx), 0, stream(TAG_MISC, 1), -16, 15)).to(dev)
    for nq in nqs:
        q = torch.from_numpy(uniform_i8((1, nq, d_idx), 0, stream(TAG_MISC, 2), -16, 15)).to(dev)
        logits = torch.empty((1, nq, C), dtype=torch.int32, device=dev)
        scores = torch.empty((1, nq, C), dtype=torch.float32, device=dev)
        row = {"nq": nq, "C": C, "d_idx": d_idx}
        for path, thr in (("gemv", 1000000000), ("mfma", 1)):
            lsa.lsa_set_tuning("score_mfma_min_nq", thr)
            for _ in range(5):
                lsa.lsa_index_score(q, K, 1.0 / (16 * d_idx), logits=logits, scores=scores)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            for _ in range(launches):
                lsa.lsa_index_score(q, K, 1.0 / (16 * d_idx), logits=logits, scores=scores)
            e.record()
            torch.cuda.synchronize()
            us = s.elapsed_time(e) * 1e3 / launches
            ops = 2.0 * nq * C * d_idx
            byts = C * d_idx + nq * d_idx + nq * C * 8
            row[path] = {"us": round(us, 2), "TOPS": round(ops / us / 1e6, 2), "GBs": round(byts / us / 1e3, 1)}
        lsa.lsa_set_tuning("score_mfma_min_nq", 0)
        # the write ceiling for these outputs: a device fill of the same bytes
        for _ in range(5):
            logits.fill_(0)
            scores.fill_(0)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(launches):
            logits.fill_(0)
            scores.fill_(0)
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1e3 / launches
        row["fill_outputs"] = {"us": round(us, 2), "GBs": round(nq * C * 8 / us / 1e3, 1)}
        row["int8_peak_TOPS"] = 5000.0
        print(json.dumps(row), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="128k")
    ap.add_argument("--n-split", type=int, default=0, help="attention splits per (request, KV head); 0 = library")
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="attention calls per timed graph replay (the dominant kernel's timing)")
    ap.add_argument("--repeats", type=int, default=5, help="timed runs of exactly --steps steps (median reported)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the all-core cpu_baseline (the 1-thread one gets 0.6x)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--kernel-only", action="store_true", help="only the timed attention calls")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--token-topk", type=int, default=0, metavar="K_TOK",
                    help="two-stage selection: attend over the K_TOK best tokens of the recalled chunks")
    ap.add_argument("--layers", type=int, default=1, help="layers sharing one selection (HBM-resident only)")
    ap.add_argument("--selection", default="topk", choices=("topk", "threshold"),
                    help="chunk selection: top-k, or sigmoid gating (sigma > 0.5) capped at k")
    ap.add_argument("--segment", type=int, default=0, metavar="S",
                    help="resident tokens per request (local window, decoded tokens, compressed entries) "
                         "attended in the same softmax as the recalled chunks (HBM-resident, one layer)")
    ap.add_argument("--fetch", default="staged", choices=("pull", "memcpy", "staged"),
                    help="host-tier fetch: DMA copies over the library's copy streams (memcpy), the same through a "
                         "host-gathered staging buffer (staged), or the device gather (pull)")
    ap.add_argument("--fetch-grid", type=int, default=0, help="workgroups of the pull fetch (0 = 16)")
    ap.add_argument("--stage-chunks", type=int, default=1024,
                    help="staged fetch: chunks of each staging buffer (two halves, one copy each)")
    ap.add_argument("--no-delta", action="store_true", help="host tier: re-fetch every selected chunk")
    ap.add_argument("--drift", action="store_true", help="host tier: a fresh indexer query every interval")
    ap.add_argument("--churn", type=float, default=0.0,
                    help="host tier: the ring indexer, whose selection moves by about this fraction per interval")
    ap.add_argument("--score-sweep", action="store_true",
                    help="batched indexer scoring: MFMA vs GEMV kernel over nq (one key set)")
    ap.add_argument("--score-nq", default="1,2,4,8,16,32,64,128,256,512",
                    help="query rows for --score-sweep (comma list)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode path here has no multi-GPU "
              "mode (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 20)
        return
    if args.score_sweep:
        import lookahead_chunk_sparse_amd  # noqa: F401
        score_sweep([int(x) for x in args.score_nq.split(",")], 16384, 128, 50)
        return

    import lookahead_chunk_sparse_amd  # noqa: F401  (fails loudly if liblsa.so is missing)
    from synth import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.drift:
        w = w.replace(drift=True, n_golden=min(w.n_golden, w.C // max(1, (args.steps + args.warmup) // w.tau + 1)))
    if args.churn:
        if not w.host_tier:
            print("--churn applies to the host tier (--workload 1m_host)", file=sys.stderr)
            sys.exit(2)
        w = w.replace(churn=args.churn)
    if args.token_topk:
        token_stage_bench(w, args.steps, args.warmup, args.token_topk, args.n_split, args.repeats)
        return
    if w.host_tier:
        host_tier_bench(w, args.steps, args.warmup, args.fetch, args.fetch_grid, args.n_split,
                        False if args.no_delta else None, stage_chunks=args.stage_chunks)
        return
    dec = setup(w, args.n_split, args.layers, args.selection)
    if args.segment:
        if args.layers != 1:
            print("--segment runs with one layer", file=sys.stderr)
            sys.exit(2)
        # synthetic resident tokens: seeded normals, every request's segment full
        gen = torch.Generator(device="cuda:0").manual_seed(w.seed + 77)
        dec.seg_kv = torch.randn((w.B, 2, w.Hkv, args.segment, w.d), generator=gen, device="cuda:0",
                                 dtype=torch.float32).to(torch.bfloat16)
        dec.seg_len = torch.full((w.B,), args.segment, dtype=torch.int32, device="cuda:0")
    n_q = max(args.steps, args.warmup, w.tau)
    q_all, qidx = make_queries(w, n_q)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda:0")
    from lookahead_chunk_sparse_amd import lsa_gather_attend_default_splits
    splits = args.n_split or lsa_gather_attend_default_splits(w.B, w.Hkv, w.k)

    if args.kernel_only:
        dec.reselect(qidx[0], 0)
        mean_ms, lo_ms, hi_ms = time_attention_launches(dec, w, q_all, args.kernel_launches)
        gbs = attend_bytes_per_launch(w, args.segment) / (mean_ms * 1e-3) / 1e9
        print(json.dumps({"kernel": "attend_split_kernel<128>+combine", "workload": w.name, "n_split": splits,
                          "launches": args.kernel_launches, "mean_ms": mean_ms, "replay_means_ms": [lo_ms, hi_ms],
                          "achieved_GBs": gbs}))
        return

    # ---- warm-up: W untimed steps ----
    if args.eager:
        if args.warmup:
            enqueue_steps(dec, w, q_all, qidx, args.warmup, out)
    else:
        if args.warmup:
            g_w = capture(dec, w, q_all, qidx, args.warmup, out)
            g_w.replay()
        g = capture(dec, w, q_all, qidx, args.steps, out)
    torch.cuda.synchronize()

    # ---- timed: exactly K steps, in each of --repeats runs ----
    t_wall = time.perf_counter()
    if args.eager:
        ms_runs = timed_runs(lambda: enqueue_steps(dec, w, q_all, qidx, args.steps, out), args.repeats)
    else:
        ms_runs = timed_runs(g.replay, args.repeats)
    t_wall = time.perf_counter() - t_wall
    ms_total = statistics.median(ms_runs)
    ms_per_step = ms_total / args.steps
    steps_s = 1000.0 / ms_per_step
    log(f"[bench] {args.repeats} runs of {args.steps} steps: median {ms_total:.3f} ms, min {min(ms_runs):.3f}, "
        f"max {max(ms_runs):.3f} (wall {t_wall * 1e3:.1f} ms for all runs)")

    gating = gating_stats(dec, w, qidx[:(args.steps + w.tau - 1) // w.tau]) if args.selection == "threshold" else None
    k_step = gating["kept_mean"] if gating else None  # chunks attended per request and step, on average

    # ---- the dominant kernel, timed with events on its own stream (interval 0's selection) ----
    dec.reselect(qidx[0], 0)
    mean_ms, lo_ms, hi_ms = time_attention_launches(dec, w, q_all, args.kernel_launches)
    a_bytes = attend_bytes_per_launch(w, args.segment, gating["kept_mean_first_interval"] if gating else None)
    achieved = a_bytes / (mean_ms * 1e-3) / 1e9
    log(f"[bench] attention call, {args.kernel_launches} calls replayed as one graph: mean {mean_ms * 1e3:.1f} us "
        f"(replays {lo_ms * 1e3:.1f}-{hi_ms * 1e3:.1f}), {achieved:.0f} GB/s algorithmic")
    traffic = traffic_for_current_kernel(w) if not args.segment else None  # counters: no segment
    copy_gbs = copy_bandwidth()
    log(f"[bench] device copy (torch, 1 GiB, read + write bytes): {copy_gbs:.0f} GB/s")
    ceiling = read_ceiling(dec.kv)
    log(f"[bench] read ceiling, random 16 KB tiles of the K/V store: {ceiling['GBs']:.0f} GB/s")

    sb = step_bytes(w, args.layers, args.segment, k_step)
    layer_txt = "one layer" if args.layers == 1 else f"{args.layers} layers sharing one selection"
    if args.segment:
        layer_txt += f", plus {args.segment} resident tokens per request in the same softmax"
    result = {
        "metric": metric_for(w),
        "value": round(steps_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name} context decode, {layer_txt}: batch {w.B}, {w.Hq} query / {w.Hkv} KV heads, "
                         f"head dim {w.d}, {w.N} tokens = {w.C} chunks of {w.T}, "
                         + (f"top-{w.k} chunks" if args.selection == "topk"
                            else f"the chunks with sigmoid score > 0.5, at most {w.k},")
                         + f" re-selected every {w.tau} steps, int8 indexer dim {w.d_idx}"),
            "global_batch": w.B,
            "seq_len": w.N,
            "retained_chunks": w.k,
            "resident_segment_tokens": args.segment,
            "n_split": splits,
            "timing": ("eager launches" if args.eager else "hipGraph replay of all steps")
                      + f"; value from the median of {args.repeats} timed runs of exactly {args.steps} steps",
            "timed_runs": spread(ms_runs),
            "tokens_per_s": round(steps_s * w.B, 1),
            "step_bytes": sb,
            "step_GBs": round(sb * steps_s / 1e9, 1),
            "step_frac_of_hbm_peak": round(sb * steps_s / 1e9 / HBM_PEAK_GBS, 4),
            "copy_GBs": round(copy_gbs, 1),
            "step_frac_of_copy": round(sb * steps_s / 1e9 / copy_gbs, 4),
            "read_ceiling_GBs": ceiling["GBs"],
            "read_ceiling": f"random {ceiling['tile_bytes'] // 1024} KB tiles of the K/V store, "
                            f"grid {ceiling['grid']}, unroll {ceiling['unroll']}",
            "attention_frac_of_read_ceiling": round(achieved / ceiling["GBs"], 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gather-attend (split kernel + combine)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": a_bytes,
            "mean_launch_us": round(mean_ms * 1e3, 2),
            "launch_timing": f"HIP events on the launch stream around replays of one graph of "
                             f"{args.kernel_launches} attention calls; median of 3 replays' per-call means",
        },
    }
    if args.selection == "threshold":
        result["metric"] = metric_for(w) + ", sigmoid gating capped at k"
        result["config"]["selection"] = "sigmoid gating: logit > 0 (sigma > 0.5), at most k chunks"
        result["config"]["gating"] = gating
        log(f"[bench] gating: {gating}")
    if not args.no_cpu_baseline and not args.segment and args.selection == "topk":  # the oracle sample has no segment
        log("[bench] timing the CPU oracle on a bounded sample (all cores, then 1 thread) ...")
        cb = cpu_baseline(w, args.cpu_budget)
        cb["single_thread"] = cpu_baseline(w, 0.6 * args.cpu_budget, threads=1)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
