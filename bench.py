#!/usr/bin/env python3
"""Throughput of the LSA decode hot path on one MI355X.

A step is one call of lsa_decode_step over the whole batch: chunk scoring,
top-k selection (re-done every `reindex_every` steps), the gather into the
resident pool when the workload keeps one, split-KV sparse attention and the
log-sum-exp merge.  Inputs are seeded synthetic data already resident in HBM.

By default each step reads a different copy ("replica") of the workload's
embeddings and K/V history, cycling through enough copies that the cycle is
more than twice the 256 MB last-level (Infinity) cache: every step streams its
bytes from HBM instead of re-reading what the previous step left in cache.
`--replicas 1` gives the cache-assisted figure.

Prints one JSON line (rank 0, one GPU).  `value` is decode steps per second
(K steps issued eagerly between two events; `graph_ms_per_step` is the same
steps replayed from a HIP graph); `roofline` reports the attention phase's
algorithmic bytes per call over its average duration: K cold calls of
lsa_sparse_decode_attn (the split-KV partial kernel and the log-sum-exp
merge, or the one kernel that merges in its last workgroups) replayed from a
HIP graph between two events, with the partial kernel alone beside it
(`partial_kernel_us`); `score_kernel` does the same for the score kernel;
`cpu_baseline` times the CPU oracle on the host on a bounded sample of the
same workload.  `--attention-only` times just the attention phase (for a
kernel trace holding only its launches); `--mode` selects the retriever,
residency, append, scorer, copy and read measurements.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20     # MI355X Infinity Cache
DEFAULT_CONFIG = "cfg2"

WORKLOAD_TEXT = {
    "cfg1": "1 stream x 4096 tokens, chunk 64 (N=64), D=64, k=8, MQA 8 heads x d64, fp32",
    "cfg2": "16 streams x 131072 tokens, chunk 64 (N=2048), D=128, k=276 (13.5%), "
            "MQA 16 heads x d128, bf16",
    "cfg3": "4 streams x 524288 tokens, chunk 64 (N=8192), D=128, k=819 (10%), "
            "MQA 32 heads x d128, bf16, re-index every 64 steps via a resident pool",
    "cfg4": "1 stream x 1048576 tokens, chunk 128 (N=8192), D=256, k=655 (8%), "
            "absorbed MLA 64 heads, d_qk 576 / d_v 512, bf16",
    "cfg5": "32 streams x U{8192..262144} tokens, chunk 64, D=128, k=ceil(13.5%), "
            "MQA 16 heads x d128, bf16",
}


def algorithmic_bytes(w):
    """Bytes the method must move per step, by phase (split partials excluded)."""
    import numpy as np

    c = w.cfg
    es = 2 if c.dtype == "bf16" else 4
    C = c.chunk_size
    n_total = int(w.chunk_off[-1])
    k_total = int(w.sel_off[-1])
    score = n_total * c.index_dim * es + c.batch * c.index_dim * es + n_total * 4
    select = n_total * 4 + k_total * 4
    # kept tokens: full chunks, except a kept partial last chunk (upper bound
    # computed with the needles' and the last chunk's positions is not known
    # before selection; the bench adds the exact count from the GPU's selection)
    row = (c.head_dim_qk + (0 if c.v_aliases_k else c.head_dim_v)) * es
    q = c.batch * c.num_q_heads * c.head_dim_qk * es
    o = c.batch * c.num_q_heads * (c.head_dim_v + 1) * 4
    return dict(score=score, select=select, row=row, q=q, o=o, C=C, k_total=k_total)


def kept_tokens(w, sel):
    """Valid tokens of the kept chunks (a kept partial last chunk counts its
    valid rows only)."""
    import numpy as np

    C = w.cfg.chunk_size
    total = 0
    for b in range(w.B):
        n = sel[w.sel_off[b]:w.sel_off[b + 1]].astype(np.int64)
        total += int(np.minimum(C, w.lengths[b] - n * C).sum())
    return total


def load_traffic(kernel_file, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    from learned_kv_chunk_amd.profiling import kernel_sources, source_hash

    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_hash(kernel_sources(kernel_file)):
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, seconds, reindex_every):
    from oracle import oracle

    threads = max(1, len(os.sched_getaffinity(0)))
    c = w.cfg
    # one step on a single thread first (about a second at 16 x 128K)
    t1 = time.perf_counter()
    s1 = oracle.score(w.q_idx, w.emb, w.chunk_off)
    sel1 = oracle.select(s1, w.chunk_off, w.sel_off)
    oracle.attention(w.queries(0), w.K, w.V, w.tok_off, sel1, w.sel_off, c.chunk_size,
                     c.softmax_scale, dv=c.head_dim_v, nthreads=1)
    single = 1.0 / (time.perf_counter() - t1)
    steps = 0
    t0 = time.perf_counter()
    sel = None
    while True:
        if steps % reindex_every == 0:
            s = oracle.score(w.q_idx, w.emb, w.chunk_off)
            sel = oracle.select(s, w.chunk_off, w.sel_off)
        oracle.attention(w.queries(steps % 4), w.K, w.V, w.tok_off, sel, w.sel_off,
                         c.chunk_size, c.softmax_scale, dv=c.head_dim_v, nthreads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": steps / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full decode step(s) of the same workload (all {c.batch} "
                      f"streams, score + select + attention, re-index every {reindex_every}) "
                      f"in {el:.1f} s, fp64 C oracle with OpenMP over (stream, head)",
            "single_thread_steps_per_s": single, "cpu_model": cpu_model()}


def run_copy(args):
    import torch

    from learned_kv_chunk_amd import lsa

    nbytes = args.copy_mib * 2 ** 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    lsa.bench_flush(src)
    for _ in range(3):
        lsa.bench_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        lsa.bench_copy(dst, src, nbytes)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"mode": "copy", "bytes_per_launch": 2 * nbytes, "read_bytes": nbytes,
                      "write_bytes": nbytes, "us_per_launch": us,
                      "gbs": 2 * nbytes / us / 1e3}), flush=True)


def run_read(args):
    """Streams --copy-mib MiB through lsa_bench_read in access pattern
    --read-pattern (0 plain, 1 non-temporal, 2 the MQA K operand pattern):
    the reference of the HBM read counters for each pattern."""
    import torch

    from learned_kv_chunk_amd import lsa

    nbytes = args.copy_mib * 2 ** 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(lsa.BENCH_READ_SINK_BYTES, dtype=torch.uint8, device="cuda")
    lsa.bench_flush(src)
    for _ in range(3):
        lsa.bench_read(src, nbytes, args.read_pattern, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        lsa.bench_read(src, nbytes, args.read_pattern, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"mode": "read", "pattern": args.read_pattern, "read_bytes": nbytes,
                      "us_per_launch": us, "gbs": nbytes / us / 1e3}), flush=True)


def run_scorer(args):
    """Times lsa_score_fp8_multihead (the released retriever's multi-head scorer
    over float8 compressed-key records) on the chunks of a workload, cold: each
    launch reads a different copy of the records."""
    import numpy as np
    import torch

    from learned_kv_chunk_amd import device as dev
    from learned_kv_chunk_amd import lsa
    from learned_kv_chunk_amd import workloads as wl
    from oracle import oracle

    cfg = wl.CONFIGS[args.config]
    w = wl.make_workload(cfg)
    heads, head_dim = 128, 128
    q_bits, hw, rec = wl.make_mh_inputs(w, heads=heads, head_dim=head_dim)
    shape = dev.problem_shape(w)
    qd = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(hw).cuda()
    co = torch.from_numpy(w.chunk_off).cuda()
    scores = torch.empty(shape.total_chunks, dtype=torch.float32, device="cuda")
    n_total = int(w.chunk_off[-1])
    launch_bytes = rec.nbytes + q_bits.nbytes + hw.nbytes + 4 * n_total
    reps = args.replicas or max(1, math.ceil(2 * MALL_BYTES / launch_bytes) + 1)
    recs = [torch.from_numpy(rec).cuda() for _ in range(min(reps, 256))]
    reps = len(recs)
    for r in recs[:3]:
        lsa.score_fp8_multihead(shape, qd, wd, r, co, scores)
    torch.cuda.synchronize()
    # a launch takes a few microseconds of device time, less than the host
    # needs to issue it through the binding: the K timed launches are replayed
    # from a HIP graph, so that the events see device time only
    us = _graph_us(lambda i: lsa.score_fp8_multihead(shape, qd, wd, recs[i % reps], co, scores),
                   args.steps)
    flops = 2.0 * n_total * heads * head_dim
    line = {
        "metric": "fp8 multi-head chunk scoring: records scored per second",
        "value": n_total / us * 1e6, "unit": "records/s", "n_gpus": 1, "steps": args.steps,
        "warmup": 3, "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 keys, bf16 queries, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{args.config} chunks: {n_total} records of {head_dim + 4} B, "
                               f"{heads} heads x {head_dim}", "replicas": reps,
                   "timing": "HIP graph of the timed launches, replayed once"},
        "roofline": {"kernel": "score_mh_kernel", "bound": "hbm",
                     "achieved": launch_bytes / us / 1e3, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": launch_bytes / us / 1e3 / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": launch_bytes, "avg_launch_us": us,
                     "mfma_tflops": flops / us / 1e6},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        threads = max(1, len(os.sched_getaffinity(0)))
        t0 = time.perf_counter()
        calls = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.score_fp8mh(q_bits, hw, rec, w.chunk_off)
            calls += 1
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": calls * n_total / el, "unit": "records/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{calls} full scoring pass(es) of all {n_total} records "
                                          f"in {el:.1f} s, single-threaded fp64 C oracle "
                                          f"({threads} cores available)"}
    print(json.dumps(line), flush=True)


def _graph_us(fn, n, warm=1):
    """Average device time of fn(i), i = 0..n-1, captured once in a HIP graph
    and replayed (the captured calls allocate and clear nothing); `warm`
    untimed replays first."""
    import torch

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fn(i)
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def run_retriever(args):
    """Times the retriever-side decode step: the three-layer ensemble of the
    float8 multi-head scorer (max), the threshold keep set with its dense
    fallback, and sparse attention over the kept set the device produced.
    Cold: each step reads a different copy of the records and of the K/V
    history.  The steps are captured once in a HIP graph and replayed, so the
    host's issue rate (four binding calls per step) is not measured."""
    import numpy as np
    import torch

    from learned_kv_chunk_amd import device as dev
    from learned_kv_chunk_amd import lsa
    from learned_kv_chunk_amd import workloads as wl

    cfg = wl.CONFIGS[args.config]
    layers, heads, head_dim, keep = 3, 128, 128, 0.135
    w = wl.make_workload(cfg)
    q, hw, rec = wl.make_mh_layer_inputs(w, layers=layers, heads=heads, head_dim=head_dim)
    base = dev.upload(w, "cuda")
    shape = dev.problem_shape(w)
    shape.max_k = shape.max_chunks        # the kept counts are known on the device only
    shape.total_k = shape.total_chunks
    shape.uniform = False
    B, n_total = w.B, int(w.chunk_off[-1])
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(hw).cuda()
    co = base.chunk_off
    scores = torch.empty(n_total, dtype=torch.float32, device="cuda")
    sel_off = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    sel_idx = torch.empty(n_total, dtype=torch.int32, device="cuda")
    fb = torch.empty(B, dtype=torch.int32, device="cuda")
    tws = torch.empty(lsa.select_threshold_workspace_bytes(shape), dtype=torch.uint8,
                      device="cuda")
    out = torch.empty_like(base.out)
    lse = torch.empty_like(base.lse)
    aws = lsa.allocate_workspace(shape, "cuda")
    rec0 = torch.from_numpy(rec).cuda()

    # the threshold: the fp32 score at the (1 - keep) quantile of an untimed
    # scoring pass, so that about `keep` of all chunks pass
    lsa.score_fp8_multihead_layers(shape, qd, wd, rec0, co, lsa.COMBINE_MAX, scores)
    torch.cuda.synchronize()
    s_host = dev.to_host(scores)
    tau = float(np.float32(np.quantile(s_host, 1.0 - keep)))
    lsa.select_threshold(shape, scores, co, tau, 0, sel_off, sel_idx, fb, tws)
    torch.cuda.synchronize()
    off_h = dev.to_host(sel_off)
    idx_h = dev.to_host(sel_idx)[:int(off_h[-1])]
    C = cfg.chunk_size
    ktok = 0
    for b in range(B):
        n = idx_h[off_h[b]:off_h[b + 1]].astype(np.int64)
        ktok += int(np.minimum(C, w.lengths[b] - n * C).sum())
    ab = algorithmic_bytes(w)
    score_bytes = rec.nbytes + q.nbytes + hw.nbytes + 4 * n_total
    thr_bytes = 2 * 4 * n_total + 4 * int(off_h[-1]) + 4 * (2 * B + 1)
    attn_bytes = ktok * ab["row"] + ab["q"]
    step_bytes = score_bytes + thr_bytes + attn_bytes + ab["o"]

    reps = args.replicas or max(1, math.ceil(2 * MALL_BYTES / step_bytes) + 1)
    recs = [rec0] + [rec0.clone() for _ in range(reps - 1)]
    Ks = [base.K] + [base.K.clone() for _ in range(reps - 1)]
    Vs = [base.V] + [None if base.V is None else base.V.clone() for _ in range(reps - 1)]
    nq = 8
    qs = [base.queries(t) for t in range(nq)]
    torch.cuda.synchronize()

    def score(i):
        lsa.score_fp8_multihead_layers(shape, qd, wd, recs[i % reps], co, lsa.COMBINE_MAX, scores)

    def select(i):
        lsa.select_threshold(shape, scores, co, tau, 0, sel_off, sel_idx, fb, tws)

    def attend(i):
        lsa.sparse_decode_attn(shape, qs[i % nq], Ks[i % reps], Vs[i % reps], base.tok_off,
                               sel_idx, sel_off, lsa.KV_STORE, out, lse, aws)

    def step(i):
        score(i)
        select(i)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    us_step = _graph_us(step, args.steps)
    us_score = _graph_us(score, args.steps)
    us_select = _graph_us(select, args.steps)
    us_attend = _graph_us(attend, args.steps)
    score_gbs = score_bytes / us_score / 1e3
    line = {
        "metric": "retriever decode steps/sec at 128K ctx (3-layer fp8 multi-head score + "
                  "threshold keep + sparse attn)",
        "value": 1e6 / us_step, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us_step / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8 keys + bf16 KV, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}; {layers} layers of "
                               f"{n_total} compressed-key records ({heads} heads x {head_dim}), "
                               f"max ensemble, threshold at the {1 - keep:.3f} score quantile",
                   "threshold": tau, "kept_chunks": int(off_h[-1]),
                   "kept_fraction": int(off_h[-1]) / n_total,
                   "fallback_streams": int(dev.to_host(fb).sum()), "replicas": reps,
                   "timing": "HIP graph of the timed steps, replayed once"},
        "phase_us": {"ensemble_score": us_score, "threshold_select": us_select,
                     "attention_and_merge": us_attend},
        "step_algorithmic_bytes": int(step_bytes),
        "roofline": {"kernel": "score_mh_kernel (3-layer ensemble)", "bound": "hbm",
                     "achieved": score_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": score_gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": int(score_bytes),
                     "avg_launch_us": us_score,
                     "attention_gbs": attn_bytes / us_attend / 1e3},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle

        threads = max(1, len(os.sched_getaffinity(0)))
        t0 = time.perf_counter()
        steps = 0
        while True:
            s = oracle.score_fp8mh_layers(q, hw, rec, w.chunk_off, oracle.COMBINE_MAX)
            o_off, o_idx, _ = oracle.select_threshold(s, w.chunk_off, tau)
            oracle.attention(w.queries(steps % 4), w.K, w.V, w.tok_off, o_idx, o_off,
                             cfg.chunk_size, cfg.softmax_scale, dv=cfg.head_dim_v,
                             nthreads=threads)
            steps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        line["cpu_baseline"] = {
            "value": steps / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full retriever step(s) (all {B} streams) in {el:.1f} s: "
                      f"single-threaded fp64 C ensemble scoring and threshold, attention "
                      f"with OpenMP over (stream, head)"}
    print(json.dumps(line), flush=True)


LINK_PEAK_GBS = 64.0   # MI355X host interface, PCIe 5.0 x16, one direction (published)


def run_residency(args):
    """Times decode with delta residency on a pool workload: every
    `reindex_every` steps the drifting indexer query is re-scored and
    re-selected and only the newly kept chunks are copied from the pinned host
    store into the pool (lsa_pool_delta_update); every step attends from the
    pool through the slot table.  Attention steps are replayed from a HIP
    graph; the re-index phase runs eagerly (its host-link copy dominates)."""
    import numpy as np
    import torch

    from learned_kv_chunk_amd import device as dev
    from learned_kv_chunk_amd import lsa
    from learned_kv_chunk_amd import workloads as wl

    name = args.config if args.config != DEFAULT_CONFIG else "cfg3"
    cfg = wl.CONFIGS[name]
    R = args.reindex_every or max(cfg.reindex_every, 1)
    eps = args.drift
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    shape = d.shape
    c = cfg
    dt = shape.dtype

    def pinned(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
            if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))
        return t.pin_memory()

    kh = pinned(w.K)
    vh = None if w.V is None else pinned(w.V)
    k_pool = torch.empty((shape.total_k, c.chunk_size, c.head_dim_qk), dtype=dt, device="cuda")
    v_pool = None if w.V is None else torch.empty((shape.total_k, c.chunk_size, c.head_dim_v),
                                                  dtype=dt, device="cuda")
    table = torch.full((shape.total_k,), -1, dtype=torch.int32, device="cuda")
    loads = torch.empty(shape.total_k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(shape.batch, dtype=torch.int32, device="cuda")
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    aws = lsa.allocate_workspace(shape, "cuda")
    n_epochs = max(2, args.epochs)
    qs_idx = []
    for e in range(n_epochs + 1):
        q = wl.drift_query(w, e, eps)
        qs_idx.append(torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
                      if q.dtype == np.uint16 else torch.from_numpy(q).cuda())
    nq = 8
    qs = [d.queries(t) for t in range(nq)]
    row = (c.head_dim_qk + (0 if c.v_aliases_k else c.head_dim_v)) * (2 if c.dtype == "bf16" else 4)
    chunk_bytes = c.chunk_size * row

    def reindex(e):
        lsa.score(shape, qs_idx[e], d.emb, d.chunk_off, d.scores)
        lsa.select_topk(shape, d.scores, d.chunk_off, d.sel_off, d.sel_idx)
        lsa.pool_delta_update(shape, kh, vh, d.tok_off, d.chunk_off, d.sel_idx, d.sel_off, table,
                              k_pool, v_pool, loads, cnt)

    def attend(i):
        lsa.sparse_decode_attn(shape, qs[i % nq], k_pool, v_pool, d.tok_off, table, d.sel_off,
                               lsa.KV_POOL, out, lse, aws)

    # epoch 0 fills the pool from empty (every kept chunk crosses the link)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reindex(0)
    e1.record()
    torch.cuda.synchronize()
    fill_us = e0.elapsed_time(e1) * 1e3
    fill_loads = int(dev.to_host(cnt).sum())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(R):
            attend(i)
    graph.replay()
    torch.cuda.synchronize()

    # timed: epochs 1..n, each a re-index with the drifted query and R steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(n_epochs)]
    churn = []
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for e in range(n_epochs):
        a, b, cc = ev[e]
        a.record()
        reindex(e + 1)
        b.record()
        graph.replay()
        cc.record()
        churn.append(cnt.clone())
    t1.record()
    torch.cuda.synchronize()
    total_us = t0.elapsed_time(t1) * 1e3
    reidx_us = [a.elapsed_time(b) * 1e3 for a, b, _ in ev]
    attn_us = [b.elapsed_time(cc) * 1e3 / R for _, b, cc in ev]
    loads_per = [int(dev.to_host(x).sum()) for x in churn]
    steps = n_epochs * R
    link_bytes = [n * chunk_bytes for n in loads_per]

    # the delta copy kernel alone: HIP events around one update of a fresh epoch
    # whose kept set differs from the pool's
    reindex_parts = []
    for e in range(2):
        lsa.score(shape, qs_idx[(n_epochs + e) % (n_epochs + 1)], d.emb, d.chunk_off, d.scores)
        lsa.select_topk(shape, d.scores, d.chunk_off, d.sel_off, d.sel_idx)
        x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        x0.record()
        lsa.pool_delta_update(shape, kh, vh, d.tok_off, d.chunk_off, d.sel_idx, d.sel_off, table,
                              k_pool, v_pool, loads, cnt)
        x1.record()
        torch.cuda.synchronize()
        reindex_parts.append((x0.elapsed_time(x1) * 1e3, int(dev.to_host(cnt).sum()) * chunk_bytes))
    delta_us, delta_bytes = reindex_parts[-1]

    # the link's achievable rate: one pinned host-to-device copy of the same size
    nb = max(delta_bytes, 1 << 20)
    src = torch.empty(nb, dtype=torch.uint8).pin_memory()
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    y0, y1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y0.record()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    y1.record()
    torch.cuda.synchronize()
    memcpy_gbs = 5 * nb / (y0.elapsed_time(y1) * 1e3) / 1e3

    delta_gbs = delta_bytes / delta_us / 1e3
    line = {
        "metric": "decode steps/sec with delta residency over a pinned host store "
                  f"(re-index every {R} steps, drifting query)",
        "value": steps / total_us * 1e6, "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": 1, "ms_per_step": total_us / steps / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": f"{name}: {WORKLOAD_TEXT[name]}; host-resident K/V, pool of the "
                               f"kept chunks", "reindex_every": R, "drift_eps": eps,
                   "epochs": n_epochs,
                   "timing": "attention steps replayed from a HIP graph, re-index eager",
                   "cache": "warm: the pool (107 MB) fits the 256 MB Infinity Cache and is "
                            "re-read every step"},
        "fill_from_empty": {"chunks": fill_loads, "bytes": fill_loads * chunk_bytes,
                            "us": fill_us},
        "chunks_loaded_per_reindex": loads_per,
        "link_bytes_per_reindex": link_bytes,
        "reindex_us": reidx_us,
        "attention_us_per_step": attn_us,
        "resident_bytes": int(shape.total_k) * chunk_bytes,
        "history_bytes": int(w.tok_off[-1]) * row,
        "roofline": {"kernel": "pool_delta_kernel + pool_load_kernel (host link)",
                     "bound": "link", "achieved": delta_gbs, "peak": LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": delta_gbs / LINK_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": int(delta_bytes), "avg_launch_us": delta_us,
                     "pinned_memcpy_gbs": memcpy_gbs},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle

        threads = max(1, len(os.sched_getaffinity(0)))
        tab = np.full(int(shape.total_k), -1, np.int32)
        pool_k = np.zeros((int(shape.total_k), c.chunk_size) + w.K.shape[1:], w.K.dtype)
        t_start = time.perf_counter()
        steps_done = reidx_done = 0
        e = 0
        while True:
            if steps_done % R == 0:
                q = wl.drift_query(w, e, eps)
                sc = oracle.score(q, w.emb, w.chunk_off)
                sel = oracle.select(sc, w.chunk_off, w.sel_off)
                tab, ld, n = oracle.pool_delta(w.chunk_off, sel, w.sel_off, tab)
                for b in range(w.B):       # copy only the loaded slots
                    for p in ld[w.sel_off[b]:w.sel_off[b] + n[b]]:
                        pool_k[p] = oracle.gather(w.K[w.tok_off[b]:w.tok_off[b + 1]], c.chunk_size,
                                                  np.array([0, w.lengths[b]], np.int64),
                                                  np.array([tab[p]], np.int32),
                                                  np.array([0, 1], np.int32))[0]
                reidx_done += 1
                e += 1
            oracle.attention(w.queries(steps_done % 4), w.K, w.V, w.tok_off, sel, w.sel_off,
                             c.chunk_size, c.softmax_scale, dv=c.head_dim_v, nthreads=threads)
            steps_done += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds:
                break
        line["cpu_baseline"] = {
            "value": steps_done / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps_done} decode step(s) with {reidx_done} re-index(es) in {el:.1f} s "
                      f"(scoring, select, slot table and K chunk copies single-threaded; "
                      f"attention with OpenMP over (stream, head))"}
    print(json.dumps(line), flush=True)


def run_append(args):
    """Times decode over a growing context: every step appends one K/V row per
    stream (lsa_append_kv), builds the keep set of the grown context
    (lsa_keep_recent: kept chunks, the last scored chunk, unscored chunks) and
    attends over the capacity layout (lsa_sparse_decode_attn_varlen); every
    `reindex_every` steps the scored chunks are re-scored and re-selected.
    Everything runs on the device, so the timed steps are replayed from one
    HIP graph; each replay starts from the same lengths."""
    import dataclasses

    import numpy as np
    import torch

    from learned_kv_chunk_amd import device as dev
    from learned_kv_chunk_amd import lsa
    from learned_kv_chunk_amd import workloads as wl

    cfg = wl.CONFIGS[args.config]
    C = cfg.chunk_size
    R = args.reindex_every or 64
    steps = args.steps
    max_recent = 2 + (steps + C - 1) // C
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    shape = d.shape
    es = 2 if cfg.dtype == "bf16" else 4
    L0 = w.lengths.astype(np.int64)
    cap = L0 + steps + C
    base = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
    dt = shape.dtype
    kd = torch.empty((int(base[-1]), cfg.head_dim_qk), dtype=dt, device="cuda")
    vd = None if w.V is None else torch.empty((int(base[-1]), cfg.head_dim_v), dtype=dt,
                                                 device="cuda")
    for b in range(w.B):
        kd[base[b]:base[b] + L0[b]] = d.K[w.tok_off[b]:w.tok_off[b + 1]]
        if vd is not None:
            vd[base[b]:base[b] + L0[b]] = d.V[w.tok_off[b]:w.tok_off[b + 1]]
    base_d = torch.from_numpy(base).cuda()
    seq0 = torch.from_numpy(L0.copy()).cuda()
    seq_d = seq0.clone()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    k_new = (torch.randn((steps, w.B, cfg.head_dim_qk), generator=g, device="cuda")
             * cfg.kv_std).to(dt)
    v_new = None if vd is None else (torch.randn((steps, w.B, cfg.head_dim_v), generator=g,
                                                 device="cuda") * cfg.kv_std).to(dt)
    n_cap = (cap + C - 1) // C
    attn_shape = dataclasses.replace(
        shape, max_chunks=int(n_cap.max()), total_chunks=int(n_cap.sum()),
        max_k=shape.max_k + max_recent, total_k=shape.total_k + w.B * max_recent,
        uniform=False)
    ws = lsa.allocate_workspace(attn_shape, "cuda")
    out_idx = torch.empty(attn_shape.total_k, dtype=torch.int32, device="cuda")
    out_off = torch.empty(w.B + 1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(d.out)
    lse = torch.empty_like(d.lse)
    nq = 8
    qs = [d.queries(t) for t in range(nq)]

    def step(t):
        if t % R == 0:
            lsa.score(shape, d.q_idx, d.emb, d.chunk_off, d.scores)
            lsa.select_topk(shape, d.scores, d.chunk_off, d.sel_off, d.sel_idx)
        lsa.append_kv(shape, k_new[t], None if v_new is None else v_new[t], base_d, seq_d, kd, vd)
        lsa.keep_recent(shape, seq_d, d.chunk_off, d.sel_idx, d.sel_off, max_recent, out_idx,
                        out_off)
        lsa.sparse_decode_attn_varlen(attn_shape, qs[t % nq], kd, vd, base_d, seq_d, out_idx,
                                      out_off, lsa.KV_STORE, out, lse, ws)

    for t in range(min(args.warmup, steps)):
        step(t)
    torch.cuda.synchronize()
    seq_d.copy_(seq0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            step(t)
    seq_d.copy_(seq0)
    graph.replay()
    torch.cuda.synchronize()
    grown = dev.to_host(seq_d)
    assert (grown == L0 + steps).all(), "every step appended one row per stream"
    seq_d.copy_(seq0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    kept = dev.to_host(out_off)
    idx = dev.to_host(out_idx)[:int(kept[-1])]
    grown = L0 + steps
    ktok = 0
    for b in range(w.B):
        n = idx[kept[b]:kept[b + 1]].astype(np.int64)
        ktok += int(np.minimum(C, grown[b] - n * C).sum())
    ab = algorithmic_bytes(w)
    attn_bytes = ktok * ab["row"] + ab["q"]
    # the attention launch alone at the grown length (partial kernel and merge)
    attn_us = _graph_us(lambda i: lsa.sparse_decode_attn_varlen(
        attn_shape, qs[i % nq], kd, vd, base_d, seq_d, out_idx, out_off, lsa.KV_STORE, out, lse,
        ws), steps)
    attn_gbs = attn_bytes / attn_us / 1e3
    line = {
        "metric": "decode steps/sec over a growing context (append + keep set + sparse attn, "
                  f"re-index every {R})",
        "value": 1e6 / us, "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": us / 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}; grows by "
                               f"{steps} tokens per stream", "reindex_every": R,
                   "max_recent": max_recent,
                   "timing": "all steps captured in one HIP graph, replayed once",
                   "cache": "warm: one K/V copy, whose kept chunks (about 146 MB at 16 x 128K) "
                            "fit the 256 MB Infinity Cache and are re-read every step"},
        "final_keep_chunks": np.diff(kept).tolist(),
        "tokens_per_s": 1e6 / us * w.B,
        "roofline": {"kernel": "attn (split-KV partial + merge) at the grown length",
                     "bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": attn_gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": int(attn_bytes), "avg_launch_us": attn_us},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle

        threads = max(1, len(os.sched_getaffinity(0)))
        Kh = [w.K[w.tok_off[b]:w.tok_off[b + 1]] for b in range(w.B)]
        Vh = None if w.V is None else [w.V[w.tok_off[b]:w.tok_off[b + 1]] for b in range(w.B)]
        kn = dev.to_host(k_new)
        vn = None if v_new is None else dev.to_host(v_new)
        t_start = time.perf_counter()
        n_done = 0
        sel = None
        while True:
            t = n_done
            if t % R == 0:
                sel = oracle.select(oracle.score(w.q_idx, w.emb, w.chunk_off), w.chunk_off,
                                    w.sel_off)
            Kh = [np.concatenate([Kh[b], kn[t % steps][b:b + 1]]) for b in range(w.B)]
            if Vh is not None:
                Vh = [np.concatenate([Vh[b], vn[t % steps][b:b + 1]]) for b in range(w.B)]
            lens = np.array([len(x) for x in Kh], np.int64)
            off, ids = oracle.keep_recent(C, lens, w.chunk_off, sel, w.sel_off, max_recent)
            tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
            oracle.attention(w.queries(t % 4), np.concatenate(Kh),
                             None if Vh is None else np.concatenate(Vh), tok, ids, off, C,
                             cfg.softmax_scale, dv=cfg.head_dim_v, nthreads=threads)
            n_done += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds or n_done >= steps:
                break
        line["cpu_baseline"] = {
            "value": n_done / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_done} growing-context decode step(s) of the same workload in "
                      f"{el:.1f} s (append and keep set single-threaded, attention with OpenMP "
                      f"over (stream, head))"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--replicas", type=int, default=0,
                    help="workload copies cycled per step (0: enough to defeat the 256 MB cache)")
    ap.add_argument("--reindex-every", type=int, default=0, help="0: the workload's schedule")
    ap.add_argument("--tiles-per-block", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--read-pattern", type=int, default=1, choices=[0, 1, 2],
                    help="--mode read: 0 plain, 1 non-temporal, 2 the MQA K operand pattern")
    ap.add_argument("--mode", choices=["step", "copy", "read", "scorer", "retriever", "residency",
                                       "append"], default="step")
    ap.add_argument("--drift", type=float, default=0.5,
                    help="residency mode: indexer query drift per re-index epoch")
    ap.add_argument("--epochs", type=int, default=4, help="residency mode: timed re-index epochs")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--attention-only", action="store_true",
                    help="step mode: time only the attention partial kernel (pass 3), so "
                         "that a kernel trace of the run holds just those launches")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the LSA hot path here has no "
              "multi-GPU component); run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_kv_chunk_amd import device as dev
    from learned_kv_chunk_amd import lsa
    from learned_kv_chunk_amd import workloads as wl

    lsa.library()  # fail loudly without the HIP library
    torch.cuda.set_device(0)
    if args.mode == "read":
        run_read(args)
        return
    if args.mode == "copy":
        run_copy(args)
        return
    if args.mode == "scorer":
        run_scorer(args)
        return
    if args.mode == "retriever":
        run_retriever(args)
        return
    if args.mode == "residency":
        run_residency(args)
        return
    if args.mode == "append":
        run_append(args)
        return

    cfg = wl.CONFIGS[args.config]
    R_idx = args.reindex_every or cfg.reindex_every
    t0 = time.perf_counter()
    w = wl.make_workload(cfg)
    print(f"bench: generated {args.config} in {time.perf_counter() - t0:.1f} s "
          f"(sum L={int(w.lengths.sum())}, sum N={int(w.chunk_off[-1])}, "
          f"sum k={int(w.sel_off[-1])})", file=sys.stderr, flush=True)
    base = dev.upload(w, "cuda", attn_tiles_per_block=args.tiles_per_block)
    ab = algorithmic_bytes(w)

    # one untimed step to learn the kept set (for the exact kept-token count)
    base.step(0, reindex=True, materialize_pool=cfg.materialize_pool)
    torch.cuda.synchronize()
    sel = dev.to_host(base.sel_idx)
    ktok = kept_tokens(w, sel)
    attn_bytes = ktok * ab["row"] + ab["q"]                      # per attention launch
    gather_bytes = 2 * ktok * ab["row"] if cfg.materialize_pool else 0
    reidx_bytes = ab["score"] + ab["select"] + gather_bytes
    step_bytes = attn_bytes + ab["o"] + reidx_bytes / R_idx      # amortised per step

    reps = args.replicas
    if reps <= 0:
        reps = max(1, math.ceil(2 * MALL_BYTES / max(1, step_bytes)) + 1)
    replicas = [base]
    for _ in range(reps - 1):
        r = dev.DeviceWorkload(
            w=w, shape=base.shape, q_idx=base.q_idx.clone(), emb=base.emb.clone(),
            chunk_off=base.chunk_off, sel_off=base.sel_off, tok_off=base.tok_off,
            K=base.K.clone(), V=None if base.V is None else base.V.clone(),
            scores=torch.empty_like(base.scores), sel_idx=base.sel_idx.clone(),
            out=torch.empty_like(base.out), lse=torch.empty_like(base.lse),
            workspace=torch.zeros_like(base.workspace),
            k_pool=None if base.k_pool is None else torch.empty_like(base.k_pool),
            v_pool=None if base.v_pool is None else torch.empty_like(base.v_pool))
        replicas.append(r)
    nq = 8
    qs = [base.queries(t) for t in range(nq)]
    for r in replicas:  # fill every replica's kept set (and pool) once; this also
        # marshals each replica's step arguments (PreparedStep) outside the timing
        r.step(0, materialize_pool=cfg.materialize_pool, q=qs[0], reindex_every=R_idx)
    torch.cuda.synchronize()
    print(f"bench: {reps} replica(s), {step_bytes / 1e6:.1f} MB per step", file=sys.stderr,
          flush=True)

    def run(n, t_begin, evs=None):
        for i in range(n):
            t = t_begin + i
            r = replicas[t % reps]
            eb, ee = (evs[i] if evs is not None else (None, None))
            r.step(t, reindex_every=R_idx, materialize_pool=cfg.materialize_pool,
                   ev_begin=eb, ev_end=ee, q=qs[t % nq])

    # pass 3 (roofline.avg_launch_us): the attention phase alone (one
    # lsa_sparse_decode_attn call: split-KV partials and their log-sum-exp
    # merge), the K calls (one per replica in turn, so each reads cold K/V)
    # replayed back to back from a HIP graph with two events around the
    # replay: no event record sits between the kernels
    pool_mode = bool(cfg.materialize_pool)

    def attention(i):
        r = replicas[i % reps]
        lsa.sparse_decode_attn(
            r.shape, qs[i % nq], r.k_pool if pool_mode else r.K,
            r.v_pool if pool_mode else r.V, r.tok_off, r.sel_idx, r.sel_off,
            lsa.KV_POOL if pool_mode else lsa.KV_STORE, out=r.out, lse=r.lse,
            workspace=r.workspace)

    def partial(i):  # the partial kernel without any merge (dominant kernel of MLA)
        r = replicas[i % reps]
        lsa.bench_attention_partial(
            r.shape, qs[i % nq], r.k_pool if pool_mode else r.K,
            r.v_pool if pool_mode else r.V, r.tok_off, r.sel_idx, r.sel_off,
            lsa.KV_POOL if pool_mode else lsa.KV_STORE, r.workspace)

    def score(i):
        r = replicas[i % reps]
        lsa.score(r.shape, r.q_idx, r.emb, r.chunk_off, scores=r.scores)

    # how the library runs attention for this shape (kernel, merge in the
    # kernel or a merge launch), as lsa_attention_plan reports it
    attn_plan = lsa.attention_plan(replicas[0].shape)
    fused = attn_plan["merge_in_kernel"]
    kernel_file = os.path.join(ROOT, "learned_kv_chunk_amd", "csrc", attn_plan["kernel"] + ".hip")
    kname = attn_plan["kernel"] + (" (split heads)" if attn_plan["split_heads"] else "")
    attn_desc = (kname + ": split-KV partials and their LSE merge in one kernel" if fused else
                 kname + " partial kernel + LSE merge kernel (the attention phase)")
    if args.attention_only:
        attn_us = _graph_us(attention, args.steps, warm=4)
        attn_gbs = attn_bytes / attn_us / 1e3
        print(json.dumps({
            "metric": "split-KV attention partial kernel launches/sec (cold K/V)",
            "value": 1e6 / attn_us, "unit": "launches/s", "n_gpus": 1, "steps": args.steps,
            "warmup": 4, "higher_is_better": True, "dtype": cfg.dtype, "data": "synthetic",
            "config": {"workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}",
                       "replicas": reps},
            "roofline": {"kernel": attn_desc,
                         "bound": "hbm", "achieved": attn_gbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS,
                         "algorithmic_bytes_per_launch": int(attn_bytes),
                         "avg_launch_us": attn_us,
                         "timing": "K cold launches replayed from a HIP graph (four untimed "
                                   "replays first)"}}), flush=True)
        return

    run(args.warmup, 0)
    torch.cuda.synchronize()
    # steps are numbered from a multiple of the re-index interval so that the
    # timed window holds steps/R_idx re-index steps
    t_first = ((args.warmup + R_idx - 1) // R_idx) * R_idx

    # pass 1 (the headline): K steps bracketed by two events only
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    g0.record()
    run(args.steps, t_first)
    g1.record()
    host_enqueue_s = time.perf_counter() - w0
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = g0.elapsed_time(g1) / args.steps
    steps_per_s = 1e3 / ms_per_step

    # pass 1b: the same K steps captured once in a HIP graph and replayed
    # between two events, as a decode loop that captures its step would issue
    # them (no host launch cost between steps)
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        run(args.steps, t_first)
    step_graph.replay()
    torch.cuda.synchronize()
    gg0, gg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gg0.record()
    step_graph.replay()
    gg1.record()
    torch.cuda.synchronize()
    graph_ms_per_step = gg0.elapsed_time(gg1) / args.steps
    del step_graph

    # pass 2: the same K steps with HIP events around the attention kernel of
    # every step (event records cost time between kernels, so this pass only
    # measures that kernel's duration)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:  # create the underlying HIP events before timing
        a.record()
        b.record()
    torch.cuda.synchronize()
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0.record()
    run(args.steps, t_first, evs)
    h1.record()
    torch.cuda.synchronize()
    attn_us_events = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    ms_per_step_with_events = h0.elapsed_time(h1) / args.steps

    # pass 3 (roofline.avg_launch_us): see the definition of `attention`; run
    # after the step passes, with the clocks up; the partial kernel alone and
    # the score kernel alone the same way
    attn_us = _graph_us(attention, args.steps)
    attn_gbs = attn_bytes / attn_us / 1e3
    partial_us = attn_us if fused else _graph_us(partial, args.steps)
    score_us = _graph_us(score, args.steps)
    score_bytes = ab["score"]

    # warm (Infinity-Cache-assisted) reference: the same steps on one replica
    warm_n = min(args.steps, 100)
    ww0, ww1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ww0.record()
    for i in range(warm_n):
        t = t_first + i
        replicas[0].step(t, reindex_every=R_idx, materialize_pool=cfg.materialize_pool,
                         q=qs[t % nq])
    ww1.record()
    torch.cuda.synchronize()
    warm_ms = ww0.elapsed_time(ww1) / warm_n

    # per-step spread: events around every step (their own cost inflates each
    # value by a few microseconds; the pass-1 mean is the headline)
    spread_n = min(args.steps, 100)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(spread_n)]
    for a0, a1 in sev:
        a0.record()
        a1.record()
    torch.cuda.synchronize()
    for i in range(spread_n):
        t = t_first + i
        sev[i][0].record()
        replicas[t % reps].step(t, reindex_every=R_idx,
                                materialize_pool=cfg.materialize_pool, q=qs[t % nq])
        sev[i][1].record()
    torch.cuda.synchronize()
    per_step = np.array([a0.elapsed_time(a1) * 1e3 for a0, a1 in sev])

    # re-index and attention-only phases of a pool workload, and the gather
    phases = None
    if R_idx > 1:
        pa0, pa1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_a = min(reps * 2, 16)
        torch.cuda.synchronize()
        pa0.record()
        for i in range(n_a):
            replicas[i % reps].step(0, reindex=True, materialize_pool=cfg.materialize_pool,
                                    q=qs[0])
        pa1.record()
        torch.cuda.synchronize()
        phase_a = pa0.elapsed_time(pa1) * 1e3 / n_a
        pb0, pb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_b = min(args.steps, 64)
        pb0.record()
        for i in range(n_b):
            replicas[i % reps].step(i + 1, reindex=False, materialize_pool=cfg.materialize_pool,
                                    q=qs[(i + 1) % nq])
        pb1.record()
        torch.cuda.synchronize()
        phase_b = pb0.elapsed_time(pb1) * 1e3 / n_b
        phases = {"reindex_step_us": phase_a, "attention_step_us": phase_b,
                  "amortised_step_us": (phase_a + (R_idx - 1) * phase_b) / R_idx}
        if cfg.materialize_pool:
            def gather(i):
                r = replicas[i % reps]
                lsa.gather_chunks(r.shape, r.K, r.V, r.tok_off, r.sel_idx, r.sel_off, r.k_pool,
                                  r.v_pool)
            g_us = _graph_us(gather, min(args.steps, 4 * reps))
            phases["gather"] = {"us": g_us, "bytes": int(gather_bytes),
                                "gbs": gather_bytes / g_us / 1e3,
                                "frac": gather_bytes / g_us / 1e3 / HBM_PEAK_GBS}

    # the achievable streaming rate on this part (1 GiB read + 1 GiB written)
    cb = 1 << 30
    csrc = torch.empty(cb, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    lsa.bench_copy(cdst, csrc, cb)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        lsa.bench_copy(cdst, csrc, cb)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * cb / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst
    traffic = load_traffic(kernel_file, args.config)
    line = {
        "metric": "LSA decode steps/sec at 128K ctx (score+top-k+attn); HBM GB/s vs peak",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {WORKLOAD_TEXT[args.config]}",
            "global_batch": cfg.batch,
            "seq_len": int(w.lengths.max()),
            "reindex_every": R_idx,
            "replicas": reps,
            "cache": "cold (replicas cycle > 2x Infinity Cache)" if reps * step_bytes >
                     2 * MALL_BYTES else "warm (cache-assisted)",
        },
        "tokens_per_s": steps_per_s * cfg.batch,
        "step_algorithmic_bytes": int(step_bytes),
        "step_gbs": step_bytes * steps_per_s / 1e9,
        "step_hbm_frac": step_bytes * steps_per_s / 1e9 / HBM_PEAK_GBS,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "host_enqueue_ms_per_step": host_enqueue_s * 1e3 / args.steps,
        "graph_ms_per_step": graph_ms_per_step,
        "graph_steps_per_s": 1e3 / graph_ms_per_step,
        "ms_per_step_with_attn_events": ms_per_step_with_events,
        "resident_fraction": w.resident_fraction(),
        "roofline": {
            "kernel": attn_desc,
            "bound": "hbm",
            "achieved": attn_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": attn_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(attn_bytes),
            "avg_launch_us": attn_us,
            "timing": "the attention phase (one lsa_sparse_decode_attn call), K cold calls "
                      "replayed from a HIP graph",
            "partial_kernel_us": partial_us,
            "avg_launch_us_events_in_step": attn_us_events,
            "measured_copy_gbs": copy_gbs,
            "frac_of_measured_copy": attn_gbs / copy_gbs,
            "attention_plan": attn_plan,
        },
        "score_kernel": {"us": score_us, "algorithmic_bytes": int(score_bytes),
                         "gbs": score_bytes / score_us / 1e3,
                         "frac": score_bytes / score_us / 1e3 / HBM_PEAK_GBS,
                         "timing": "K cold launches replayed from a HIP graph"},
        "warm_ms_per_step": warm_ms,
        "warm_note": "one replica, back to back: Infinity-Cache-assisted",
        "step_us_p10_p50_p90_with_events": [float(np.percentile(per_step, q)) for q in
                                            (10, 50, 90)],
        "phases": phases,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, R_idx)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
