"""Shared checks of the GPU path against the CPU oracle, with the tolerances
the GPU tests apply.  Helpers only; the tests live in test_gpu_*.py.

Tolerances (floating point; integer and index results are bit-exact):
* scores: |s_gpu - s_ref| <= 1e-4 * max(|s_ref|, |q| |e|)  (1e-4 relative,
  scaled by the Cauchy-Schwarz bound so near-orthogonal chunks, whose fp32
  accumulation error is absolute, are not judged relatively);
* selection: bit-identical to the oracle's top-k of the GPU's own fp32
  scores; against the oracle's fp64 scores, identical wherever the k-th and
  (k+1)-th scores differ by more than 1e-3, else every differing chunk lies
  within 1e-3 of that boundary;
* attention, fp32 inputs: per (stream, head) row, max|dO| <= 1e-5 max|O_ref|
  and |dLSE| <= 1e-5 |LSE_ref|;
* attention, bf16 inputs: max|dO| <= 2e-2 (absolute), and, because that bound
  is loose for small outputs, also ||dO||_2 <= 1e-2 ||O_ref||_2 per row and
  |dLSE| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle


def f64(a):
    return wl.as_f32(a).astype(np.float64)


def check_scores(w: wl.Workload, s_gpu: np.ndarray, s_ref: np.ndarray) -> None:
    q = f64(w.q_idx)
    e = f64(w.emb)
    qn = np.repeat(np.linalg.norm(q, axis=1), np.diff(w.chunk_off))
    bound = np.maximum(np.abs(s_ref), qn * np.linalg.norm(e, axis=1))
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    worst = float((err / bound).max())
    assert worst <= 1e-4, f"score error {worst:.3e} x bound"


def check_selection(w: wl.Workload, s_gpu: np.ndarray, sel_gpu: np.ndarray,
                    s_ref: np.ndarray) -> None:
    # strong check: the GPU's top-k of its own scores equals the oracle's top-k of them
    mine = oracle.select(s_gpu.astype(np.float64), w.chunk_off, w.sel_off)
    np.testing.assert_array_equal(sel_gpu, mine)
    # against fp64 scores: equality where the k/k+1 gap exceeds 1e-3
    ref = oracle.select(s_ref, w.chunk_off, w.sel_off)
    for b in range(w.B):
        a = set(sel_gpu[w.sel_off[b]:w.sel_off[b + 1]].tolist())
        r = set(ref[w.sel_off[b]:w.sel_off[b + 1]].tolist())
        if a == r:
            continue
        srt = np.sort(s_ref[w.chunk_off[b]:w.chunk_off[b + 1]])[::-1]
        k = int(w.keep[b])
        assert k < len(srt)
        gap = srt[k - 1] - srt[k]
        assert gap <= 1e-3, f"stream {b}: sets differ with k/k+1 gap {gap}"
        mid = 0.5 * (srt[k - 1] + srt[k])
        for n in a ^ r:
            assert abs(s_ref[w.chunk_off[b] + n] - mid) <= 1e-3


def check_needles(w: wl.Workload, sel_gpu: np.ndarray) -> None:
    for b in range(w.B):
        if len(w.needles[b]) <= int(w.keep[b]):
            kept = set(sel_gpu[w.sel_off[b]:w.sel_off[b + 1]].tolist())
            missing = set(w.needles[b].tolist()) - kept
            assert not missing, f"stream {b} dropped needles {missing}"


def check_attention(dtype: str, out_gpu, lse_gpu, out_ref, lse_ref, rows=None) -> dict:
    """Returns the worst errors seen; asserts the tolerances of the module doc."""
    og = np.asarray(out_gpu, dtype=np.float64)
    lg = np.asarray(lse_gpu, dtype=np.float64)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    d = og - out_ref
    stats = {}
    if dtype == "f32":
        rel = np.abs(d).max(-1) / np.maximum(np.abs(out_ref).max(-1), 1e-30)
        lrel = np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1e-30)
        stats = {"max_rel_out": float(rel.max()), "max_rel_lse": float(lrel.max())}
        assert rel.max() <= 1e-5, stats
        assert lrel.max() <= 1e-5, stats
    else:
        norm_rel = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(out_ref, axis=-1),
                                                            1e-30)
        stats = {"max_abs_out": float(np.abs(d).max()), "max_norm_rel_out": float(norm_rel.max()),
                 "max_abs_lse": float(np.abs(lg - lse_ref).max())}
        assert np.abs(d).max() <= 2e-2, stats
        assert norm_rel.max() <= 1e-2, stats
        assert np.abs(lg - lse_ref).max() <= 1e-3, stats
    return stats


def run_phases(d: dev.DeviceWorkload, step: int = 0):
    """Per-phase entry points (score, select, attention from the store)."""
    s = d.shape
    lsa.score(s, d.q_idx, d.emb, d.chunk_off, d.scores)
    lsa.select_topk(s, d.scores, d.chunk_off, d.sel_off, d.sel_idx)
    lsa.sparse_decode_attn(s, d.queries(step), d.K, d.V, d.tok_off, d.sel_idx, d.sel_off,
                           lsa.KV_STORE, d.out, d.lse, d.workspace)
    torch.cuda.synchronize()
    return (dev.to_host(d.scores), dev.to_host(d.sel_idx), dev.to_host(d.out),
            dev.to_host(d.lse))


def oracle_attention_on(w: wl.Workload, step: int, sel: np.ndarray, streams=None,
                        nthreads: int = 0):
    """Oracle attention for the given kept set; optionally only some streams
    (their rows of K/V and offsets are cut out so the oracle reads nothing else)."""
    c = w.cfg
    nthreads = nthreads or max(1, oracle.max_threads())
    Q = w.queries(step)
    if streams is None:
        return oracle.attention(Q, w.K, w.V, w.tok_off, sel, w.sel_off, c.chunk_size,
                                c.softmax_scale, dv=c.head_dim_v, nthreads=nthreads)
    outs, lses = [], []
    for b in streams:
        r0, r1 = int(w.tok_off[b]), int(w.tok_off[b + 1])
        sl = sel[w.sel_off[b]:w.sel_off[b + 1]]
        o, l = oracle.attention(Q[b:b + 1], w.K[r0:r1], None if w.V is None else w.V[r0:r1],
                                np.array([0, r1 - r0], np.int64), sl,
                                np.array([0, len(sl)], np.int32), c.chunk_size,
                                c.softmax_scale, dv=c.head_dim_v, nthreads=nthreads)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)
