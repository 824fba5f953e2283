"""Parity of the retriever-side keep path with the CPU oracle, through the C
ABI: the layer ensemble of the float8 multi-head scorer (max and mean), the
threshold keep set with its cap and dense fallback, and sparse attention over
the kept set the device produced (its CSR offsets exist only on the device).

Tolerances.  Scores: |s_gpu - s_ref| <= 1e-4 * max(|s_ref|, A), A the largest
over layers of sum_h |w_h| |c| sum_d |q_hd k_d| (fp32 accumulation error is
relative to that magnitude; a head whose dot product is near zero may fall on
either side of the ReLU).  Keep sets: both sides decide on the GPU's fp32
scores, so sel_off, the kept indices and the fallback flags must be identical.
Attention: the tolerances of tests/parity.py, with the oracle run on the
GPU's kept set."""
import json
import os

import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _abs_bound_layers(q, hw, rec, chunk_off):
    L, B, Hs, D = q.shape
    out = np.zeros(rec.shape[1])
    for l in range(L):
        ql = np.abs(wl.bf16_bits_to_f32(q[l]).astype(np.float64))
        k = np.abs(torch.from_numpy(np.ascontiguousarray(rec[l, :, :D]))
                   .view(torch.float8_e4m3fn).double().numpy())
        c = np.abs(np.ascontiguousarray(rec[l, :, D:]).view("<f4").reshape(-1).astype(np.float64))
        for b in range(B):
            r0, r1 = chunk_off[b], chunk_off[b + 1]
            bl = c[r0:r1] * ((k[r0:r1] @ ql[b].T) @ np.abs(hw[l, b]).astype(np.float64))
            out[r0:r1] = np.maximum(out[r0:r1], bl)
    return out


def _gpu_scores(w, q, hw, rec, combine):
    shape = dev.problem_shape(w)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    s = lsa.score_fp8_multihead_layers(shape, qd, torch.from_numpy(hw).cuda(),
                                       torch.from_numpy(rec).cuda(),
                                       torch.from_numpy(w.chunk_off).cuda(), combine)
    torch.cuda.synchronize()
    return dev.to_host(s)


def _check_scores(w, q, hw, rec, combine, s_gpu):
    s_ref = oracle.score_fp8mh_layers(q, hw, rec, w.chunk_off, combine)
    bound = np.maximum(np.abs(s_ref), _abs_bound_layers(q, hw, rec, w.chunk_off))
    err = float((np.abs(s_gpu.astype(np.float64) - s_ref) / bound).max())
    assert err <= 1e-4, f"score error {err:.3e} x bound"
    return s_ref, err


def _threshold_shape(B, chunk_off):
    n = np.diff(chunk_off)
    return lsa.ProblemShape(batch=B, chunk_size=64, index_dim=128, num_q_heads=16,
                            head_dim_qk=128, head_dim_v=128, v_aliases_k=False,
                            dtype=torch.bfloat16, softmax_scale=128 ** -0.5,
                            max_chunks=int(n.max()), max_k=int(n.max()),
                            total_chunks=int(chunk_off[-1]), total_k=int(chunk_off[-1]))


def _gpu_threshold(scores_f32, chunk_off, tau, cap, shape=None):
    B = len(chunk_off) - 1
    shape = shape or _threshold_shape(B, chunk_off)
    off, idx, fb = lsa.select_threshold(shape, torch.from_numpy(scores_f32).cuda(),
                                        torch.from_numpy(chunk_off).cuda(), np.float32(tau), cap)
    torch.cuda.synchronize()
    off, idx, fb = dev.to_host(off), dev.to_host(idx), dev.to_host(fb)
    return off, idx[:int(off[-1])], fb


def _check_threshold(scores_f32, chunk_off, tau, cap):
    got = _gpu_threshold(scores_f32, chunk_off, tau, cap)
    ref = oracle.select_threshold(scores_f32.astype(np.float64), chunk_off,
                                  float(np.float32(tau)), cap)
    for g, r, name in zip(got, ref, ("sel_off", "sel_idx", "fallback")):
        np.testing.assert_array_equal(g, r, err_msg=f"{name} (tau={tau}, cap={cap})")
    return got


@pytest.mark.parametrize("combine", [oracle.COMBINE_MAX, oracle.COMBINE_MEAN])
@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_layer_ensemble_small_ragged(name, combine):
    w = wl.make_workload(wl.small_variant(name))
    q, hw, rec = wl.make_mh_layer_inputs(w, layers=3)
    s_gpu = _gpu_scores(w, q, hw, rec, combine)
    print(name, combine, _check_scores(w, q, hw, rec, combine, s_gpu)[1])


@pytest.mark.parametrize("layers,heads,head_dim", [(1, 128, 128), (2, 32, 64), (4, 16, 128)])
def test_layer_ensemble_shapes(layers, heads, head_dim):
    w = wl.make_workload(wl.small_variant("cfg2", lengths=(64 * 100 + 3, 64 * 37, 64 * 5 + 9)))
    q, hw, rec = wl.make_mh_layer_inputs(w, layers=layers, heads=heads, head_dim=head_dim)
    for combine in (oracle.COMBINE_MAX, oracle.COMBINE_MEAN):
        s_gpu = _gpu_scores(w, q, hw, rec, combine)
        _check_scores(w, q, hw, rec, combine, s_gpu)
    if layers == 1:
        # one layer: the same scores as the single-layer entry point, bit for bit
        shape = dev.problem_shape(w)
        one = lsa.score_fp8_multihead(
            shape, torch.from_numpy(q[0].view(np.int16)).view(torch.bfloat16).cuda(),
            torch.from_numpy(hw[0]).cuda(), torch.from_numpy(rec[0]).cuda(),
            torch.from_numpy(w.chunk_off).cuda())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(dev.to_host(one), s_gpu)


def test_threshold_golden_on_device():
    g = json.load(open(os.path.join(GOLDEN, "select_threshold.json")))
    streams = [[float(x) for x in s] for s in g["streams"]]
    co = np.concatenate([[0], np.cumsum([len(s) for s in streams])]).astype(np.int32)
    s = np.array(sum(streams, []), np.float32)
    for case in g["cases"]:
        off, idx, fb = _check_threshold(s, co, float(case["tau"]), case["max_keep"])
        assert off.tolist() == case["sel_off"] and idx.tolist() == case["sel_idx"]
        assert fb.tolist() == case["fallback"]


@pytest.mark.parametrize("n_list", [(1,), (5, 1, 300), (2048,) * 4, (8192,), (9000, 17, 4100),
                                    (64,) * 40])
def test_threshold_random_ties_caps_fallbacks(n_list):
    rng = np.random.default_rng(len(n_list) * 1000 + n_list[0])
    co = np.concatenate([[0], np.cumsum(n_list)]).astype(np.int32)
    B = len(n_list)
    # per-stream offsets spread the streams' maxima so that a threshold can
    # leave some streams with no passing chunk (the fallback)
    off = np.repeat(rng.uniform(-2, 2, size=B), n_list)
    cont = (rng.standard_normal(int(co[-1])) + off).astype(np.float32)
    ties = (np.round(cont * 2) / 2).astype(np.float32)          # heavy ties
    for s in (cont, ties):
        maxes = np.array([s[co[b]:co[b + 1]].max() for b in range(B)])
        taus = [np.quantile(s, 0.865), np.quantile(s, 0.5), float(np.median(maxes)),
                float(maxes.max()) + 1.0, -np.inf, float(s[0])]
        for tau in taus:
            for cap in (0, 1, 7, 276):
                _check_threshold(s, co, tau, cap)


def test_threshold_nan_and_signed_zero():
    s = np.array([np.nan, -0.0, 0.0, 1.0, np.nan, -1.0, 0.0], np.float32)
    co = np.array([0, 4, 7], np.int32)
    for tau in (0.0, -0.0, 0.5, 2.0, -np.inf):
        for cap in (0, 1, 2):
            _check_threshold(s, co, tau, cap)


def _retriever_attention(w, q, hw, rec, combine, tau_quantile, cap, streams=None):
    """Ensemble score -> threshold keep set -> sparse attention from the store,
    all on the device; the attention shape carries the bounds total_chunks /
    max_chunks since the kept counts are known on the device only."""
    c = w.cfg
    d = dev.upload(w, "cuda")
    s_gpu = _gpu_scores(w, q, hw, rec, combine)
    s_ref, _ = _check_scores(w, q, hw, rec, combine, s_gpu)
    tau = float(np.float32(np.quantile(s_ref, tau_quantile)))
    shape = dev.problem_shape(w)
    shape.max_k = shape.max_chunks       # the kept counts are known on the device only
    shape.total_k = shape.total_chunks
    shape.uniform = False
    off_d, idx_d, fb_d = lsa.select_threshold(shape, torch.from_numpy(s_gpu).cuda(), d.chunk_off,
                                              tau, cap)
    out, lse = lsa.sparse_decode_attn(shape, d.queries(0), d.K, d.V, d.tok_off, idx_d, off_d)
    torch.cuda.synchronize()
    off, fb = dev.to_host(off_d), dev.to_host(fb_d)
    idx = dev.to_host(idx_d)[:int(off[-1])]
    ref = oracle.select_threshold(s_gpu.astype(np.float64), w.chunk_off, tau, cap)
    np.testing.assert_array_equal(off, ref[0])
    np.testing.assert_array_equal(idx, ref[1])
    np.testing.assert_array_equal(fb, ref[2])
    streams = list(range(w.B)) if streams is None else streams
    outs, lses = [], []
    Q = w.queries(0)
    for b in streams:
        r0, r1 = int(w.tok_off[b]), int(w.tok_off[b + 1])
        sl = idx[off[b]:off[b + 1]]
        o, l = oracle.attention(Q[b:b + 1], w.K[r0:r1], None if w.V is None else w.V[r0:r1],
                                np.array([0, r1 - r0], np.int64), sl,
                                np.array([0, len(sl)], np.int32), c.chunk_size, c.softmax_scale,
                                dv=c.head_dim_v, nthreads=max(1, oracle.max_threads()))
        outs.append(o[0])
        lses.append(l[0])
    stats = P.check_attention(c.dtype, dev.to_host(out)[streams], dev.to_host(lse)[streams],
                              np.stack(outs), np.stack(lses))
    return off, fb, stats


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_retriever_path_small(name):
    w = wl.make_workload(wl.small_variant(name))
    q, hw, rec = wl.make_mh_layer_inputs(w, layers=3)
    for quantile, cap in ((0.865, 0), (0.5, 8), (0.9999999, 0)):
        off, fb, stats = _retriever_attention(w, q, hw, rec, oracle.COMBINE_MAX, quantile, cap)
        print(name, quantile, cap, np.diff(off).tolist(), fb.tolist(), stats)


def test_retriever_path_full_size():
    # 16 streams x 128K tokens, three layers of 2048 compressed-key records each
    w = wl.make_workload(wl.CONFIGS["cfg2"])
    q, hw, rec = wl.make_mh_layer_inputs(w, layers=3)
    off, fb, stats = _retriever_attention(w, q, hw, rec, oracle.COMBINE_MAX, 0.865, 0,
                                          streams=[0, w.B // 2, w.B - 1])
    print("cfg2 full", np.diff(off).tolist(), fb.tolist(), stats)
