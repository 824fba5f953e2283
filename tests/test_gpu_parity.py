"""Parity of the HIP path (through the C ABI) with the CPU oracle on reduced
workloads: the same structure, dtypes and head shapes as the five benchmark
workloads, at lengths the oracle finishes in seconds, spanning many tiles and
ragged partial last chunks.  Tolerances are those of tests/parity.py."""
import math

import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu

SMALL = ["cfg1", "cfg2", "cfg3", "cfg4", "cfg5"]


def small_cfg(name):
    return wl.CONFIGS["cfg1"] if name == "cfg1" else wl.small_variant(name)


_cache = {}


def small_workload(name):
    if name not in _cache:
        w = wl.make_workload(small_cfg(name))
        _cache[name] = (w, dev.upload(w, "cuda", with_pool=True))
    return _cache[name]


@pytest.mark.parametrize("name", SMALL)
def test_phases_match_oracle(name):
    w, d = small_workload(name)
    s_gpu, sel, out, lse = P.run_phases(d, 0)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    P.check_needles(w, sel)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    print(name, P.check_attention(w.cfg.dtype, out, lse, o_ref, l_ref))


@pytest.mark.parametrize("name", SMALL)
def test_fused_step_equals_phases_and_reuses_selection(name):
    w, d = small_workload(name)
    _, sel_a, out_a, lse_a = P.run_phases(d, 0)
    d.sel_idx.fill_(-1)
    d.step(0, reindex=True, materialize_pool=w.cfg.materialize_pool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.to_host(d.sel_idx), sel_a)
    np.testing.assert_array_equal(dev.to_host(d.out), out_a)
    np.testing.assert_array_equal(dev.to_host(d.lse), lse_a)
    # next step: no re-index, fresh queries, same kept set
    d.scores.fill_(float("nan"))
    d.step(1, reindex=False, materialize_pool=w.cfg.materialize_pool)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.to_host(d.sel_idx), sel_a)
    o_ref, l_ref = P.oracle_attention_on(w, 1, sel_a)
    P.check_attention(w.cfg.dtype, dev.to_host(d.out), dev.to_host(d.lse), o_ref, l_ref)


@pytest.mark.parametrize("name", ["cfg2", "cfg3", "cfg1", "cfg4"])
def test_gather_is_bit_exact_and_pool_attention_matches_store(name):
    w, d = small_workload(name)
    _, sel, out_store, lse_store = P.run_phases(d, 0)
    s = d.shape
    lsa.gather_chunks(s, d.K, d.V, d.tok_off, d.sel_idx, d.sel_off, d.k_pool, d.v_pool)
    torch.cuda.synchronize()
    C = w.cfg.chunk_size
    np.testing.assert_array_equal(dev.to_host(d.k_pool),
                                  oracle.gather(w.K, C, w.tok_off, sel, w.sel_off))
    if w.V is not None:  # latent attention: V is part of K, there is no value pool
        np.testing.assert_array_equal(dev.to_host(d.v_pool),
                                      oracle.gather(w.V, C, w.tok_off, sel, w.sel_off))
    out, lse = lsa.sparse_decode_attn(s, d.queries(0), d.k_pool, d.v_pool, d.tok_off, d.sel_idx,
                                      d.sel_off, lsa.KV_POOL, workspace=d.workspace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.to_host(out), out_store)
    np.testing.assert_array_equal(dev.to_host(lse), lse_store)


def test_reindex_schedule_over_several_steps():
    cfg = wl.small_variant("cfg3", steps=5, reindex_every=2)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    Qs = [w.queries(t) for t in range(cfg.steps)]
    ref = oracle.decode(w.q_idx, w.emb, w.chunk_off, w.sel_off, Qs, w.K, w.V, w.tok_off,
                        cfg.chunk_size, cfg.softmax_scale, cfg.reindex_every,
                        nthreads=oracle.max_threads())
    for t in range(cfg.steps):
        d.step(t, reindex=(t % cfg.reindex_every == 0), materialize_pool=True)
        torch.cuda.synchronize()
        sel = dev.to_host(d.sel_idx)
        np.testing.assert_array_equal(sel, ref[t][0])   # no near-ties in this workload
        P.check_attention("bf16", dev.to_host(d.out), dev.to_host(d.lse), ref[t][1], ref[t][2])


def test_keep_all_equals_dense_attention():
    cfg = wl.small_variant("cfg2", keep_num=1, keep_den=1, n_needles=0)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    _, sel, out, lse = P.run_phases(d, 0)
    all_idx, all_off = oracle.all_chunks(w.tok_off, cfg.chunk_size)
    np.testing.assert_array_equal(sel, all_idx)
    o_ref, l_ref = oracle.attention(w.queries(0), w.K, w.V, w.tok_off, all_idx, all_off,
                                    cfg.chunk_size, cfg.softmax_scale,
                                    nthreads=oracle.max_threads())
    P.check_attention("bf16", out, lse, o_ref, l_ref)


def test_split_count_changes_results_only_by_rounding():
    # Each split rounds its softmax weights to bf16 relative to its own running
    # maximum, so different splits differ by that rounding (~2^-9 relative per
    # weight), never by more; every split must also meet the oracle bar.
    w, d = small_workload("cfg2")
    _, sel, out_a, lse_a = P.run_phases(d, 0)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    for per in [4, 8, 36, 256]:
        s = dev.problem_shape(w, attn_tiles_per_block=per)
        out, lse = lsa.sparse_decode_attn(s, d.queries(0), d.K, d.V, d.tok_off, d.sel_idx,
                                          d.sel_off)
        torch.cuda.synchronize()
        o, l = dev.to_host(out), dev.to_host(lse)
        P.check_attention("bf16", o, l, o_ref, l_ref)
        rel = np.linalg.norm(o - out_a, axis=-1) / np.linalg.norm(out_a, axis=-1)
        assert rel.max() <= 5e-3, (per, rel.max())
        assert np.abs(l - lse_a).max() <= 1e-5


def test_reruns_are_bit_identical():
    w, d = small_workload("cfg5")
    a = P.run_phases(d, 0)
    b = P.run_phases(d, 0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def _single_stream(w: wl.Workload, b: int) -> wl.Workload:
    r0, r1 = int(w.tok_off[b]), int(w.tok_off[b + 1])
    c0, c1 = int(w.chunk_off[b]), int(w.chunk_off[b + 1])
    cfg = w.cfg.replace(batch=1, lengths=(r1 - r0,))
    sub = wl.Workload(cfg=cfg, lengths=w.lengths[b:b + 1], tok_off=np.array([0, r1 - r0]),
                      chunk_off=np.array([0, c1 - c0], np.int32), keep=w.keep[b:b + 1],
                      sel_off=np.array([0, w.keep[b]], np.int32), q_idx=w.q_idx[b:b + 1],
                      emb=w.emb[c0:c1], needles=[w.needles[b]], K=w.K[r0:r1],
                      V=None if w.V is None else w.V[r0:r1])
    sub._q_cache = {0: np.ascontiguousarray(w.queries(0)[b:b + 1])}
    return sub


def test_a_stream_alone_equals_the_same_stream_in_a_batch():
    w, _ = small_workload("cfg5")
    full = dev.upload(w, "cuda", attn_tiles_per_block=8)
    _, sel, out, lse = P.run_phases(full, 0)
    for b in [0, w.B - 1]:
        one = dev.upload(_single_stream(w, b), "cuda", attn_tiles_per_block=8)
        _, sel1, out1, lse1 = P.run_phases(one, 0)
        np.testing.assert_array_equal(sel1, sel[w.sel_off[b]:w.sel_off[b + 1]])
        np.testing.assert_array_equal(out1[0], out[b])
        np.testing.assert_array_equal(lse1[0], lse[b])


# ----------------------------------------------------------------------------- select edge cases
def _select_case(scores_per_stream, keep):
    chunk_off = np.concatenate([[0], np.cumsum([len(s) for s in scores_per_stream])]).astype(np.int32)
    sel_off = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)
    scores = np.concatenate(scores_per_stream).astype(np.float32)
    shape = lsa.ProblemShape(batch=len(keep), chunk_size=64, index_dim=128, num_q_heads=16,
                             head_dim_qk=128, head_dim_v=128, v_aliases_k=False,
                             dtype=torch.bfloat16, softmax_scale=0.1,
                             max_chunks=int(np.diff(chunk_off).max()), max_k=int(max(keep)),
                             total_chunks=int(chunk_off[-1]), total_k=int(sel_off[-1]))
    t = lambda a: torch.from_numpy(a).cuda()
    sel = lsa.select_topk(shape, t(scores), t(chunk_off), t(sel_off))
    torch.cuda.synchronize()
    got = dev.to_host(sel)
    np.testing.assert_array_equal(got, oracle.select(scores.astype(np.float64), chunk_off, sel_off))
    return got


@pytest.mark.parametrize("n", [8192, 20000])
def test_select_long_streams_bucket_and_radix_paths(n):
    # long streams take the bucket pass first: continuous scores resolve there;
    # ties, NaN and infinities, an outlier that crowds every other score into
    # one bin, and a boundary bin over 64 keys send it to the radix passes
    rng = np.random.default_rng(n)
    cont = rng.standard_normal(n)
    ties = np.round(rng.standard_normal(n) * 4) / 4
    special = rng.standard_normal(n)
    special[rng.choice(n, 40, replace=False)] = np.nan
    special[:3] = [np.inf, -np.inf, -0.0]
    outlier = rng.standard_normal(n) * 1e-3
    outlier[n // 3] = 1e30
    dense = np.concatenate([rng.standard_normal(n - 200), np.full(200, 0.5)])
    subnormal = rng.standard_normal(n) * 1e-42
    streams = [cont, ties, special, outlier, dense, subnormal]
    for k in (1, 63, n // 8, n // 2, n - 1):
        _select_case(streams, [k] * len(streams))


def test_select_ties_nan_signed_zero_and_extremes():
    rng = np.random.default_rng(0)
    golden = np.array([0.5, 0.9, 0.5, 0.9, -0.0, 0.0, 0.1, np.nan], np.float32)
    for k in range(1, 9):
        _select_case([golden], [k])
    streams = [np.full(300, 0.25), rng.choice([-1.0, 0.0, -0.0, 2.0, np.nan], 1000),
               np.array([3.0]), rng.standard_normal(4097), np.array([np.inf, -np.inf, 1.0, np.nan]),
               rng.integers(0, 3, 17).astype(np.float64)]
    keeps = [7, 500, 1, 1000, 3, 17]
    _select_case(streams, keeps)
    for k in [1, 2, 999, 2048, 4095, 4096]:
        _select_case([rng.standard_normal(4096)], [k])


def test_select_radix_passes_that_stop_early():
    # the radix passes stop once every key of the chosen digit is kept; these
    # streams resolve after the first digit (4.0 against 0.25), after the
    # second (1.5 against 1.0: same leading byte), with a boundary digit that
    # is kept whole (two of 1.5 under 1.75) or must be split by index (five
    # of 1.5, two kept), with negative scores, and in a single-wave stream
    rng = np.random.default_rng(7)

    def mix(n, values, counts, rest):
        v = np.full(n, rest)
        idx = rng.permutation(n)
        at = 0
        for val, c in zip(values, counts):
            v[idx[at:at + c]] = val
            at += c
        return v

    cases = [(mix(2048, [4.0], [276], 0.25), 276),
             (mix(2048, [1.5], [276], 1.0), 276),
             (mix(2048, [1.75, 1.5], [274, 2], 1.0), 276),
             (mix(2048, [1.75, 1.5], [274, 5], 1.0), 276),
             (mix(3000, [-1.0, -1.5], [10, 90], -3.0), 100),
             (mix(3000, [-1.0, -1.5], [10, 90], -3.0), 50),
             (mix(40, [2.0, 1.5], [3, 4], 1.0), 7),
             (mix(40, [2.0, 1.5], [3, 4], 1.0), 5),
             (1.0 + rng.random(2048) * 2.0 ** -20, 276)]
    for v, k in cases:
        _select_case([v], [k])
    _select_case([v for v, _ in cases], [k for _, k in cases])


def test_select_large_streams():
    rng = np.random.default_rng(1)
    s = [rng.standard_normal(65536).astype(np.float32) * 1e-3,
         np.round(rng.standard_normal(20000), 2), rng.standard_normal(8192)]
    _select_case(s, [6000, 19999, 655])


# ----------------------------------------------------------------------------- shape coverage
@pytest.mark.parametrize("variant", [
    dict(num_q_heads=8),                                   # padded head group
    dict(num_q_heads=24),                                  # two head groups, partially padded
    dict(num_q_heads=32, head_dim_qk=64, head_dim_v=64),   # d = 64
    dict(num_q_heads=40),                                  # two teams, the second partly padded
    dict(num_q_heads=64),                                  # two teams of two head groups
    dict(num_q_heads=48, head_dim_qk=64, head_dim_v=64),   # two teams, d = 64
    dict(num_q_heads=12, head_dim_qk=96, head_dim_v=80),   # portable kernel, bf16
    dict(chunk_size=48),                                   # chunk not a multiple of the tile
    dict(chunk_size=128, index_dim=256),
    dict(chunk_size=16, index_dim=64),
])
def test_attention_shape_variants(variant):
    cfg = wl.small_variant("cfg2", **variant)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    s_gpu, sel, out, lse = P.run_phases(d, 0)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    print(variant, P.check_attention("bf16", out, lse, o_ref, l_ref))


# ----------------------------------------------------------------------------- MLA (absorbed latent)
def _mla_cfg(**kw):
    # three ragged streams with partial last chunks, a quarter of the chunks kept,
    # so that runs of several tiles start and end inside chunks
    base = dict(lengths=(128 * 61 + 37, 128 * 30, 128 * 47 + 100), keep_num=1, keep_den=4)
    base.update(kw)
    return wl.small_variant("cfg4", **base)


@pytest.mark.parametrize("per", [0, 1, 2, 3, 7, 40])
def test_mla_attention_split_variants(per):
    w = wl.make_workload(_mla_cfg())
    d = dev.upload(w, "cuda", attn_tiles_per_block=per)
    s_gpu, sel, out, lse = P.run_phases(d, 0)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    print(per, P.check_attention("bf16", out, lse, o_ref, l_ref))


@pytest.mark.parametrize("heads", [1, 7, 16, 40, 64])
def test_mla_attention_head_counts(heads):
    w = wl.make_workload(_mla_cfg(num_q_heads=heads, kv_std=1.0, q_std=1.0))
    d = dev.upload(w, "cuda", attn_tiles_per_block=5)
    _, sel, out, lse = P.run_phases(d, 0)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    rel = np.linalg.norm(out - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)
    assert rel.max() <= 1e-2, rel.max()
    assert (np.abs(lse - l_ref) / np.abs(l_ref)).max() <= 1e-4


def test_fp32_portable_attention_ragged():
    cfg = wl.small_variant("cfg1", lengths=(4096 + 17, 300, 64 * 40), keep_num=1, keep_den=4)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    s_gpu, sel, out, lse = P.run_phases(d, 0)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    P.check_attention("f32", out, lse, o_ref, l_ref)


@pytest.mark.parametrize("std", [1.0, 3.0])
def test_stress_large_logits(std):
    # unscaled keys and queries: logits of O(10)-O(100), far from uniform weights
    cfg = wl.small_variant("cfg2", kv_std=std, q_std=std)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    _, sel, out, lse = P.run_phases(d, 0)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    rel = np.linalg.norm(out - o_ref, axis=-1) / np.linalg.norm(o_ref, axis=-1)
    assert rel.max() <= 1e-2, rel.max()
    assert (np.abs(lse - l_ref) / np.abs(l_ref)).max() <= 1e-4


def test_hot_token_dominates():
    cfg = wl.small_variant("cfg2", n_needles=8)
    w = wl.make_workload(cfg)
    # plant, in stream 1, a key row equal to 40x head 3's query: one token takes ~all weight
    sel_full = oracle.select(oracle.score(w.q_idx, w.emb, w.chunk_off), w.chunk_off, w.sel_off)
    b, h = 1, 3
    n = int(sel_full[w.sel_off[b] + 2])
    row = int(w.tok_off[b]) + n * cfg.chunk_size + 5
    q = wl.as_f32(w.queries(0))[b, h]
    w.K[row] = wl.to_bf16_bits(40.0 * q / np.linalg.norm(q) * math.sqrt(cfg.head_dim_qk))
    d = dev.upload(w, "cuda")
    _, sel, out, lse = P.run_phases(d, 0)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    P.check_attention("bf16", out, lse, o_ref, l_ref)
    v = wl.as_f32(w.V[row])
    assert np.abs(out[b, h] - v).max() < 0.05 * np.abs(v).max()


def test_workspace_is_reusable_across_calls_and_shapes():
    # one workspace serves calls of different shapes, repeatedly
    wa, da = small_workload("cfg2")
    wb, db = small_workload("cfg5")
    big = torch.zeros(max(da.workspace.numel(), db.workspace.numel()), dtype=torch.uint8,
                      device="cuda")
    _, _, out_a, lse_a = P.run_phases(da, 0)
    _, _, out_b, lse_b = P.run_phases(db, 0)
    for _ in range(3):
        for d, out_ref, lse_ref in [(da, out_a, lse_a), (db, out_b, lse_b)]:
            out, lse = lsa.sparse_decode_attn(d.shape, d.queries(0), d.K, d.V, d.tok_off,
                                              d.sel_idx, d.sel_off, workspace=big)
            d.step(0, reindex=True)  # fused score+select uses the other counters
            torch.cuda.synchronize()
            np.testing.assert_array_equal(dev.to_host(out), out_ref)
            np.testing.assert_array_equal(dev.to_host(lse), lse_ref)


# ----------------------------------------------------------------------------- uniform shapes
@pytest.mark.parametrize("name", ["cfg2", "cfg3", "cfg4"])
def test_uniform_shape_flag_is_only_a_shortcut(name):
    # equal stream lengths: every stream has the same chunk and kept counts, so
    # the shape may carry LSA_SHAPE_UNIFORM; with and without it the decode
    # step (score, select, gather, attention, merge) must give the same bits
    L = wl.small_variant(name).lengths[0]
    cfg = wl.small_variant(name, lengths=(L, L, L))
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    assert d.shape.uniform
    results = []
    for uniform in (True, False):
        d.shape.uniform = uniform
        d.sel_idx.zero_()
        d.out.zero_()
        d.lse.zero_()
        d.step(0, reindex=True, materialize_pool=cfg.materialize_pool)
        torch.cuda.synchronize()
        results.append([dev.to_host(t).copy() for t in (d.sel_idx, d.out, d.lse)])
    d.shape.uniform = True
    for a, b in zip(*results):
        np.testing.assert_array_equal(a, b)
    sel, out, lse = results[0]
    s_gpu = dev.to_host(d.scores)
    P.check_selection(w, s_gpu, sel, oracle.score(w.q_idx, w.emb, w.chunk_off))
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    P.check_attention(cfg.dtype, out, lse, o_ref, l_ref)


@pytest.mark.parametrize("uniform", [False, True])
def test_more_than_64_streams(uniform):
    # the work plan and the merge look streams up 64 at a time: 80 streams
    # cross that window (ragged lengths, or all equal for the uniform shape)
    rng = np.random.default_rng(80)
    if uniform:
        lengths = (64 * 70 + 13,) * 80
    else:
        lengths = tuple(int(x) for x in rng.integers(64 * 64, 64 * 90, size=80))
    cfg = wl.small_variant("cfg2", lengths=lengths)
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    assert d.shape.uniform == uniform
    s_gpu, sel, out, lse = P.run_phases(d, 0)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    o_ref, l_ref = P.oracle_attention_on(w, 0, sel)
    P.check_attention("bf16", out, lse, o_ref, l_ref)
