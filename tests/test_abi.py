"""Host-side checks of the C ABI (include/lsa.h) that need no GPU: the library
loads and exports every declared entry point, the integer helpers agree with
the oracle's independent implementation, workspace sizing is monotone, and
every invalid call is rejected with its documented status before anything is
enqueued (the dummy pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

from learned_kv_chunk_amd import lsa
from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lsa.LIB_PATH),
                                reason="liblsa.so not built (run __graft_entry__.build())")


def declared_entry_points():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_entry_points()
    assert len(names) >= 11, names
    lib = ctypes.CDLL(lsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lsa.h but not exported"
    assert set(names) == set(lsa._SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    assert lsa.library().lsa_abi_version() == 4
    for code, name in [(0, "LSA_OK"), (1, "LSA_ERR_INVALID_ARGUMENT"), (2, "LSA_ERR_UNSUPPORTED"),
                       (3, "LSA_ERR_WORKSPACE_TOO_SMALL"), (4, "LSA_ERR_HIP")]:
        assert lsa.status_string(code) == name
    assert lsa.status_string(99) == "LSA_ERR_UNKNOWN"


def test_keep_count_agrees_with_oracle():
    for n in list(range(0, 300)) + [2048, 4096, 8192, 65536]:
        for num, den in [(135, 1000), (1, 8), (10, 100), (8, 100), (1, 1), (3, 2)]:
            for up in (False, True):
                assert lsa.keep_count(n, num, den, up) == oracle.keep_count(n, num, den, up)
    assert lsa.keep_count(2048, 135, 1000, False) == 276
    assert lsa.keep_count(5, 0, 1, False) == 0


def shape(**kw):
    base = dict(batch=16, chunk_size=64, index_dim=128, num_q_heads=16, head_dim_qk=128,
                head_dim_v=128, v_aliases_k=False, dtype=torch.bfloat16,
                softmax_scale=128 ** -0.5, max_chunks=2048, max_k=276, total_chunks=16 * 2048,
                total_k=16 * 276)
    base.update(kw)
    return lsa.ProblemShape(**base)


def test_attention_plan_names_kernel_merge_and_form():
    # no GPU here: the plan is made for the 256 compute units of an MI355X
    p = lsa.attention_plan(shape())
    assert p["kernel"] == "attn_mqa" and not p["split_heads"] and p["tiles_per_chunk"] == 2
    assert not p["merge_in_kernel"] and p["select_in_kernel"]  # 16 workgroups per stream
    assert p["grid"] >= 256 and p["partial_rows"] >= p["grid"]
    # 32 ragged streams: eight workgroups each on average, merged in the kernel
    p = lsa.attention_plan(shape(batch=32, max_chunks=4096, max_k=553, total_chunks=68733,
                                 total_k=9294))
    assert p["merge_in_kernel"] and p["select_in_kernel"]
    mla = lsa.attention_plan(shape(batch=1, chunk_size=128, index_dim=256, num_q_heads=64,
                                   head_dim_qk=576, head_dim_v=512, v_aliases_k=True,
                                   max_chunks=8192, max_k=655, total_chunks=8192, total_k=655))
    assert mla["kernel"] == "attn_mla" and not mla["merge_in_kernel"]
    assert not mla["select_in_kernel"] and mla["tiles_per_chunk"] == 4
    # the 4K fp32 workload: 16 tiles, the split-heads form, merged in the kernel
    f32 = dict(batch=1, index_dim=64, num_q_heads=8, head_dim_qk=64, head_dim_v=64,
               dtype=torch.float32, max_chunks=64, max_k=8, total_chunks=64, total_k=8)
    p = lsa.attention_plan(shape(**f32))
    assert p["kernel"] == "attn_portable" and p["split_heads"] and p["merge_in_kernel"]
    assert p["select_in_kernel"]
    # more tiles than compute units: the tile-parallel form, no top-k inside
    p = lsa.attention_plan(shape(**dict(f32, max_chunks=4096, max_k=600, total_chunks=4096,
                                        total_k=600)))
    assert not p["split_heads"] and not p["select_in_kernel"]
    with pytest.raises(lsa.LsaError):
        lsa.attention_plan(shape(num_q_heads=100))


def test_workspace_sizes_positive_and_monotone():
    ws = lsa.workspace_bytes
    assert ws(shape()) > 0
    assert ws(shape(batch=1, total_chunks=2048, total_k=276)) <= ws(shape())
    assert ws(shape(num_q_heads=8)) <= ws(shape())
    assert ws(shape(head_dim_qk=64, head_dim_v=64)) <= ws(shape())
    prev = 0
    for k in [1, 8, 64, 276, 1000, 2048]:
        cur = ws(shape(max_k=k, total_k=16 * k))
        assert cur >= prev
        prev = cur
    # the five workload shapes are all supported
    assert ws(shape(batch=1, chunk_size=64, index_dim=64, num_q_heads=8, head_dim_qk=64,
                    head_dim_v=64, dtype=torch.float32, max_chunks=64, max_k=8, total_chunks=64,
                    total_k=8)) > 0
    assert ws(shape(batch=4, num_q_heads=32, max_chunks=8192, max_k=819, total_chunks=4 * 8192,
                    total_k=4 * 819)) > 0
    # invalid shapes report 0
    assert ws(shape(batch=0)) == 0
    assert ws(shape(total_k=10 ** 9)) == 0


DUMMY = ctypes.c_void_p(0x100000)  # aligned, never dereferenced


def _score(s, q=DUMMY, e=DUMMY, off=DUMMY, out=DUMMY):
    return lsa.library().lsa_score(ctypes.byref(s.c()), q, e, off, out, None)


def _select(s, sc=DUMMY, off=DUMMY, soff=DUMMY, idx=DUMMY):
    return lsa.library().lsa_select_topk(ctypes.byref(s.c()), sc, off, soff, idx, None)


def _attn(s, ws_bytes=None, kv_mode=0, v=DUMMY, ws=DUMMY, q=DUMMY, lse=DUMMY):
    if ws_bytes is None:
        ws_bytes = max(lsa.workspace_bytes(s), 1)
    return lsa.library().lsa_sparse_decode_attn(ctypes.byref(s.c()), kv_mode, q, DUMMY, v, DUMMY,
                                                DUMMY, DUMMY, DUMMY, lse, ws, ws_bytes, None)


def _gather(s, v_store=DUMMY, v_pool=DUMMY):
    return lsa.library().lsa_gather_chunks(ctypes.byref(s.c()), DUMMY, v_store, DUMMY, DUMMY,
                                           DUMMY, DUMMY, v_pool, None)


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(chunk_size=0), dict(chunk_size=2048), dict(max_chunks=0),
    dict(max_k=0), dict(max_k=3000), dict(total_chunks=15), dict(total_chunks=16 * 2048 + 1),
    dict(total_k=15), dict(total_k=16 * 276 + 1), dict(attn_tiles_per_block=-1),
    # a uniform shape must have total_chunks = B * max_chunks and total_k = B * max_k
    dict(uniform=True, total_chunks=16 * 2048 - 1), dict(uniform=True, total_k=16 * 276 - 1),
])
def test_invalid_shapes_rejected_everywhere(bad):
    s = shape(**bad)
    assert _score(s) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _select(s) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _attn(s) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _gather(s) == lsa.LSA_ERR_INVALID_ARGUMENT


def test_shape_flags():
    # LSA_SHAPE_UNIFORM is the only flag; a consistent uniform shape is accepted
    c = shape(uniform=True).c()
    assert c.flags == lsa.SHAPE_UNIFORM
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(c)) > 0
    c.flags = 2
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(c)) == 0
    assert shape().c().flags == 0


def test_null_and_misaligned_pointers_rejected():
    s = shape()
    assert _score(s, q=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _score(s, out=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _score(s, e=ctypes.c_void_p(0x100008)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _select(s, idx=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _select(s, sc=ctypes.c_void_p(0x100002)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _attn(s, q=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _attn(s, ws=ctypes.c_void_p(0x100010)) == lsa.LSA_ERR_INVALID_ARGUMENT  # not 256-aligned
    assert _attn(s, v=None) == lsa.LSA_ERR_INVALID_ARGUMENT        # separate V required
    assert _attn(s, kv_mode=7) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _gather(s, v_store=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert lsa.library().lsa_score(None, DUMMY, DUMMY, DUMMY, DUMMY, None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT
    assert lsa.library().lsa_decode_step(None, None, DUMMY, 1, None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert lsa.library().lsa_bench_copy(DUMMY, DUMMY, 17, None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert lsa.library().lsa_bench_flush(None, 16, None) == lsa.LSA_ERR_INVALID_ARGUMENT


def test_reindex_schedule_helper_and_step_arg_checks():
    lib = lsa.library()
    assert [lib.lsa_reindex_due(t, 3) for t in range(8)] == [1, 0, 0, 1, 0, 0, 1, 0]
    assert [lib.lsa_reindex_due(t, 1) for t in range(4)] == [1, 1, 1, 1]
    assert lib.lsa_reindex_due(64 * 5, 64) == 1 and lib.lsa_reindex_due(64 * 5 + 1, 64) == 0
    assert lib.lsa_reindex_due(2 ** 40, 64) == 1
    assert lib.lsa_reindex_due(0, 0) == -1 and lib.lsa_reindex_due(-1, 4) == -1
    assert lsa.reindex_due(6, 3) and not lsa.reindex_due(7, 3)
    with pytest.raises(ValueError):
        lsa.reindex_due(1, 0)
    s = shape()
    ws = lsa.workspace_bytes(s)
    base = dict(q_idx_dev=DUMMY, emb_dev=DUMMY, chunk_off_dev=DUMMY, scores_dev=DUMMY,
                sel_off_dev=DUMMY, sel_idx_dev=DUMMY, q_dev=DUMMY, k_store_dev=DUMMY,
                v_store_dev=DUMMY, tok_off_dev=DUMMY, out_dev=DUMMY)
    for bad in [dict(reindex_every=-1), dict(reindex_every=4, step=-3), dict(reserved=1)]:
        a = lsa.StepArgs(**base, **bad)
        assert lib.lsa_decode_step(ctypes.byref(s.c()), ctypes.byref(a), DUMMY, ws, None) == \
            lsa.LSA_ERR_INVALID_ARGUMENT, bad
    # with the schedule in charge, a re-index step needs the scoring inputs
    a = lsa.StepArgs(**dict(base, q_idx_dev=None), reindex_every=4, step=8)
    assert lib.lsa_decode_step(ctypes.byref(s.c()), ctypes.byref(a), DUMMY, ws, None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT


def test_static_step_checks_before_touching_the_device():
    # no GPU is needed: every refusal happens before the scratch is looked up
    lib = lsa.library()
    base = dict(q_idx_dev=DUMMY, emb_dev=DUMMY, chunk_off_dev=DUMMY, scores_dev=DUMMY,
                sel_off_dev=DUMMY, sel_idx_dev=DUMMY, q_dev=DUMMY, k_store_dev=DUMMY,
                v_store_dev=DUMMY, tok_off_dev=DUMMY, out_dev=DUMMY, reindex=1)
    s = shape()
    assert lib.lsa_decode_step_static(None, ctypes.byref(lsa.StepArgs(**base)), None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT
    assert lib.lsa_decode_step_static(ctypes.byref(s.c()), None, None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT
    a = lsa.StepArgs(**dict(base, q_dev=None))
    assert lib.lsa_decode_step_static(ctypes.byref(s.c()), ctypes.byref(a), None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT
    a = lsa.StepArgs(**base, reindex_every=-2)
    assert lib.lsa_decode_step_static(ctypes.byref(s.c()), ctypes.byref(a), None) == \
        lsa.LSA_ERR_INVALID_ARGUMENT
    big = shape(attn_tiles_per_block=1)   # one partial per 32-token tile: 73 MB
    assert lsa.workspace_bytes(big) > lsa.STATIC_SCRATCH_BYTES
    a = lsa.StepArgs(**base)
    assert lib.lsa_decode_step_static(ctypes.byref(big.c()), ctypes.byref(a), None) == \
        lsa.LSA_ERR_WORKSPACE_TOO_SMALL
    assert lsa.workspace_bytes(shape()) <= lsa.STATIC_SCRATCH_BYTES


def test_alias_requires_null_value_pointers():
    s = shape(v_aliases_k=True, head_dim_qk=576, head_dim_v=512, num_q_heads=64)
    assert _gather(s) == lsa.LSA_ERR_INVALID_ARGUMENT           # V pointers must be NULL
    assert _attn(s, v=DUMMY) in (lsa.LSA_ERR_INVALID_ARGUMENT, lsa.LSA_ERR_UNSUPPORTED)


def test_unsupported_shapes():
    assert _score(shape(index_dim=12)) == lsa.LSA_ERR_UNSUPPORTED       # 24 bytes per row
    assert _score(shape(index_dim=2048)) == lsa.LSA_ERR_UNSUPPORTED
    assert _select(shape(max_chunks=70000, total_chunks=16 * 70000)) == lsa.LSA_ERR_UNSUPPORTED
    assert _attn(shape(num_q_heads=100)) == lsa.LSA_ERR_UNSUPPORTED
    assert _attn(shape(head_dim_qk=96, head_dim_v=80, num_q_heads=32)) == lsa.LSA_ERR_UNSUPPORTED
    assert _attn(shape(head_dim_qk=12)) == lsa.LSA_ERR_UNSUPPORTED       # 24-byte rows
    assert lsa.workspace_bytes(shape(num_q_heads=100)) == 0


def test_workspace_too_small():
    s = shape()
    need = lsa.workspace_bytes(s)
    assert _attn(s, ws_bytes=need - 1) == lsa.LSA_ERR_WORKSPACE_TOO_SMALL


def test_python_layer_rejects_host_tensors():
    s = shape()
    with pytest.raises(ValueError):
        lsa.score(s, torch.zeros(16, 128, dtype=torch.bfloat16),
                  torch.zeros(16 * 2048, 128, dtype=torch.bfloat16),
                  torch.zeros(17, dtype=torch.int32))


def test_workspace_holds_every_partial():
    # one partial (max, sum, output row) per head for every workgroup the plan
    # can launch
    for per in [4, 8, 64, 256]:
        for B, k, H, dv in [(1, 8, 8, 64), (16, 276, 16, 128), (4, 819, 32, 128)]:
            s = shape(batch=B, max_k=k, total_k=B * k, num_q_heads=H, head_dim_qk=dv,
                      head_dim_v=dv, attn_tiles_per_block=per, max_chunks=max(2048, k),
                      total_chunks=B * max(2048, k))
            tiles = B * k * 2
            wgs = -(-tiles // per) + B
            need = wgs * H * (dv + 2) * 4
            assert lsa.workspace_bytes(s) >= need, (per, B, k, H, dv)


def test_workspace_holds_every_mla_partial():
    # absorbed MLA: the output rows of its partials are bf16 (2 bytes per
    # latent column), the maxima and sums fp32
    for per in [4, 8, 64, 256]:
        for H, k in [(64, 655), (16, 40), (1, 8)]:
            s = shape(batch=1, max_k=k, total_k=k, num_q_heads=H, head_dim_qk=576,
                      head_dim_v=512, v_aliases_k=1, chunk_size=128,
                      softmax_scale=576 ** -0.5, attn_tiles_per_block=per,
                      max_chunks=8192, total_chunks=8192, index_dim=256)
            tiles = k * 4
            wgs = -(-tiles // per) + 1
            need = wgs * H * (512 * 2 + 2 * 4)
            assert lsa.workspace_bytes(s) >= need, (per, H, k)
    # the 1M-token shape's default plan (about 256 workgroups): half of what
    # fp32 rows would take
    s = shape(batch=1, max_k=655, total_k=655, num_q_heads=64, head_dim_qk=576,
              head_dim_v=512, v_aliases_k=1, chunk_size=128, softmax_scale=576 ** -0.5,
              max_chunks=8192, total_chunks=8192, index_dim=256)
    assert lsa.workspace_bytes(s) < 256 * 64 * 512 * 4


def _mh(s, heads=128, dim=128, q=DUMMY, w=DUMMY, rec=DUMMY, co=DUMMY, out=DUMMY):
    return lsa.library().lsa_score_fp8_multihead(ctypes.byref(s.c()), heads, dim, q, w, rec, co,
                                                 out, None)


def test_multihead_scorer_validation():
    s = shape()
    assert _mh(s, q=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mh(s, out=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mh(s, q=ctypes.c_void_p(0x100008)) == lsa.LSA_ERR_INVALID_ARGUMENT   # 16-byte aligned
    assert _mh(s, rec=ctypes.c_void_p(0x100002)) == lsa.LSA_ERR_INVALID_ARGUMENT  # 4-byte aligned
    assert _mh(s, heads=0) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mh(shape(batch=0)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mh(s, heads=48) == lsa.LSA_ERR_UNSUPPORTED
    assert _mh(s, dim=96) == lsa.LSA_ERR_UNSUPPORTED
    assert _mh(shape(dtype=torch.float32)) == lsa.LSA_ERR_UNSUPPORTED


def _mhl(s, layers=3, combine=lsa.COMBINE_MAX, heads=128, dim=128, q=DUMMY, w=DUMMY, rec=DUMMY,
         co=DUMMY, out=DUMMY):
    return lsa.library().lsa_score_fp8_multihead_layers(ctypes.byref(s.c()), layers, combine,
                                                        heads, dim, q, w, rec, co, out, None)


def test_layer_ensemble_scorer_validation():
    s = shape()
    assert _mhl(s, layers=0) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, layers=17) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, combine=2) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, combine=-1) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, w=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, q=ctypes.c_void_p(0x100004)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _mhl(s, heads=8) == lsa.LSA_ERR_UNSUPPORTED
    assert _mhl(shape(dtype=torch.float32)) == lsa.LSA_ERR_UNSUPPORTED


def _thr(s, tau=0.5, cap=0, scores=DUMMY, co=DUMMY, off=DUMMY, idx=DUMMY, fb=DUMMY, ws=DUMMY,
         ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lsa.select_threshold_workspace_bytes(s)
    return lsa.library().lsa_select_threshold(ctypes.byref(s.c()), scores, co, tau, cap, off, idx,
                                              fb, ws, ws_bytes, None)


def test_threshold_select_validation():
    s = shape()
    need = lsa.select_threshold_workspace_bytes(s)
    assert need >= 4 * s.batch and need % 256 == 0
    assert lsa.select_threshold_workspace_bytes(shape(batch=0)) == 0
    assert _thr(s, tau=float("nan")) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, cap=-1) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, scores=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, off=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, idx=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, ws=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, ws=ctypes.c_void_p(0x100080)) == lsa.LSA_ERR_INVALID_ARGUMENT  # 256-byte aligned
    assert _thr(s, fb=ctypes.c_void_p(0x100002)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _thr(s, ws_bytes=need - 1) == lsa.LSA_ERR_WORKSPACE_TOO_SMALL
    assert _thr(shape(max_chunks=65537, total_chunks=16 * 65537)) == lsa.LSA_ERR_UNSUPPORTED


def _delta(s, k_host, v_host=DUMMY, pool_v=DUMMY, **kw):
    args = dict(tok=DUMMY, co=DUMMY, sel=DUMMY, so=DUMMY, table=DUMMY, loads=DUMMY, cnt=DUMMY,
                pool_k=DUMMY)
    args.update(kw)
    return lsa.library().lsa_pool_delta_update(
        ctypes.byref(s.c()), k_host, v_host, args["tok"], args["co"], args["sel"], args["so"],
        args["table"], args["loads"], args["cnt"], args["pool_k"], pool_v, None)


def test_pool_delta_validation():
    import numpy as np
    s = shape()
    plain = np.zeros(4096, np.uint8)            # ordinary (not page-locked) host memory
    p = ctypes.c_void_p(plain.ctypes.data)
    assert _delta(s, None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _delta(s, DUMMY, table=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _delta(s, DUMMY, v_host=None) == lsa.LSA_ERR_INVALID_ARGUMENT   # V needed
    assert _delta(shape(v_aliases_k=True, head_dim_v=64), DUMMY) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _delta(s, DUMMY, loads=ctypes.c_void_p(0x100002)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert _delta(shape(max_chunks=65537, total_chunks=16 * 65537), DUMMY) == \
        lsa.LSA_ERR_UNSUPPORTED
    assert _delta(shape(head_dim_qk=6, head_dim_v=6, dtype=torch.float32), DUMMY) == \
        lsa.LSA_ERR_UNSUPPORTED                                             # 16-byte rows
    # pointers that are not page-locked host memory are refused before any launch
    assert _delta(s, p, v_host=p) == lsa.LSA_ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        lsa.pool_delta_update(lsa.ProblemShape(**{**dict(
            batch=1, chunk_size=64, index_dim=128, num_q_heads=16, head_dim_qk=128,
            head_dim_v=128, v_aliases_k=False, dtype=torch.bfloat16, softmax_scale=0.1,
            max_chunks=4, max_k=2, total_chunks=4, total_k=2)}),
            torch.zeros(256, 128, dtype=torch.bfloat16), None, None, None, None, None, None,
            None)


def test_append_and_keep_recent_validation():
    s = shape()
    lib = lsa.library()
    ap = lambda sh, kn=DUMMY, vn=DUMMY, bo=DUMMY, sl=DUMMY, ks=DUMMY, vs=DUMMY: \
        lib.lsa_append_kv(ctypes.byref(sh.c()), kn, vn, bo, sl, ks, vs, None)
    assert ap(s, kn=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert ap(s, vn=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert ap(shape(v_aliases_k=True, head_dim_v=64)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert ap(s, sl=ctypes.c_void_p(0x100004)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert ap(shape(head_dim_qk=6, head_dim_v=6, dtype=torch.float32)) == lsa.LSA_ERR_UNSUPPORTED
    kr = lambda sh, mr=4, sl=DUMMY, oi=DUMMY: lib.lsa_keep_recent(
        ctypes.byref(sh.c()), sl, DUMMY, DUMMY, DUMMY, mr, oi, DUMMY, None)
    assert kr(s, mr=-1) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert kr(s, sl=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert kr(s, oi=ctypes.c_void_p(0x100002)) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert kr(shape(batch=0)) == lsa.LSA_ERR_INVALID_ARGUMENT
    need = lsa.workspace_bytes(s)
    av = lambda sh, sl=DUMMY: lib.lsa_sparse_decode_attn_varlen(
        ctypes.byref(sh.c()), lsa.KV_STORE, DUMMY, DUMMY, DUMMY, DUMMY, sl, DUMMY, DUMMY, DUMMY,
        DUMMY, DUMMY, need, None)
    assert av(s, sl=None) == lsa.LSA_ERR_INVALID_ARGUMENT
    assert av(s, sl=ctypes.c_void_p(0x100004)) == lsa.LSA_ERR_INVALID_ARGUMENT


def test_header_compiles_as_c_and_links(tmp_path):
    # include/lsa.h from plain C99, linked against liblsa.so: the host-side
    # calls that need no GPU behave as the header states
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_from_c.c")
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(lsa.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-o", exe, src,
                        "-L" + libdir, "-llsa", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "abi_from_c ok" in r.stdout, r.stdout + r.stderr
