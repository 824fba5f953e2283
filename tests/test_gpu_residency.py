"""Parity of delta residency (lsa_pool_delta_update) with the CPU oracle,
through the C ABI: over re-index epochs whose indexer query drifts, the slot
table, the list and number of loaded slots are identical to the oracle's;
the pool is bit-identical to the oracle's gather of the new table (so slots
that were not loaded kept their bytes, and loaded ones came from the pinned
host store); attention read from the pool through the table (chunks in slot
order) matches the oracle over the kept set within tests/parity.py's
tolerances."""
import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


def _pinned(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) \
        if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))
    return t.pin_memory()


def _run_epochs(w, epochs=4, eps=0.5, attention=True):
    c = w.cfg
    d = dev.upload(w, "cuda")
    shape = d.shape
    kh = _pinned(w.K)
    vh = None if w.V is None else _pinned(w.V)
    dt = shape.dtype
    k_pool = torch.empty((shape.total_k, c.chunk_size, c.head_dim_qk), dtype=dt, device="cuda")
    v_pool = None if w.V is None else torch.empty((shape.total_k, c.chunk_size, c.head_dim_v),
                                                  dtype=dt, device="cuda")
    table = torch.full((shape.total_k,), -1, dtype=torch.int32, device="cuda")
    churn = []
    for e in range(epochs):
        q = wl.drift_query(w, e, eps)
        qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda() if q.dtype == np.uint16 \
            else torch.from_numpy(q).cuda()
        scores = lsa.score(shape, qd, d.emb, d.chunk_off)
        sel = lsa.select_topk(shape, scores, d.chunk_off, d.sel_off)
        torch.cuda.synchronize()
        before = dev.to_host(table)
        loads, cnt = lsa.pool_delta_update(shape, kh, vh, d.tok_off, d.chunk_off, sel, d.sel_off,
                                           table, k_pool, v_pool)
        torch.cuda.synchronize()
        sel_h, tab, ld, n = (dev.to_host(x) for x in (sel, table, loads, cnt))
        r_tab, r_ld, r_n = oracle.pool_delta(w.chunk_off, sel_h, w.sel_off, before)
        np.testing.assert_array_equal(tab, r_tab)
        np.testing.assert_array_equal(n, r_n)
        for b in range(w.B):
            s0 = w.sel_off[b]
            np.testing.assert_array_equal(ld[s0:s0 + n[b]], r_ld[s0:s0 + n[b]])
        np.testing.assert_array_equal(dev.to_host(k_pool).reshape(shape.total_k, -1),
                                      oracle.gather(w.K, c.chunk_size, w.tok_off, tab, w.sel_off)
                                      .reshape(shape.total_k, -1))
        if v_pool is not None:
            np.testing.assert_array_equal(
                dev.to_host(v_pool).reshape(shape.total_k, -1),
                oracle.gather(w.V, c.chunk_size, w.tok_off, tab, w.sel_off)
                .reshape(shape.total_k, -1))
        churn.append(int(n.sum()))
        if attention:
            out, lse = lsa.sparse_decode_attn(shape, d.queries(e), k_pool, v_pool, d.tok_off,
                                              table, d.sel_off, lsa.KV_POOL)
            torch.cuda.synchronize()
            o_ref, l_ref = oracle.attention(w.queries(e), w.K, w.V, w.tok_off, sel_h, w.sel_off,
                                            c.chunk_size, c.softmax_scale, dv=c.head_dim_v,
                                            nthreads=max(1, oracle.max_threads()))
            P.check_attention(c.dtype, dev.to_host(out), dev.to_host(lse), o_ref, l_ref)
    assert churn[0] == int(w.sel_off[-1])          # the first epoch loads every kept chunk
    return churn


@pytest.mark.parametrize("name", ["cfg3", "cfg5", "cfg4", "cfg1"])
def test_delta_residency_small(name):
    w = wl.make_workload(wl.small_variant(name))
    churn = _run_epochs(w)
    print(name, "chunks loaded per epoch", churn)
    assert sum(churn[1:]) > 0, "the drifting query never changed the kept set"


def test_delta_residency_repeated_set_loads_nothing():
    w = wl.make_workload(wl.small_variant("cfg3"))
    churn = _run_epochs(w, epochs=3, eps=0.0, attention=False)
    assert churn[1:] == [0, 0]


def test_delta_residency_full_size_pool_workload():
    # 4 streams x 512K tokens, 819 kept chunks per stream; epochs of a drifting query
    w = wl.make_workload(wl.CONFIGS["cfg3"])
    churn = _run_epochs(w, epochs=3, attention=False)
    print("cfg3 full: chunks loaded per epoch", churn)
