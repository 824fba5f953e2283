"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (one lsa_decode_step per step, default split-KV plan).

The oracle recomputes every score and ranks every stream's chunks (cheap at
any size); attention is checked on every stream (for the ragged 32-stream
batch too), each against the oracle run on exactly that stream's rows.
Tolerances are those of tests/parity.py."""
import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


def _check_step(w, d, t, sel, streams):
    o_ref, l_ref = P.oracle_attention_on(w, t, sel, streams=streams)
    out = dev.to_host(d.out)[streams]
    lse = dev.to_host(d.lse)[streams]
    return P.check_attention(w.cfg.dtype, out, lse, o_ref, l_ref)


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg4", "cfg5"])
def test_full_size_decode_step(name):
    cfg = wl.CONFIGS[name]
    w = wl.make_workload(cfg)
    d = dev.upload(w, "cuda")
    print(f"{name}: sum L={int(w.lengths.sum())} sum N={int(w.chunk_off[-1])} "
          f"sum k={int(w.sel_off[-1])}", flush=True)

    d.step(0, materialize_pool=cfg.materialize_pool, reindex_every=cfg.reindex_every)
    torch.cuda.synchronize()
    s_gpu = dev.to_host(d.scores)
    sel = dev.to_host(d.sel_idx)
    s_ref = oracle.score(w.q_idx, w.emb, w.chunk_off)
    P.check_scores(w, s_gpu, s_ref)
    P.check_selection(w, s_gpu, sel, s_ref)
    P.check_needles(w, sel)
    streams = list(range(w.B))
    print(name, "step 0", _check_step(w, d, 0, sel, streams), flush=True)

    if cfg.materialize_pool:
        # the pool the step gathered is a bit-exact copy of the kept chunks
        C = cfg.chunk_size
        np.testing.assert_array_equal(dev.to_host(d.k_pool),
                                      oracle.gather(w.K, C, w.tok_off, sel, w.sel_off))
        if w.V is not None:
            np.testing.assert_array_equal(dev.to_host(d.v_pool),
                                          oracle.gather(w.V, C, w.tok_off, sel, w.sel_off))

    # a following step: without re-indexing when the schedule says so (the
    # kept set and pool are reused), else re-indexed with fresh queries
    d.step(1, materialize_pool=cfg.materialize_pool, reindex_every=cfg.reindex_every)
    torch.cuda.synchronize()
    sel1 = dev.to_host(d.sel_idx)
    np.testing.assert_array_equal(sel1, sel)  # same query embedding, same kept set
    print(name, "step 1", _check_step(w, d, 1, sel1, streams), flush=True)
