"""lsa_decode_step_static (no workspace, allocates nothing) against
lsa_decode_step with a caller workspace, through the C ABI: two calls in a
row on one device -- the second on a smaller input, so the static scratch
still holds the first call's larger partials -- each bit-identical to the
workspace entry point and within the oracle's tolerances; and a shape whose
partials exceed the static scratch is refused before anything runs."""
import dataclasses

import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


def _static_step(d, t, reindex=True, pool=False):
    lsa.decode_step_static(d.shape, q_idx=d.q_idx, emb=d.emb, chunk_off=d.chunk_off,
                           scores=d.scores, sel_off=d.sel_off, sel_idx=d.sel_idx,
                           q=d.queries(t), k_store=d.K, v_store=d.V, tok_off=d.tok_off,
                           out=d.out, lse=d.lse, reindex=reindex, materialize_pool=pool,
                           k_pool=d.k_pool, v_pool=d.v_pool)


def _host(d):
    torch.cuda.synchronize()
    return dev.to_host(d.sel_idx), dev.to_host(d.out), dev.to_host(d.lse)


def _cfg(name):
    if name == "cfg1":
        return wl.CONFIGS["cfg1"]
    if name == "cfg5":  # eight ragged streams
        return wl.small_variant("cfg5", lengths=tuple(64 * (40 + 9 * i) + 7 * i for i in range(8)))
    return wl.small_variant(name)


@pytest.mark.parametrize("first,second", [("cfg5", "cfg2"), ("cfg4", "cfg1"), ("cfg3", "cfg2")])
def test_static_step_equals_workspace_step_twice(first, second):
    sizes = []
    for name in (first, second):  # the second input is the smaller one
        w = wl.make_workload(_cfg(name))
        d = dev.upload(w, "cuda", with_pool=bool(w.cfg.materialize_pool))
        sizes.append(lsa.workspace_bytes(d.shape))
        pool = bool(w.cfg.materialize_pool)
        d.step(0, reindex=True, materialize_pool=pool)
        sel_a, out_a, lse_a = _host(d)
        d.sel_idx.fill_(-1)
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        _static_step(d, 0, pool=pool)
        sel_b, out_b, lse_b = _host(d)
        np.testing.assert_array_equal(sel_b, sel_a)
        np.testing.assert_array_equal(out_b, out_a)
        np.testing.assert_array_equal(lse_b, lse_a)
        o_ref, l_ref = P.oracle_attention_on(w, 0, sel_b)
        print(name, P.check_attention(w.cfg.dtype, out_b, lse_b, o_ref, l_ref))
        # a step that reuses the kept set, fresh queries
        d.step(1, reindex=False, materialize_pool=pool)
        _, out_c, lse_c = _host(d)
        _static_step(d, 1, reindex=False, pool=pool)
        _, out_d, lse_d = _host(d)
        np.testing.assert_array_equal(out_d, out_c)
        np.testing.assert_array_equal(lse_d, lse_c)
    assert sizes[1] < sizes[0] <= lsa.STATIC_SCRATCH_BYTES, sizes


@pytest.mark.parametrize("name", ["cfg5", "cfg2"])
def test_static_step_replayed_from_a_graph(name):
    # the callers it is for capture it: a re-indexing step (its partials merged
    # in the kernel for the ragged batch, by the merge launch for 16 x 128K)
    # captured once, replayed three times with eager work and a different
    # eager step between the replays; every replay equals the eager step bit
    # for bit
    w = wl.make_workload(_cfg(name))
    d = dev.upload(w, "cuda")
    _static_step(d, 0)
    sel_e, out_e, lse_e = _host(d)
    d.queries(1)  # every input the loop uses exists before the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _static_step(d, 0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _static_step(d, 0)
    for _ in range(3):
        d.sel_idx.fill_(-1)
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        sel_r, out_r, lse_r = _host(d)
        np.testing.assert_array_equal(sel_r, sel_e)
        np.testing.assert_array_equal(out_r, out_e)
        np.testing.assert_array_equal(lse_r, lse_e)
        _static_step(d, 1, reindex=False)
        torch.cuda.synchronize()


def test_static_step_refuses_partials_beyond_the_scratch():
    w = wl.make_workload(wl.small_variant("cfg2"))
    d = dev.upload(w, "cuda")
    big = dataclasses.replace(d.shape, attn_tiles_per_block=1, num_q_heads=64,
                              total_k=d.shape.total_k * 64, max_k=d.shape.max_k * 64,
                              total_chunks=d.shape.total_chunks * 64,
                              max_chunks=d.shape.max_chunks * 64, uniform=False)
    assert lsa.workspace_bytes(big) > lsa.STATIC_SCRATCH_BYTES
    d.out.fill_(7.0)
    with pytest.raises(lsa.LsaError) as e:
        lsa.decode_step_static(big, q_idx=d.q_idx, emb=d.emb, chunk_off=d.chunk_off,
                               scores=d.scores, sel_off=d.sel_off, sel_idx=d.sel_idx,
                               q=d.queries(0), k_store=d.K, v_store=d.V, tok_off=d.tok_off,
                               out=d.out, lse=d.lse, reindex=False)
    assert e.value.status == lsa.LSA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert (dev.to_host(d.out) == 7.0).all()   # nothing ran
