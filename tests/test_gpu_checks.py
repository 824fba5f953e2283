"""lsa_check_tables on the device: every table of tests/table_cases.py (each
breaking one precondition, every entry inside the documented array sizes)
reports exactly its error bits, as the host build of the same checks does;
and the Python layer's debug mode stops a decode step whose kept indices are
out of range before anything runs."""
import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from tests.table_cases import CASES, as_arrays

pytestmark = pytest.mark.gpu


def _shape(case):
    tc, tk = case.totals()
    return lsa.ProblemShape(batch=case.B, chunk_size=case.C, index_dim=64, num_q_heads=8,
                            head_dim_qk=64, head_dim_v=64, v_aliases_k=False,
                            dtype=torch.bfloat16, softmax_scale=0.125,
                            max_chunks=case.max_chunks, max_k=case.max_k, total_chunks=tc,
                            total_k=tk, uniform=case.uniform)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_device_table_checks(case):
    tok, chunk, sel_off, sel_idx = (torch.from_numpy(a).cuda() for a in as_arrays(case))
    bits = lsa.check_tables(_shape(case), chunk, sel_off, tok, sel_idx,
                            kept_ascending=case.ascending)
    assert bits == case.expect, (case.name, bits)
    # without the optional tables only the offset and keep-count bits remain
    bits = lsa.check_tables(_shape(case), chunk, sel_off)
    assert bits == case.expect & ~(lsa.TABLE_ERR_TOK_OFF | lsa.TABLE_ERR_SEL_IDX), case.name


def test_selection_and_workload_tables_pass(monkeypatch):
    w = wl.make_workload(wl.small_variant("cfg5"))
    d = dev.upload(w, "cuda")
    d.step(0, reindex=True)
    torch.cuda.synchronize()
    assert lsa.check_tables(d.shape, d.chunk_off, d.sel_off, d.tok_off, d.sel_idx) == 0
    # debug mode: a kept index one past stream 0's chunks is caught before the
    # step is enqueued (that index would only select masked tokens anyway)
    monkeypatch.setattr(lsa, "_DEBUG_CHECKS", True)
    d.step(1, reindex=False)  # the valid set passes
    bad = dev.to_host(d.sel_idx).copy()
    bad[int(w.sel_off[1]) - 1] = int(w.chunk_off[1] - w.chunk_off[0])
    d.sel_idx.copy_(torch.from_numpy(bad).cuda())
    with pytest.raises(ValueError, match="preconditions"):
        d.step(2, reindex=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.to_host(d.sel_idx), bad)
