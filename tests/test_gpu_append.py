"""Parity of decode-time context growth with the CPU oracle, through the C
ABI: over a decode loop that appends one K/V row per stream and step
(crossing chunk boundaries, starting from partial last chunks), seq_len
advances, the stores hold exactly the appended rows, the attention keep set
(kept chunks, the last scored chunk, every unscored chunk) equals the
oracle's, and attention over the capacity layout matches the oracle run on
the grown context within tests/parity.py's tolerances."""
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


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("name,max_recent", [("cfg2", 4), ("cfg5", 4), ("cfg4", 4), ("cfg1", 4),
                                             ("cfg2", 2)])
def test_append_decode_loop(name, max_recent):
    # max_recent = 2 binds once a stream has three candidate chunks: the
    # newest two must be attended
    w = wl.make_workload(wl.small_variant(name))
    c = w.cfg
    C = c.chunk_size
    steps = 2 * C + 9
    L0 = w.lengths.astype(np.int64)
    cap = L0 + steps + 3
    base = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
    rows_k = np.zeros((int(base[-1]), c.head_dim_qk), w.K.dtype)
    rows_v = None if w.V is None else np.zeros((int(base[-1]), c.head_dim_v), w.V.dtype)
    for b in range(w.B):
        rows_k[base[b]:base[b] + L0[b]] = w.K[w.tok_off[b]:w.tok_off[b + 1]]
        if rows_v is not None:
            rows_v[base[b]:base[b] + L0[b]] = w.V[w.tok_off[b]:w.tok_off[b + 1]]
    rng = np.random.default_rng(2024)

    def new_rows(d):
        x = (rng.standard_normal((w.B, d)) * c.kv_std).astype(np.float32)
        return wl.to_bf16_bits(x) if c.dtype == "bf16" else x

    d = dev.upload(w, "cuda")
    shape = d.shape
    s_gpu = lsa.score(shape, d.q_idx, d.emb, d.chunk_off)
    sel = lsa.select_topk(shape, s_gpu, d.chunk_off, d.sel_off)
    torch.cuda.synchronize()
    sel_h = dev.to_host(sel)
    n_cap = (cap + C - 1) // C
    attn_shape = dataclasses.replace(
        shape, max_chunks=int(n_cap.max()), total_chunks=int(n_cap.sum()),
        max_k=shape.max_k + max_recent, total_k=shape.total_k + w.B * max_recent,
        uniform=False)
    kd, vd = _t(rows_k), None if rows_v is None else _t(rows_v)
    base_d = torch.from_numpy(base).cuda()
    seq_d = torch.from_numpy(L0.copy()).cuda()
    ws = lsa.allocate_workspace(attn_shape, "cuda")
    worst = {}
    for t in range(steps):
        kn = new_rows(c.head_dim_qk)
        vn = None if rows_v is None else new_rows(c.head_dim_v)
        for b in range(w.B):
            rows_k[base[b] + L0[b] + t] = kn[b]
            if rows_v is not None:
                rows_v[base[b] + L0[b] + t] = vn[b]
        lsa.append_kv(shape, _t(kn), None if vn is None else _t(vn), base_d, seq_d, kd, vd)
        off_d, idx_d = lsa.keep_recent(shape, seq_d, d.chunk_off, sel, d.sel_off, max_recent)
        Q = w.queries(t)
        out, lse = lsa.sparse_decode_attn_varlen(attn_shape, _t(Q), kd, vd, base_d, seq_d, idx_d,
                                                 off_d, workspace=ws)
        torch.cuda.synchronize()
        seq_h = dev.to_host(seq_d)
        np.testing.assert_array_equal(seq_h, L0 + t + 1)
        off_h = dev.to_host(off_d)
        idx_h = dev.to_host(idx_d)[:int(off_h[-1])]
        r_off, r_idx = oracle.keep_recent(C, seq_h, w.chunk_off, sel_h, w.sel_off, max_recent)
        np.testing.assert_array_equal(off_h, r_off)
        np.testing.assert_array_equal(idx_h, r_idx)
        for b in range(w.B):  # the chunk of the token just written is attended
            assert (seq_h[b] - 1) // C in idx_h[off_h[b]:off_h[b + 1]], (t, b)
        if t % 5 == 0 or t == steps - 1:
            # the grown context packed back to back for the oracle
            tok = np.concatenate([[0], np.cumsum(seq_h)]).astype(np.int64)
            Kp = np.concatenate([rows_k[base[b]:base[b] + seq_h[b]] for b in range(w.B)])
            Vp = None if rows_v is None else \
                np.concatenate([rows_v[base[b]:base[b] + seq_h[b]] for b in range(w.B)])
            o_ref, l_ref = oracle.attention(Q, Kp, Vp, tok, idx_h, off_h, C, c.softmax_scale,
                                            dv=c.head_dim_v, nthreads=max(1, oracle.max_threads()))
            worst = P.check_attention(c.dtype, dev.to_host(out), dev.to_host(lse), o_ref, l_ref)
    np.testing.assert_array_equal(dev.to_host(kd), rows_k)
    if rows_v is not None:
        np.testing.assert_array_equal(dev.to_host(vd), rows_v)
    print(name, "steps", steps, "final keep per stream", np.diff(off_h).tolist(), worst)


def test_append_full_stream_is_left_unchanged():
    w = wl.make_workload(wl.small_variant("cfg2", lengths=(64 * 3 + 5, 64 * 2)))
    c = w.cfg
    L0 = w.lengths.astype(np.int64)
    cap = L0 + np.array([1, 0])          # stream 1 is already full
    base = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
    shape = dev.problem_shape(w)
    kd = torch.zeros((int(base[-1]), c.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    seq = torch.from_numpy(L0.copy()).cuda()
    kn = torch.ones((2, c.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        lsa.append_kv(shape, kn, kn, torch.from_numpy(base).cuda(), seq, kd, vd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev.to_host(seq), L0 + np.array([1, 0]))
    k_h = dev.to_host(kd)
    assert (k_h[base[0] + L0[0]] != 0).all() and (k_h[base[1]:] == 0).all()
