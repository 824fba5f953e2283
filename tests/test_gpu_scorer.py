"""Parity of the float8 compressed-key multi-head scorer (through the C ABI)
with the CPU oracle: every score within the tolerance below, the GPU's top-k
of its own scores bit-identical to the oracle's ranking of them, and every
planted needle kept.

Tolerance: |s_gpu - s_ref| <= 1e-4 * max(|s_ref|, A), with A the sum over heads
of |w_h| |c| sum_d |q_hd k_d| (the score's magnitude bound: fp32 accumulation
error is relative to it, and a head whose dot product is near zero may fall on
either side of the ReLU)."""
import numpy as np
import pytest
import torch

from learned_kv_chunk_amd import device as dev
from learned_kv_chunk_amd import lsa
from learned_kv_chunk_amd import workloads as wl
from oracle import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


def _abs_bound(q_bits, hw, rec, chunk_off):
    B, Hs, D = q_bits.shape
    q = np.abs(wl.bf16_bits_to_f32(q_bits).astype(np.float64))
    k = np.abs(torch.from_numpy(np.ascontiguousarray(rec[:, :D])).view(torch.float8_e4m3fn)
               .double().numpy())
    c = np.abs(np.ascontiguousarray(rec[:, D:]).view("<f4").reshape(-1).astype(np.float64))
    out = np.empty(len(rec))
    for b in range(B):
        r0, r1 = chunk_off[b], chunk_off[b + 1]
        out[r0:r1] = c[r0:r1] * ((k[r0:r1] @ q[b].T) @ np.abs(hw[b]).astype(np.float64))
    return out


def _run(w, heads=128, head_dim=128):
    q_bits, hw, rec = wl.make_mh_inputs(w, heads=heads, head_dim=head_dim)
    shape = dev.problem_shape(w)
    qd = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(hw).cuda()
    rd = torch.from_numpy(rec).cuda()
    co = torch.from_numpy(w.chunk_off).cuda()
    so = torch.from_numpy(w.sel_off).cuda()
    s_gpu = lsa.score_fp8_multihead(shape, qd, wd, rd, co)
    sel = lsa.select_topk(shape, s_gpu, co, so)
    torch.cuda.synchronize()
    s_gpu = dev.to_host(s_gpu)
    sel = dev.to_host(sel)
    s_ref = oracle.score_fp8mh(q_bits, hw, rec, w.chunk_off)
    bound = np.maximum(np.abs(s_ref), _abs_bound(q_bits, hw, rec, w.chunk_off))
    err = float((np.abs(s_gpu.astype(np.float64) - s_ref) / bound).max())
    assert err <= 1e-4, f"score error {err:.3e} x bound"
    np.testing.assert_array_equal(sel, oracle.select(s_gpu.astype(np.float64), w.chunk_off,
                                                     w.sel_off))
    P.check_needles(w, sel)
    return err


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_multihead_scorer_small_ragged(name):
    w = wl.make_workload(wl.small_variant(name))
    print(name, _run(w))


@pytest.mark.parametrize("heads,head_dim", [(16, 128), (32, 64), (64, 128)])
def test_multihead_scorer_head_shapes(heads, head_dim):
    w = wl.make_workload(wl.small_variant("cfg2", lengths=(64 * 100 + 3, 64 * 37, 64 * 5 + 9)))
    print(heads, head_dim, _run(w, heads, head_dim))


def test_multihead_scorer_full_size():
    # the 16 x 128K workload: 32768 compressed-key records of 132 bytes
    w = wl.make_workload(wl.CONFIGS["cfg2"])
    print("cfg2 full", _run(w))
