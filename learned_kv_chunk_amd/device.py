"""Device-resident copy of a synthetic workload plus the buffers one decode
step writes (scores, kept indices, pools, outputs, workspace).  Data movement
only: every computation goes through :mod:`learned_kv_chunk_amd.lsa`."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import lsa
from .workloads import Workload


def _to_device(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 tensors come back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def problem_shape(w: Workload, attn_tiles_per_block: int = 0) -> lsa.ProblemShape:
    c = w.cfg
    n_chunks = np.diff(w.chunk_off)
    return lsa.ProblemShape(
        batch=c.batch, chunk_size=c.chunk_size, index_dim=c.index_dim,
        num_q_heads=c.num_q_heads, head_dim_qk=c.head_dim_qk, head_dim_v=c.head_dim_v,
        v_aliases_k=c.v_aliases_k, dtype=torch.bfloat16 if c.dtype == "bf16" else torch.float32,
        softmax_scale=c.softmax_scale, max_chunks=int(n_chunks.max()), max_k=int(w.keep.max()),
        total_chunks=int(w.chunk_off[-1]), total_k=int(w.sel_off[-1]),
        attn_tiles_per_block=attn_tiles_per_block,
        uniform=bool((n_chunks == n_chunks[0]).all() and (w.keep == w.keep[0]).all()))


@dataclasses.dataclass
class DeviceWorkload:
    w: Workload
    shape: lsa.ProblemShape
    q_idx: torch.Tensor
    emb: torch.Tensor
    chunk_off: torch.Tensor
    sel_off: torch.Tensor
    tok_off: torch.Tensor
    K: torch.Tensor
    V: Optional[torch.Tensor]
    scores: torch.Tensor
    sel_idx: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    workspace: torch.Tensor
    k_pool: Optional[torch.Tensor] = None
    v_pool: Optional[torch.Tensor] = None
    _q: dict = dataclasses.field(default_factory=dict)
    _prepared: dict = dataclasses.field(default_factory=dict)

    def queries(self, step: int) -> torch.Tensor:
        if step not in self._q:
            self._q[step] = _to_device(self.w.queries(step), self.K.device)
        return self._q[step]

    def prepared(self, materialize_pool: bool, reindex_every: int) -> lsa.PreparedStep:
        """The step's arguments marshalled once (cached per pool mode and
        re-index interval)."""
        key = (bool(materialize_pool), int(reindex_every))
        p = self._prepared.get(key)
        if p is None:
            p = lsa.PreparedStep(self.shape, q_idx=self.q_idx, emb=self.emb,
                                 chunk_off=self.chunk_off, scores=self.scores,
                                 sel_off=self.sel_off, sel_idx=self.sel_idx, q=self.queries(0),
                                 k_store=self.K, v_store=self.V, tok_off=self.tok_off,
                                 out=self.out, lse=self.lse, workspace=self.workspace,
                                 materialize_pool=materialize_pool, k_pool=self.k_pool,
                                 v_pool=self.v_pool, reindex_every=reindex_every)
            self._prepared[key] = p
        return p

    def step(self, t: int, reindex: bool = False, materialize_pool: bool = False,
             ev_begin=None, ev_end=None, q: Optional[torch.Tensor] = None,
             reindex_every: int = 0) -> None:
        """Decode step t.  reindex_every > 0: the library's schedule decides
        whether step t re-indexes (``reindex`` is ignored), through the
        prepared arguments."""
        if reindex_every > 0:
            self.prepared(materialize_pool, reindex_every).run(
                t, q=self.queries(t) if q is None else q, ev_attn_begin=ev_begin,
                ev_attn_end=ev_end)
            return
        lsa.decode_step(self.shape, q_idx=self.q_idx, emb=self.emb, chunk_off=self.chunk_off,
                        scores=self.scores, sel_off=self.sel_off, sel_idx=self.sel_idx,
                        q=self.queries(t) if q is None else q, k_store=self.K, v_store=self.V,
                        tok_off=self.tok_off, out=self.out, lse=self.lse,
                        workspace=self.workspace, reindex=reindex,
                        materialize_pool=materialize_pool, k_pool=self.k_pool,
                        v_pool=self.v_pool, ev_attn_begin=ev_begin, ev_attn_end=ev_end,
                        step=t, reindex_every=reindex_every)


def upload(w: Workload, device="cuda", attn_tiles_per_block: int = 0,
           with_pool: Optional[bool] = None) -> DeviceWorkload:
    shape = problem_shape(w, attn_tiles_per_block)
    c = w.cfg
    if with_pool is None:
        with_pool = c.materialize_pool
    d = DeviceWorkload(
        w=w, shape=shape, q_idx=_to_device(w.q_idx, device), emb=_to_device(w.emb, device),
        chunk_off=_to_device(w.chunk_off, device), sel_off=_to_device(w.sel_off, device),
        tok_off=_to_device(w.tok_off, device), K=_to_device(w.K, device),
        V=_to_device(w.V, device),
        scores=torch.empty(shape.total_chunks, dtype=torch.float32, device=device),
        sel_idx=torch.empty(shape.total_k, dtype=torch.int32, device=device),
        out=torch.empty((c.batch, c.num_q_heads, c.head_dim_v), dtype=torch.float32,
                        device=device),
        lse=torch.empty((c.batch, c.num_q_heads), dtype=torch.float32, device=device),
        workspace=lsa.allocate_workspace(shape, device))
    if with_pool:
        dt = shape.dtype
        d.k_pool = torch.empty((shape.total_k, c.chunk_size, c.head_dim_qk), dtype=dt,
                               device=device)
        if not c.v_aliases_k:
            d.v_pool = torch.empty((shape.total_k, c.chunk_size, c.head_dim_v), dtype=dt,
                                   device=device)
    return d
