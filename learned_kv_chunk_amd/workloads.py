"""Seeded synthetic inputs for the LSA decode hot path.

This module only draws and lays out input data (random values, lengths,
planted needles, CSR offsets, bf16 rounding of inputs).  It computes none of
the method's arithmetic -- no scores, selections or attention -- and is the
one module shared by the HIP path's tests/benchmark and by the CPU oracle.

Recipe (every draw comes from its own PCG64 stream keyed by
``SeedSequence(seed, spawn_key=(config, purpose, stream, block))``, so a value
does not depend on the block size used to draw its neighbours or on threads):

* stream lengths: fixed per configuration, or uniform integers in
  [lo, hi] inclusive (the ragged batch);
* chunking: chunk n of a stream covers tokens [n*C, min((n+1)*C, L)), so
  N = ceil(L / C) and the last chunk may be partial;
* indexer query q* and chunk embeddings: standard Gaussian, L2-normalised
  (a dual-encoder cosine space);
* needles: ``n_needles`` distinct chunk indices per stream drawn uniformly;
  their embedding is 0.9*q* + sqrt(1-0.81)*u with u a unit vector orthogonal
  to q* (Gram-Schmidt on a Gaussian draw), so cosine(q*, needle) = 0.9;
* K, V and the per-step decode queries Q_t: Gaussian with the configured
  standard deviation (1/sqrt(d));
* bf16 configurations: values are drawn in fp32 and rounded to bf16 with
  round-to-nearest-even; both the oracle and the GPU read those bit patterns.

Inputs of the multi-head compressed-key scorer (``make_mh_inputs``): per
stream, Hs head queries of dimension D (Gaussian, std 1/sqrt(D), bf16) and Hs
non-negative head weights (|Gaussian| / Hs, fp32); per chunk a record of D
float8 e4m3 key values and a float32 scale: the key is Gaussian (std 1),
the scale is max|key| / 448 and the values are key / scale rounded to the
nearest e4m3 value (ties to the even code).  Needle chunks (the same positions
as the embedding needles) get the key 3 sqrt(D) u, with u the unit vector of
the weighted head-query sum sum_h w_h q_h.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

DTYPES = ("f32", "bf16")

# purpose tags of the random streams
(_P_LENGTHS, _P_QIDX, _P_EMB, _P_NEEDLE_POS, _P_NEEDLE_DIR, _P_K, _P_V, _P_Q,
 _P_MH_Q, _P_MH_W, _P_MH_KEY, _P_DRIFT) = range(12)

_ROWS_PER_BLOCK = 1 << 14


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: shapes, dtypes and schedule of a batch of decode streams."""
    name: str
    batch: int
    chunk_size: int
    index_dim: int
    num_q_heads: int
    head_dim_qk: int
    head_dim_v: int
    v_aliases_k: bool
    dtype: str
    keep_num: int            # keep ratio numerator
    keep_den: int            # keep ratio denominator
    keep_round_up: bool      # ceil (True) or floor (False) of N*num/den
    length: int = 0          # fixed context length, or 0 for a uniform draw
    length_lo: int = 0
    length_hi: int = 0
    lengths: Optional[tuple] = None   # explicit per-stream lengths (overrides the above)
    n_needles: int = 0
    kv_std: float = 1.0
    q_std: float = 1.0
    steps: int = 1
    reindex_every: int = 1
    materialize_pool: bool = False
    config_id: int = 0
    seed: int = 0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads of the benchmark table.
CONFIGS = {
    "cfg1": Config(name="cfg1", config_id=1, batch=1, length=4096, chunk_size=64, index_dim=64,
                   keep_num=1, keep_den=8, keep_round_up=False, n_needles=4,
                   num_q_heads=8, head_dim_qk=64, head_dim_v=64, v_aliases_k=False,
                   dtype="f32", kv_std=1 / 8, q_std=1 / 8, steps=16, reindex_every=1),
    "cfg2": Config(name="cfg2", config_id=2, batch=16, length=131072, chunk_size=64,
                   index_dim=128, keep_num=135, keep_den=1000, keep_round_up=False,
                   n_needles=8, num_q_heads=16, head_dim_qk=128, head_dim_v=128,
                   v_aliases_k=False, dtype="bf16", kv_std=1 / math.sqrt(128),
                   q_std=1 / math.sqrt(128), steps=200, reindex_every=1),
    "cfg3": Config(name="cfg3", config_id=3, batch=4, length=524288, chunk_size=64,
                   index_dim=128, keep_num=10, keep_den=100, keep_round_up=False,
                   n_needles=16, num_q_heads=32, head_dim_qk=128, head_dim_v=128,
                   v_aliases_k=False, dtype="bf16", kv_std=1 / math.sqrt(128),
                   q_std=1 / math.sqrt(128), steps=256, reindex_every=64,
                   materialize_pool=True),
    "cfg4": Config(name="cfg4", config_id=4, batch=1, length=1048576, chunk_size=128,
                   index_dim=256, keep_num=8, keep_den=100, keep_round_up=False,
                   n_needles=0, num_q_heads=64, head_dim_qk=576, head_dim_v=512,
                   v_aliases_k=True, dtype="bf16", kv_std=1 / 24, q_std=1 / 24,
                   steps=16, reindex_every=1),
    "cfg5": Config(name="cfg5", config_id=5, batch=32, length=0, length_lo=8192,
                   length_hi=262144, chunk_size=64, index_dim=128, keep_num=135,
                   keep_den=1000, keep_round_up=True, n_needles=8, num_q_heads=16,
                   head_dim_qk=128, head_dim_v=128, v_aliases_k=False, dtype="bf16",
                   kv_std=1 / math.sqrt(128), q_std=1 / math.sqrt(128), steps=16,
                   reindex_every=1),
}


def _rng(cfg: Config, purpose: int, stream: int, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=(cfg.config_id, purpose, stream, block))
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """The float32 values an input array holds (bf16 patterns are widened exactly)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@dataclasses.dataclass
class Workload:
    """Host arrays of one workload (bf16 tensors are uint16 bit patterns)."""
    cfg: Config
    lengths: np.ndarray      # [B] int64
    tok_off: np.ndarray      # [B+1] int64
    chunk_off: np.ndarray    # [B+1] int32
    keep: np.ndarray         # [B] int32, k_b
    sel_off: np.ndarray      # [B+1] int32
    q_idx: np.ndarray        # [B, D]
    emb: np.ndarray          # [sum N, D]
    needles: list            # per stream: sorted needle chunk indices
    K: np.ndarray            # [sum L, dqk]
    V: Optional[np.ndarray]  # [sum L, dv], or None when V aliases K
    _q_cache: dict = dataclasses.field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.cfg.batch

    def queries(self, step: int) -> np.ndarray:
        """Decode queries Q_t [B, H, dqk] of step t."""
        if step not in self._q_cache:
            c = self.cfg
            qs = [_rng(c, _P_Q, b, step).standard_normal((c.num_q_heads, c.head_dim_qk),
                                                           dtype=np.float32) * np.float32(c.q_std)
                  for b in range(c.batch)]
            self._q_cache[step] = _encode(np.stack(qs), c.dtype)
        return self._q_cache[step]

    def resident_fraction(self) -> float:
        return float((self.keep.astype(np.int64) * self.cfg.chunk_size).sum()
                     / self.lengths.sum())


def stream_lengths(cfg: Config) -> np.ndarray:
    if cfg.lengths is not None:
        return np.asarray(cfg.lengths, dtype=np.int64)
    if cfg.length > 0:
        return np.full(cfg.batch, cfg.length, dtype=np.int64)
    g = _rng(cfg, _P_LENGTHS, 0)
    return g.integers(cfg.length_lo, cfg.length_hi, size=cfg.batch, endpoint=True).astype(np.int64)


def keep_counts(cfg: Config, n_chunks: np.ndarray) -> np.ndarray:
    """k_b from the configured keep ratio, in integer arithmetic, within [1, N_b]."""
    p = n_chunks.astype(np.int64) * cfg.keep_num
    k = (p + cfg.keep_den - 1) // cfg.keep_den if cfg.keep_round_up else p // cfg.keep_den
    return np.clip(k, 1, n_chunks).astype(np.int32)


def _fill_gaussian(cfg: Config, purpose: int, lengths: np.ndarray, tok_off: np.ndarray,
                   width: int, std: float) -> np.ndarray:
    total = int(tok_off[-1])
    itemsize = 2 if cfg.dtype == "bf16" else 4
    out = np.empty((total, width), dtype=np.uint16 if itemsize == 2 else np.float32)
    jobs = []
    for b in range(cfg.batch):
        for blk, r0 in enumerate(range(0, int(lengths[b]), _ROWS_PER_BLOCK)):
            r1 = min(int(lengths[b]), r0 + _ROWS_PER_BLOCK)
            jobs.append((b, blk, int(tok_off[b]) + r0, r1 - r0))

    def work(job):
        b, blk, row0, nrows = job
        x = _rng(cfg, purpose, b, blk).standard_normal((nrows, width), dtype=np.float32)
        x *= np.float32(std)
        out[row0:row0 + nrows] = _encode(x, cfg.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))
    return out


def make_workload(cfg: Config) -> Workload:
    C, D = cfg.chunk_size, cfg.index_dim
    lengths = stream_lengths(cfg)
    if (lengths < 1).any():
        raise ValueError("every stream needs at least one token")
    n_chunks = (lengths + C - 1) // C
    tok_off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    chunk_off = np.concatenate([[0], np.cumsum(n_chunks)]).astype(np.int32)
    keep = keep_counts(cfg, n_chunks)
    sel_off = np.concatenate([[0], np.cumsum(keep)]).astype(np.int32)

    q_rows, e_rows, needles = [], [], []
    for b in range(cfg.batch):
        q = _unit_rows(_rng(cfg, _P_QIDX, b).standard_normal(D))
        e = _unit_rows(_rng(cfg, _P_EMB, b).standard_normal((int(n_chunks[b]), D)))
        nn = min(cfg.n_needles, int(n_chunks[b]))
        pos = np.sort(_rng(cfg, _P_NEEDLE_POS, b).choice(int(n_chunks[b]), size=nn,
                                                          replace=False)) if nn else \
            np.zeros(0, np.int64)
        if nn:
            g = _rng(cfg, _P_NEEDLE_DIR, b).standard_normal((nn, D))
            u = _unit_rows(g - np.outer(g @ q, q))
            e[pos] = 0.9 * q + math.sqrt(1.0 - 0.81) * u
        q_rows.append(q)
        e_rows.append(e)
        needles.append(pos.astype(np.int32))
    q_idx = _encode(np.stack(q_rows).astype(np.float32), cfg.dtype)
    emb = _encode(np.concatenate(e_rows).astype(np.float32), cfg.dtype)

    K = _fill_gaussian(cfg, _P_K, lengths, tok_off, cfg.head_dim_qk, cfg.kv_std)
    V = None if cfg.v_aliases_k else _fill_gaussian(cfg, _P_V, lengths, tok_off,
                                                    cfg.head_dim_v, cfg.kv_std)
    return Workload(cfg=cfg, lengths=lengths, tok_off=tok_off, chunk_off=chunk_off, keep=keep,
                    sel_off=sel_off, q_idx=q_idx, emb=emb, needles=needles, K=K, V=V)


def drift_query(w: Workload, epoch: int, eps: float = 0.5) -> np.ndarray:
    """Indexer queries of re-index epoch `epoch` under drift: per stream
    normalize(q + eps * g) with q the workload's query (as drawn, before
    rounding) and g a unit Gaussian direction of its own per (stream, epoch);
    epoch 0 returns the workload's own queries.  Encoded like q_idx."""
    if epoch == 0:
        return w.q_idx.copy()
    cfg = w.cfg
    rows = []
    for b in range(cfg.batch):
        q = _unit_rows(_rng(cfg, _P_QIDX, b).standard_normal(cfg.index_dim))
        g = _unit_rows(_rng(cfg, _P_DRIFT, b, epoch).standard_normal(cfg.index_dim))
        rows.append(_unit_rows(q + eps * g))
    return _encode(np.stack(rows).astype(np.float32), cfg.dtype)


def small_variant(name: str, **overrides) -> Config:
    """A reduced-length copy of a named workload (same structure, dtypes, head
    shapes and keep ratio) sized for the oracle to finish in seconds.  Default
    lengths are a ragged mix with partial last chunks and enough chunks that
    every stream keeps at least max(8, n_needles) of them."""
    base = CONFIGS[name]
    C = base.chunk_size
    need = max(8, base.n_needles)
    n0 = -(-need * base.keep_den // base.keep_num) + 2
    mix = [(n0, 5), (n0 + 13, C // 2), (n0 + 5, 1), (n0 + 7, 0)]
    count = max(1, min(base.batch, 4))
    default_lengths = tuple(n * C + extra if extra else n * C for n, extra in mix[:count])
    kw = dict(lengths=default_lengths, batch=len(default_lengths), steps=2,
              name=base.name + "_small", config_id=100 + base.config_id)
    kw.update(overrides)
    if "lengths" in overrides and "batch" not in overrides:
        kw["batch"] = len(overrides["lengths"])
    return base.replace(**kw)


# ----------------------------------------------------------------------------- float8 inputs
def _e4m3_nonneg_values() -> np.ndarray:
    """Values of the non-negative finite float8 e4m3 codes 0x00..0x7e, in code
    order (which is increasing value order)."""
    codes = np.arange(0x7F)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e.astype(np.float64) - 10))


_E4M3 = _e4m3_nonneg_values()


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round values with |x| <= 448 to the nearest float8 e4m3 code (ties to
    the even code); returns uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if (a > 448.0).any() or np.isnan(a).any():
        raise ValueError("float8 e4m3 encoding needs finite |x| <= 448")
    hi = np.clip(np.searchsorted(_E4M3, a), 1, len(_E4M3) - 1)
    lo = hi - 1
    dlo = a - _E4M3[lo]
    dhi = _E4M3[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)  # sign kept, also on -0


def make_mh_inputs(w: Workload, heads: int = 128, head_dim: int = 128, layer: int = 0):
    """Head queries [B][heads][head_dim] (bf16 bit patterns), head weights
    [B][heads] (fp32) and compressed-key records [sum N][head_dim + 4] (uint8)
    for the multi-head scorer, aligned with the workload's chunks.  `layer`
    selects independent draws for one layer of an ensemble; the needles sit
    at the same chunks in every layer."""
    cfg = w.cfg
    B = cfg.batch
    n_total = int(w.chunk_off[-1])
    q = np.stack([_rng(cfg, _P_MH_Q, b, layer).standard_normal((heads, head_dim),
                                                                 dtype=np.float32)
                  / np.float32(math.sqrt(head_dim)) for b in range(B)])
    wt = np.stack([np.abs(_rng(cfg, _P_MH_W, b, layer).standard_normal(heads, dtype=np.float32))
                   / np.float32(heads) for b in range(B)])
    q_bits = to_bf16_bits(q)
    rec = np.empty((n_total, head_dim + 4), dtype=np.uint8)
    for b in range(B):
        r0, r1 = int(w.chunk_off[b]), int(w.chunk_off[b + 1])
        keys = _rng(cfg, _P_MH_KEY, b, layer).standard_normal((r1 - r0, head_dim))
        pos = w.needles[b]
        if len(pos):
            dvec = (wt[b][:, None].astype(np.float64) * bf16_bits_to_f32(q_bits[b])).sum(0)
            keys[pos] = 3.0 * math.sqrt(head_dim) * dvec / np.linalg.norm(dvec)
        scale = (np.abs(keys).max(axis=1) / 448.0).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0))
        # |key / scale| <= 448 up to the rounding of the scale to fp32
        vals = np.clip(keys / scale.astype(np.float64)[:, None], -448.0, 448.0)
        rec[r0:r1, :head_dim] = to_e4m3_codes(vals)
        rec[r0:r1, head_dim:] = scale.astype("<f4").view(np.uint8).reshape(-1, 4)
    return q_bits, wt.astype(np.float32), rec


def make_mh_layer_inputs(w: Workload, layers: int = 3, heads: int = 128, head_dim: int = 128):
    """make_mh_inputs for `layers` layers, stacked layer-major: queries
    [L][B][heads][head_dim], weights [L][B][heads], records [L][sum N][head_dim + 4]."""
    parts = [make_mh_inputs(w, heads, head_dim, layer=l) for l in range(layers)]
    return tuple(np.ascontiguousarray(np.stack([p[i] for p in parts])) for i in range(3))
