"""Python front end of the CPU oracle for the LSA decode hot path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the product package never does.  It loads
``liblsa_oracle.so`` (built from ``lsa_oracle.c`` with gcc, no HIP headers)
and shares nothing with the HIP library.

Step definitions (cited to the pages' sections, see ``lsa_oracle.c``):
  score      dual-encoder inner product per chunk (wiki note flowchart and
             "Key points"; review section 3-2-4; arXiv abstract v2)
  select     top-k keep set per stream (review section 3-2-3 step 5)
  gather     resident pool of kept chunks (wiki note flowchart; molayo
             explainer, gathering only the selected chunks)
  attention  softmax attention over the kept chunks' tokens (review section
             3-2-3 steps 6-7)
  score_fp8mh  multi-head relevance of float8 compressed-key chunk records
             (review sections 3-2-1, 3-2-2 and 4-3)
  score_fp8mh_layers  the same over several layers, combined by max or
             mean (review section 3-2-2, the layer ensemble)
  select_threshold  threshold keep mask capped by a top-k, with a dense
             fallback where no chunk passes (review section 3-2-3 step 5,
             sections 4-3 and 5-1)
  pool_delta the pool's slot table after a re-index when only newly kept
             chunks are copied in from host memory (wiki note flowchart)
  keep_recent the attention keep set of a context grown since the last
             re-index: kept chunks, the last scored chunk, unscored chunks
  decode     the review's decode loop (section 3-2-3 steps 3-7): re-score and
             re-select every ``reindex_every`` steps, attend every step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblsa_oracle.so")
# another build of the same source (the sanitizer run of
# learned_kv_chunk_amd/sanitize.py) may be named here; it is loaded as is
_LIB_OVERRIDE = os.environ.get("LSA_ORACLE_LIBRARY")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile liblsa_oracle.so with the host C compiler (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE:
            build()
        lib = ctypes.CDLL(_LIB_OVERRIDE or _LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_keep_count.argtypes = [i32, i32, i32, i32]
        lib.oracle_keep_count.restype = i32
        lib.oracle_score.argtypes = [i32, i32, i32, P, P, P, P]
        lib.oracle_score.restype = None
        lib.oracle_select.argtypes = [i32, P, P, P, P]
        lib.oracle_select.restype = i32
        lib.oracle_gather.argtypes = [i32, i32, i64, P, P, P, P, P]
        lib.oracle_gather.restype = None
        lib.oracle_attention.argtypes = [i32, i32, i32, i32, i32, i32, i32, f64,
                                         P, P, P, P, P, P, P, P, i32]
        lib.oracle_attention.restype = None
        lib.oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_e4m3.restype = f64
        lib.oracle_score_fp8mh.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
        lib.oracle_score_fp8mh.restype = None
        lib.oracle_score_fp8mh_layers.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P]
        lib.oracle_score_fp8mh_layers.restype = None
        lib.oracle_select_threshold.argtypes = [i32, P, P, f64, i32, P, P, P]
        lib.oracle_select_threshold.restype = None
        lib.oracle_pool_delta.argtypes = [i32, P, P, P, P, P, P, P]
        lib.oracle_pool_delta.restype = None
        lib.oracle_keep_recent.argtypes = [i32, i32, P, P, P, P, i32, P, P]
        lib.oracle_keep_recent.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _elements(a: np.ndarray) -> tuple[np.ndarray, int]:
    """Return (contiguous array, dtype code): float32 or bfloat16 bit patterns (uint16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bit patterns (uint16), got {a.dtype}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def keep_count(n_chunks: int, num: int, den: int, round_up: bool) -> int:
    return int(_load().oracle_keep_count(n_chunks, num, den, int(round_up)))


def score(q: np.ndarray, emb: np.ndarray, chunk_off: np.ndarray) -> np.ndarray:
    """fp64 scores [sum N_b] of each chunk embedding against its stream's query."""
    q, dt = _elements(q)
    emb, dt2 = _elements(emb)
    assert dt == dt2, "q and emb must share an element type"
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    B, D = q.shape
    assert emb.shape[1] == D and emb.shape[0] == chunk_off[-1]
    out = np.empty(int(chunk_off[-1]), dtype=np.float64)
    _load().oracle_score(B, D, dt, _ptr(q), _ptr(emb), _ptr(chunk_off), _ptr(out))
    return out


def fp8_e4m3(code: int) -> float:
    """Exact value of one float8 e4m3 code."""
    return float(_load().oracle_fp8_e4m3(int(code) & 0xFF))


def score_fp8mh(q_heads: np.ndarray, head_w: np.ndarray, rec: np.ndarray,
                chunk_off: np.ndarray) -> np.ndarray:
    """fp64 multi-head scores [sum N_b] of compressed-key chunk records.
    q_heads: [B][Hs][D] float32 or bf16 patterns; head_w: [B][Hs] float32;
    rec: [sum N_b][D + 4] uint8 (D float8 e4m3 values, then a float32 scale)."""
    q, dt = _elements(q_heads)
    w = np.ascontiguousarray(head_w, dtype=np.float32)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    B, Hs, D = q.shape
    assert w.shape == (B, Hs) and rec.shape == (int(chunk_off[-1]), D + 4)
    out = np.empty(int(chunk_off[-1]), dtype=np.float64)
    _load().oracle_score_fp8mh(B, Hs, D, dt, _ptr(q), _ptr(w), _ptr(rec), _ptr(chunk_off),
                               _ptr(out))
    return out


COMBINE_MAX = 0
COMBINE_MEAN = 1


def score_fp8mh_layers(q_heads: np.ndarray, head_w: np.ndarray, rec: np.ndarray,
                       chunk_off: np.ndarray, combine: int) -> np.ndarray:
    """fp64 ensemble scores [sum N_b] over L layers: q_heads [L][B][Hs][D],
    head_w [L][B][Hs], rec [L][sum N_b][D + 4]; combine COMBINE_MAX or
    COMBINE_MEAN."""
    q, dt = _elements(q_heads)
    w = np.ascontiguousarray(head_w, dtype=np.float32)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    L, B, Hs, D = q.shape
    assert w.shape == (L, B, Hs) and rec.shape == (L, int(chunk_off[-1]), D + 4)
    assert combine in (COMBINE_MAX, COMBINE_MEAN)
    out = np.empty(int(chunk_off[-1]), dtype=np.float64)
    _load().oracle_score_fp8mh_layers(L, combine, B, Hs, D, dt, _ptr(q), _ptr(w), _ptr(rec),
                                      _ptr(chunk_off), _ptr(out))
    return out


def select_threshold(scores: np.ndarray, chunk_off: np.ndarray, tau: float,
                     max_keep: int = 0) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Threshold keep mask: (sel_off [B+1], ascending kept indices, fallback
    flags [B]); see oracle_select_threshold."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    B = len(chunk_off) - 1
    sel_off = np.empty(B + 1, dtype=np.int32)
    sel_idx = np.empty(max(1, int(chunk_off[-1])), dtype=np.int32)
    fb = np.empty(B, dtype=np.int32)
    _load().oracle_select_threshold(B, _ptr(s), _ptr(chunk_off), float(tau), int(max_keep),
                                    _ptr(sel_off), _ptr(sel_idx), _ptr(fb))
    return sel_off, sel_idx[:int(sel_off[-1])].copy(), fb


def select(scores: np.ndarray, chunk_off: np.ndarray, sel_off: np.ndarray) -> np.ndarray:
    """Ascending kept chunk indices per stream (CSR by sel_off)."""
    s = np.ascontiguousarray(scores, dtype=np.float64)  # float32 -> float64 is exact
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    sel_off = np.ascontiguousarray(sel_off, dtype=np.int32)
    B = len(chunk_off) - 1
    out = np.empty(int(sel_off[-1]), dtype=np.int32)
    rc = _load().oracle_select(B, _ptr(s), _ptr(chunk_off), _ptr(sel_off), _ptr(out))
    if rc != 0:
        raise ValueError("keep count outside [0, N_b]")
    return out


def gather(store: np.ndarray, C: int, tok_off: np.ndarray, sel_idx: np.ndarray,
           sel_off: np.ndarray) -> np.ndarray:
    """Pool [sum k_b, C, row] holding the kept chunks; rows past L_b are zero."""
    store = np.ascontiguousarray(store)
    tok_off = np.ascontiguousarray(tok_off, dtype=np.int64)
    sel_idx = np.ascontiguousarray(sel_idx, dtype=np.int32)
    sel_off = np.ascontiguousarray(sel_off, dtype=np.int32)
    B = len(tok_off) - 1
    row_shape = store.shape[1:]
    row_bytes = store.itemsize * int(np.prod(row_shape))
    pool = np.empty((int(sel_off[-1]), C) + tuple(row_shape), dtype=store.dtype)
    _load().oracle_gather(B, C, row_bytes, _ptr(store), _ptr(tok_off), _ptr(sel_idx),
                          _ptr(sel_off), _ptr(pool))
    return pool


def pool_delta(chunk_off: np.ndarray, sel_idx: np.ndarray, sel_off: np.ndarray,
               table: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(new slot table [sum k_b], loaded slots [sum k_b] of which the first
    load_count[b] after sel_off[b] are meaningful, load_count [B])."""
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    sel_idx = np.ascontiguousarray(sel_idx, dtype=np.int32)
    sel_off = np.ascontiguousarray(sel_off, dtype=np.int32)
    table = np.ascontiguousarray(table, dtype=np.int32)
    B = len(chunk_off) - 1
    assert len(table) == len(sel_idx) == int(sel_off[-1])
    out = np.empty_like(table)
    loads = np.full(max(1, len(table)), -1, dtype=np.int32)
    count = np.empty(B, dtype=np.int32)
    _load().oracle_pool_delta(B, _ptr(chunk_off), _ptr(sel_idx), _ptr(sel_off), _ptr(table),
                              _ptr(out), _ptr(loads), _ptr(count))
    return out, loads[:len(table)], count


def keep_recent(C: int, seq_len: np.ndarray, chunk_off: np.ndarray, sel_idx: np.ndarray,
                sel_off: np.ndarray, max_recent: int) -> tuple[np.ndarray, np.ndarray]:
    """(out_off [B+1], ascending attention keep set) of a grown context."""
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int64)
    chunk_off = np.ascontiguousarray(chunk_off, dtype=np.int32)
    sel_idx = np.ascontiguousarray(sel_idx, dtype=np.int32)
    sel_off = np.ascontiguousarray(sel_off, dtype=np.int32)
    B = len(seq_len)
    out = np.empty(int(sel_off[-1]) + B * max(0, max_recent) + 1, dtype=np.int32)
    off = np.empty(B + 1, dtype=np.int32)
    _load().oracle_keep_recent(B, C, _ptr(seq_len), _ptr(chunk_off), _ptr(sel_idx),
                               _ptr(sel_off), int(max_recent), _ptr(out), _ptr(off))
    return off, out[:int(off[-1])].copy()


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray | None, tok_off: np.ndarray,
              sel_idx: np.ndarray, sel_off: np.ndarray, C: int, scale: float,
              dv: int | None = None, nthreads: int = 1) -> tuple[np.ndarray, np.ndarray]:
    """Sparse attention (out [B,H,dv] fp64, lse [B,H] fp64).

    V=None means the value rows alias the first dv columns of the key rows.
    """
    Q, dt = _elements(Q)
    K, dtk = _elements(K)
    assert dt == dtk
    B, H, dqk = Q.shape
    assert K.shape[1] == dqk
    if V is None:
        alias = 1
        assert dv is not None and dv <= dqk
        Vp = K
    else:
        alias = 0
        V, dtv = _elements(V)
        assert dtv == dt and V.shape[0] == K.shape[0]
        dv = V.shape[1]
        Vp = V
    tok_off = np.ascontiguousarray(tok_off, dtype=np.int64)
    sel_idx = np.ascontiguousarray(sel_idx, dtype=np.int32)
    sel_off = np.ascontiguousarray(sel_off, dtype=np.int32)
    assert len(tok_off) == B + 1 and len(sel_off) == B + 1
    out = np.empty((B, H, dv), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    _load().oracle_attention(B, H, dqk, dv, alias, dt, C, float(scale), _ptr(Q), _ptr(K),
                             _ptr(Vp), _ptr(tok_off), _ptr(sel_idx), _ptr(sel_off),
                             _ptr(out), _ptr(lse), int(nthreads))
    return out, lse


def all_chunks(tok_off: np.ndarray, C: int) -> tuple[np.ndarray, np.ndarray]:
    """(sel_idx, sel_off) that keeps every chunk: the dense-attention case."""
    lens = np.diff(np.asarray(tok_off, dtype=np.int64))
    n = (lens + C - 1) // C
    sel_off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    sel_idx = np.concatenate([np.arange(x, dtype=np.int32) for x in n]) if len(n) else \
        np.zeros(0, np.int32)
    return sel_idx.astype(np.int32), sel_off


def decode(q_idx, emb: np.ndarray, chunk_off: np.ndarray, sel_off: np.ndarray,
           Qs: list, K: np.ndarray, V: np.ndarray | None, tok_off: np.ndarray, C: int,
           scale: float, reindex_every: int, dv: int | None = None, nthreads: int = 1):
    """The review's decode loop (section 3-2-3 steps 4-7, with the re-scoring
    interval of the section 3-1 table and section 4-3): at step t the indexer
    scores the chunks and a new kept set is selected only when t is a multiple
    of ``reindex_every``; every step attends over the kept set of the most
    recent re-index with that step's decode queries Qs[t].

    ``q_idx`` is the indexer query embedding of every step: one [B, D] array
    used at every re-index, or a sequence with one [B, D] array per step (the
    query a real indexer computes from the current hidden state; only the
    entries of re-index steps are read).  Returns a list of (sel_idx, out,
    lse) per step."""
    R = int(reindex_every)
    if R < 1:
        raise ValueError("reindex_every must be >= 1")
    per_step = not (isinstance(q_idx, np.ndarray) and q_idx.ndim == 2)
    if per_step and len(q_idx) < len(Qs):
        raise ValueError("one indexer query per step is needed")
    results = []
    sel_idx = None
    for t, Q in enumerate(Qs):
        if t % R == 0:
            s = score(q_idx[t] if per_step else q_idx, emb, chunk_off)
            sel_idx = select(s, chunk_off, sel_off)
        out, lse = attention(Q, K, V, tok_off, sel_idx, sel_off, C, scale, dv=dv,
                             nthreads=nthreads)
        results.append((sel_idx, out, lse))
    return results
