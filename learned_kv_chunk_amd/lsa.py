"""ctypes binding of liblsa.so (include/lsa.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module checks
tensor devices, dtypes, shapes and contiguity, fills the lsa_shape struct and
passes raw device pointers plus torch's current HIP stream.  PyTorch provides
device memory and streams only.  If the library is missing or fails to load,
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LSA_LIBRARY may name another build of the same sources (the host-sanitizer
# build of sanitize.py); there is still no fallback when it is missing
LIB_PATH = os.environ.get("LSA_LIBRARY") or os.path.join(_HERE, "liblsa.so")

LSA_OK = 0
LSA_ERR_INVALID_ARGUMENT = 1
LSA_ERR_UNSUPPORTED = 2
LSA_ERR_WORKSPACE_TOO_SMALL = 3
LSA_ERR_HIP = 4

COMBINE_MAX = 0
COMBINE_MEAN = 1

DTYPE_F32 = 0
DTYPE_BF16 = 1
KV_STORE = 0
KV_POOL = 1
SHAPE_UNIFORM = 1  # lsa_shape.flags: LSA_SHAPE_UNIFORM


class LsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("v_aliases_k", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("max_chunks", ctypes.c_int32),
        ("max_k", ctypes.c_int32),
        ("total_chunks", ctypes.c_int64),
        ("total_k", ctypes.c_int64),
        ("attn_tiles_per_block", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("q_idx_dev", ctypes.c_void_p),
        ("emb_dev", ctypes.c_void_p),
        ("chunk_off_dev", ctypes.c_void_p),
        ("scores_dev", ctypes.c_void_p),
        ("sel_off_dev", ctypes.c_void_p),
        ("sel_idx_dev", ctypes.c_void_p),
        ("q_dev", ctypes.c_void_p),
        ("k_store_dev", ctypes.c_void_p),
        ("v_store_dev", ctypes.c_void_p),
        ("tok_off_dev", ctypes.c_void_p),
        ("k_pool_dev", ctypes.c_void_p),
        ("v_pool_dev", ctypes.c_void_p),
        ("out_dev", ctypes.c_void_p),
        ("lse_dev", ctypes.c_void_p),
        ("reindex", ctypes.c_int32),
        ("materialize_pool", ctypes.c_int32),
        ("ev_attn_begin", ctypes.c_void_p),
        ("ev_attn_end", ctypes.c_void_p),
        ("reindex_every", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("step", ctypes.c_int64),
    ]


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("grid", ctypes.c_int64),
        ("partial_rows", ctypes.c_int64),
        ("kernel", ctypes.c_int32),
        ("tiles_per_chunk", ctypes.c_int32),
        ("merge_in_kernel", ctypes.c_int32),
        ("split_heads", ctypes.c_int32),
        ("select_in_kernel", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


ATTN_KERNEL_NAMES = {0: "attn_mqa", 1: "attn_mla", 2: "attn_portable"}


# Exported symbols of include/lsa.h with their (argtypes, restype).
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGNATURES = {
    "lsa_status_string": ([_I32], ctypes.c_char_p),
    "lsa_abi_version": ([], _I32),
    "lsa_check_tables": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _I32, _P, _P], _I32),
    "lsa_decode_step_static": ([ctypes.POINTER(Shape), ctypes.POINTER(StepArgs), _P], _I32),
    "lsa_reindex_due": ([ctypes.c_int64, _I32], _I32),
    "lsa_keep_count": ([_I32, _I32, _I32, _I32], _I32),
    "lsa_workspace_bytes": ([ctypes.POINTER(Shape)], ctypes.c_size_t),
    "lsa_attention_plan": ([ctypes.POINTER(Shape), ctypes.POINTER(AttnPlanInfo)], _I32),
    "lsa_score": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _P], _I32),
    "lsa_score_fp8_multihead": ([ctypes.POINTER(Shape), _I32, _I32, _P, _P, _P, _P, _P, _P],
                                _I32),
    "lsa_score_fp8_multihead_layers": ([ctypes.POINTER(Shape), _I32, _I32, _I32, _I32, _P, _P,
                                        _P, _P, _P, _P], _I32),
    "lsa_select_topk": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _P], _I32),
    "lsa_select_threshold_workspace_bytes": ([ctypes.POINTER(Shape)], ctypes.c_size_t),
    "lsa_select_threshold": ([ctypes.POINTER(Shape), _P, _P, ctypes.c_float, _I32, _P, _P, _P,
                              _P, ctypes.c_size_t, _P], _I32),
    "lsa_gather_chunks": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P], _I32),
    "lsa_append_kv": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P], _I32),
    "lsa_keep_recent": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _I32, _P, _P, _P], _I32),
    "lsa_sparse_decode_attn_varlen": ([ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P], _I32),
    "lsa_pool_delta_update": ([ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P], _I32),
    "lsa_sparse_decode_attn": ([ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, ctypes.c_size_t, _P], _I32),
    "lsa_decode_step": ([ctypes.POINTER(Shape), ctypes.POINTER(StepArgs), _P, ctypes.c_size_t,
                         _P], _I32),
    "lsa_bench_copy": ([_P, _P, ctypes.c_size_t, _P], _I32),
    "lsa_bench_attention_partial": ([ctypes.POINTER(Shape), _I32, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P], _I32),
    "lsa_bench_flush": ([_P, ctypes.c_size_t, _P], _I32),
    "lsa_bench_read": ([_P, ctypes.c_size_t, _I32, _P, ctypes.c_size_t, _P], _I32),
}

_lib = None


def library() -> ctypes.CDLL:
    """The loaded liblsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    try:
        return library().lsa_status_string(status).decode()
    except Exception:  # pragma: no cover - library unavailable while formatting an error
        return f"status {status}"


def _check(status: int, where: str) -> None:
    if status != LSA_OK:
        raise LsaError(status, where)


# ----------------------------------------------------------------------------- shapes
@dataclass
class ProblemShape:
    batch: int
    chunk_size: int
    index_dim: int
    num_q_heads: int
    head_dim_qk: int
    head_dim_v: int
    v_aliases_k: bool
    dtype: torch.dtype
    softmax_scale: float
    max_chunks: int
    max_k: int
    total_chunks: int
    total_k: int
    attn_tiles_per_block: int = 0
    # every stream has max_chunks chunks and keeps max_k of them
    # (LSA_SHAPE_UNIFORM): the kernels derive the offsets instead of reading
    # them.  Set it to False for keep sets whose sizes the device decides.
    uniform: bool = False

    def c(self) -> Shape:
        if self.dtype == torch.bfloat16:
            dt = DTYPE_BF16
        elif self.dtype == torch.float32:
            dt = DTYPE_F32
        else:
            raise ValueError(f"unsupported dtype {self.dtype}")
        return Shape(self.batch, self.chunk_size, self.index_dim, self.num_q_heads,
                      self.head_dim_qk, self.head_dim_v, int(bool(self.v_aliases_k)), dt,
                      float(self.softmax_scale), self.max_chunks, self.max_k,
                      self.total_chunks, self.total_k, self.attn_tiles_per_block,
                      SHAPE_UNIFORM if self.uniform else 0)


def keep_count(n_chunks: int, ratio_num: int, ratio_den: int, round_up: bool) -> int:
    return int(library().lsa_keep_count(n_chunks, ratio_num, ratio_den, int(round_up)))


def workspace_bytes(shape: ProblemShape) -> int:
    return int(library().lsa_workspace_bytes(ctypes.byref(shape.c())))


def attention_plan(shape: ProblemShape) -> dict:
    """lsa_attention_plan: how attention runs for this shape on the current
    device (kernel, launch grid, whether the partials merge in the kernel,
    split-heads form, top-k inside the kernel)."""
    info = AttnPlanInfo()
    _check(library().lsa_attention_plan(ctypes.byref(shape.c()), ctypes.byref(info)),
           "lsa_attention_plan")
    return {"kernel": ATTN_KERNEL_NAMES.get(info.kernel, str(info.kernel)), "grid": info.grid,
            "partial_rows": info.partial_rows, "tiles_per_chunk": info.tiles_per_chunk,
            "merge_in_kernel": bool(info.merge_in_kernel), "split_heads": bool(info.split_heads),
            "select_in_kernel": bool(info.select_in_kernel)}


def allocate_workspace(shape: ProblemShape, device) -> torch.Tensor:
    """Workspace for lsa_sparse_decode_attn / lsa_decode_step, zero-filled
    as the library requires before first use (calls leave it zeroed)."""
    n = workspace_bytes(shape)
    if n == 0:
        raise LsaError(LSA_ERR_UNSUPPORTED, "lsa_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def select_threshold_workspace_bytes(shape: ProblemShape) -> int:
    return int(library().lsa_select_threshold_workspace_bytes(ctypes.byref(shape.c())))


# ----------------------------------------------------------------------------- helpers
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    # torch's current HIP stream of the current device (the capture stream
    # under graph capture), read without building a Stream object
    return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return t


# ----------------------------------------------------------------------------- entry points
def score(shape: ProblemShape, q_idx, emb, chunk_off, scores=None, stream=None) -> torch.Tensor:
    """lsa_score: fp32 scores [total_chunks]."""
    _dev(q_idx, "q_idx", shape.dtype, 2)
    _dev(emb, "emb", shape.dtype, 2)
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    if scores is None:
        scores = torch.empty(shape.total_chunks, dtype=torch.float32, device=emb.device)
    _dev(scores, "scores", torch.float32, 1)
    _check(library().lsa_score(ctypes.byref(shape.c()), _ptr(q_idx), _ptr(emb), _ptr(chunk_off),
                               _ptr(scores), _stream(stream)), "lsa_score")
    return scores


def score_fp8_multihead(shape: ProblemShape, q_heads, head_w, records, chunk_off, scores=None,
                        stream=None) -> torch.Tensor:
    """lsa_score_fp8_multihead: fp32 multi-head scores [total_chunks] of
    compressed-key records.  q_heads [B][heads][head_dim] bf16, head_w
    [B][heads] fp32, records [total_chunks][head_dim + 4] uint8."""
    _dev(q_heads, "q_heads", torch.bfloat16, 3)
    _dev(head_w, "head_w", torch.float32, 2)
    _dev(records, "records", torch.uint8, 2)
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    B, heads, head_dim = q_heads.shape
    if head_w.shape != (B, heads) or records.shape != (shape.total_chunks, head_dim + 4):
        raise ValueError("q_heads / head_w / records shapes do not agree")
    if scores is None:
        scores = torch.empty(shape.total_chunks, dtype=torch.float32, device=records.device)
    _dev(scores, "scores", torch.float32, 1)
    _check(library().lsa_score_fp8_multihead(ctypes.byref(shape.c()), heads, head_dim,
                                             _ptr(q_heads), _ptr(head_w), _ptr(records),
                                             _ptr(chunk_off), _ptr(scores), _stream(stream)),
           "lsa_score_fp8_multihead")
    return scores


def score_fp8_multihead_layers(shape: ProblemShape, q_heads, head_w, records, chunk_off,
                               combine: int = COMBINE_MAX, scores=None,
                               stream=None) -> torch.Tensor:
    """lsa_score_fp8_multihead_layers: fp32 ensemble scores [total_chunks] over
    L layers.  q_heads [L][B][heads][head_dim] bf16, head_w [L][B][heads]
    fp32, records [L][total_chunks][head_dim + 4] uint8."""
    _dev(q_heads, "q_heads", torch.bfloat16, 4)
    _dev(head_w, "head_w", torch.float32, 3)
    _dev(records, "records", torch.uint8, 3)
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    L, B, heads, head_dim = q_heads.shape
    if head_w.shape != (L, B, heads) or records.shape != (L, shape.total_chunks, head_dim + 4):
        raise ValueError("q_heads / head_w / records shapes do not agree")
    if scores is None:
        scores = torch.empty(shape.total_chunks, dtype=torch.float32, device=records.device)
    _dev(scores, "scores", torch.float32, 1)
    _check(library().lsa_score_fp8_multihead_layers(
        ctypes.byref(shape.c()), L, int(combine), heads, head_dim, _ptr(q_heads), _ptr(head_w),
        _ptr(records), _ptr(chunk_off), _ptr(scores), _stream(stream)),
        "lsa_score_fp8_multihead_layers")
    return scores


def select_threshold(shape: ProblemShape, scores, chunk_off, threshold: float, max_keep: int = 0,
                     sel_off=None, sel_idx=None, fallback=None, workspace=None, stream=None):
    """lsa_select_threshold: (sel_off [B+1], sel_idx [total_chunks] of which
    the first sel_off[B] are meaningful, fallback [B]) int32 tensors."""
    _dev(scores, "scores", torch.float32, 1)
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    dev = scores.device
    if sel_off is None:
        sel_off = torch.empty(shape.batch + 1, dtype=torch.int32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty(shape.total_chunks, dtype=torch.int32, device=dev)
    if fallback is None:
        fallback = torch.empty(shape.batch, dtype=torch.int32, device=dev)
    if workspace is None:
        n = select_threshold_workspace_bytes(shape)
        if n == 0:
            raise LsaError(LSA_ERR_UNSUPPORTED, "lsa_select_threshold_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _dev(sel_off, "sel_off", torch.int32, 1)
    _dev(sel_idx, "sel_idx", torch.int32, 1)
    _dev(fallback, "fallback", torch.int32, 1)
    _dev(workspace, "workspace", torch.uint8, 1)
    if sel_off.numel() != shape.batch + 1 or sel_idx.numel() < shape.total_chunks or \
            fallback.numel() != shape.batch:
        raise ValueError("sel_off / sel_idx / fallback sizes do not match the shape")
    _check(library().lsa_select_threshold(
        ctypes.byref(shape.c()), _ptr(scores), _ptr(chunk_off), float(threshold), int(max_keep),
        _ptr(sel_off), _ptr(sel_idx), _ptr(fallback), _ptr(workspace), workspace.numel(),
        _stream(stream)), "lsa_select_threshold")
    return sel_off, sel_idx, fallback


def select_topk(shape: ProblemShape, scores, chunk_off, sel_off, sel_idx=None,
                stream=None) -> torch.Tensor:
    """lsa_select_topk: ascending kept chunk indices [total_k] int32."""
    _dev(scores, "scores", torch.float32, 1)
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    _dev(sel_off, "sel_off", torch.int32, 1)
    if sel_idx is None:
        sel_idx = torch.empty(shape.total_k, dtype=torch.int32, device=scores.device)
    _dev(sel_idx, "sel_idx", torch.int32, 1)
    _check(library().lsa_select_topk(ctypes.byref(shape.c()), _ptr(scores), _ptr(chunk_off),
                                     _ptr(sel_off), _ptr(sel_idx), _stream(stream)),
           "lsa_select_topk")
    return sel_idx


def gather_chunks(shape: ProblemShape, k_store, v_store, tok_off, sel_idx, sel_off,
                  k_pool=None, v_pool=None, stream=None):
    """lsa_gather_chunks: (k_pool [total_k, C, dqk], v_pool or None)."""
    _dev(k_store, "k_store", shape.dtype, 2)
    _dev(tok_off, "tok_off", torch.int64, 1)
    _dev(sel_idx, "sel_idx", torch.int32, 1)
    _dev(sel_off, "sel_off", torch.int32, 1)
    C = shape.chunk_size
    if k_pool is None:
        k_pool = torch.empty((shape.total_k, C, shape.head_dim_qk), dtype=shape.dtype,
                             device=k_store.device)
    _dev(k_pool, "k_pool", shape.dtype)
    if shape.v_aliases_k:
        if v_store is not None or v_pool is not None:
            raise ValueError("v_store / v_pool must be None when V aliases K")
    else:
        _dev(v_store, "v_store", shape.dtype, 2)
        if v_pool is None:
            v_pool = torch.empty((shape.total_k, C, shape.head_dim_v), dtype=shape.dtype,
                                 device=k_store.device)
        _dev(v_pool, "v_pool", shape.dtype)
    _check(library().lsa_gather_chunks(ctypes.byref(shape.c()), _ptr(k_store), _ptr(v_store),
                                       _ptr(tok_off), _ptr(sel_idx), _ptr(sel_off),
                                       _ptr(k_pool), _ptr(v_pool), _stream(stream)),
           "lsa_gather_chunks")
    return k_pool, v_pool


def append_kv(shape: ProblemShape, k_new, v_new, base_off, seq_len, k_store, v_store=None,
              stream=None) -> None:
    """lsa_append_kv: row seq_len[b] of each stream receives k_new[b] (and
    v_new[b]); seq_len advances in place."""
    _dev(k_new, "k_new", shape.dtype, 2)
    _dev(k_store, "k_store", shape.dtype, 2)
    if shape.v_aliases_k:
        if v_new is not None or v_store is not None:
            raise ValueError("v_new / v_store must be None when V aliases K")
    else:
        _dev(v_new, "v_new", shape.dtype, 2)
        _dev(v_store, "v_store", shape.dtype, 2)
    _dev(base_off, "base_off", torch.int64, 1)
    _dev(seq_len, "seq_len", torch.int64, 1)
    if k_new.shape[0] != shape.batch or seq_len.numel() != shape.batch or \
            base_off.numel() != shape.batch + 1:
        raise ValueError("k_new / seq_len / base_off sizes do not match the batch")
    _check(library().lsa_append_kv(ctypes.byref(shape.c()), _ptr(k_new), _ptr(v_new),
                                   _ptr(base_off), _ptr(seq_len), _ptr(k_store), _ptr(v_store),
                                   _stream(stream)), "lsa_append_kv")


def keep_recent(shape: ProblemShape, seq_len, chunk_off, sel_idx, sel_off, max_recent: int,
                out_idx=None, out_off=None, stream=None):
    """lsa_keep_recent: (out_off [B+1], out_idx [total_k + B*max_recent]) of
    which the first out_off[B] indices are meaningful."""
    _dev(seq_len, "seq_len", torch.int64, 1)
    for t, n in ((chunk_off, "chunk_off"), (sel_idx, "sel_idx"), (sel_off, "sel_off")):
        _dev(t, n, torch.int32, 1)
    dev = sel_idx.device
    cap = shape.total_k + shape.batch * max(0, int(max_recent))
    if out_idx is None:
        out_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if out_off is None:
        out_off = torch.empty(shape.batch + 1, dtype=torch.int32, device=dev)
    _dev(out_idx, "out_idx", torch.int32, 1)
    _dev(out_off, "out_off", torch.int32, 1)
    if out_idx.numel() < cap or out_off.numel() != shape.batch + 1:
        raise ValueError("out_idx / out_off too small for the shape")
    _check(library().lsa_keep_recent(ctypes.byref(shape.c()), _ptr(seq_len), _ptr(chunk_off),
                                     _ptr(sel_idx), _ptr(sel_off), int(max_recent),
                                     _ptr(out_idx), _ptr(out_off), _stream(stream)),
           "lsa_keep_recent")
    return out_off, out_idx


def sparse_decode_attn_varlen(shape: ProblemShape, q, k_base, v_base, base_off, seq_len, sel_idx,
                              sel_off, kv_mode: int = KV_STORE, out=None, lse=None,
                              workspace=None, stream=None):
    """lsa_sparse_decode_attn_varlen: (out [B, H, dv], lse [B, H]) over a
    capacity layout (rows of stream b from base_off[b], L_b = seq_len[b])."""
    _dev(q, "q", shape.dtype, 3)
    _dev(k_base, "k_base", shape.dtype)
    if shape.v_aliases_k:
        if v_base is not None:
            raise ValueError("v_base must be None when V aliases K")
    else:
        _dev(v_base, "v_base", shape.dtype)
    _dev(base_off, "base_off", torch.int64, 1)
    _dev(seq_len, "seq_len", torch.int64, 1)
    _dev(sel_idx, "sel_idx", torch.int32, 1)
    _dev(sel_off, "sel_off", torch.int32, 1)
    dev = q.device
    if out is None:
        out = torch.empty((shape.batch, shape.num_q_heads, shape.head_dim_v),
                          dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((shape.batch, shape.num_q_heads), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = allocate_workspace(shape, dev)
    _dev(workspace, "workspace", torch.uint8, 1)
    _check(library().lsa_sparse_decode_attn_varlen(
        ctypes.byref(shape.c()), int(kv_mode), _ptr(q), _ptr(k_base), _ptr(v_base),
        _ptr(base_off), _ptr(seq_len), _ptr(sel_idx), _ptr(sel_off), _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream(stream)), "lsa_sparse_decode_attn_varlen")
    return out, lse


def _pinned(t, name: str, dtype):
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned():
        raise ValueError(f"{name} must be a page-locked (pinned) host tensor")
    if not t.is_contiguous() or t.dtype != dtype or t.dim() != 2:
        raise ValueError(f"{name} must be a contiguous 2-D {dtype} tensor")
    return t


def pool_delta_update(shape: ProblemShape, k_host, v_host, tok_off, chunk_off, sel_idx, sel_off,
                      table, k_pool, v_pool=None, loads=None, load_count=None, stream=None):
    """lsa_pool_delta_update: copies the newly kept chunks from the pinned host
    stores into the pool and rewrites the slot table in place; returns
    (loads [total_k], load_count [B]) int32 device tensors."""
    _pinned(k_host, "k_host", shape.dtype)
    if shape.v_aliases_k:
        if v_host is not None or v_pool is not None:
            raise ValueError("v_host / v_pool must be None when V aliases K")
    else:
        _pinned(v_host, "v_host", shape.dtype)
        _dev(v_pool, "v_pool", shape.dtype)
    _dev(k_pool, "k_pool", shape.dtype)
    for t, n in ((tok_off, "tok_off"),):
        _dev(t, n, torch.int64, 1)
    for t, n in ((chunk_off, "chunk_off"), (sel_idx, "sel_idx"), (sel_off, "sel_off"),
                 (table, "table")):
        _dev(t, n, torch.int32, 1)
    dev = table.device
    if loads is None:
        loads = torch.empty(shape.total_k, dtype=torch.int32, device=dev)
    if load_count is None:
        load_count = torch.empty(shape.batch, dtype=torch.int32, device=dev)
    _dev(loads, "loads", torch.int32, 1)
    _dev(load_count, "load_count", torch.int32, 1)
    if table.numel() != shape.total_k or loads.numel() != shape.total_k or \
            load_count.numel() != shape.batch:
        raise ValueError("table / loads / load_count sizes do not match the shape")
    _check(library().lsa_pool_delta_update(
        ctypes.byref(shape.c()), _ptr(k_host), _ptr(v_host), _ptr(tok_off), _ptr(chunk_off),
        _ptr(sel_idx), _ptr(sel_off), _ptr(table), _ptr(loads), _ptr(load_count), _ptr(k_pool),
        _ptr(v_pool), _stream(stream)), "lsa_pool_delta_update")
    return loads, load_count


def sparse_decode_attn(shape: ProblemShape, q, k_base, v_base, tok_off, sel_idx, sel_off,
                       kv_mode: int = KV_STORE, out=None, lse=None, workspace=None,
                       stream=None):
    """lsa_sparse_decode_attn: (out [B, H, dv] fp32, lse [B, H] fp32)."""
    _dev(q, "q", shape.dtype, 3)
    _dev(k_base, "k_base", shape.dtype)
    if shape.v_aliases_k:
        if v_base is not None:
            raise ValueError("v_base must be None when V aliases K")
    else:
        _dev(v_base, "v_base", shape.dtype)
    _dev(tok_off, "tok_off", torch.int64, 1)
    _dev(sel_idx, "sel_idx", torch.int32, 1)
    _dev(sel_off, "sel_off", torch.int32, 1)
    dev = q.device
    if out is None:
        out = torch.empty((shape.batch, shape.num_q_heads, shape.head_dim_v),
                          dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((shape.batch, shape.num_q_heads), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32)
    _dev(lse, "lse", torch.float32)
    if workspace is None:
        workspace = allocate_workspace(shape, dev)
    _dev(workspace, "workspace", torch.uint8, 1)
    _check(library().lsa_sparse_decode_attn(
        ctypes.byref(shape.c()), int(kv_mode), _ptr(q), _ptr(k_base), _ptr(v_base),
        _ptr(tok_off), _ptr(sel_idx), _ptr(sel_off), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)), "lsa_sparse_decode_attn")
    return out, lse


TABLE_ERR_CHUNK_OFF = 1
TABLE_ERR_SEL_OFF = 2
TABLE_ERR_KEEP = 4
TABLE_ERR_TOK_OFF = 8
TABLE_ERR_SEL_IDX = 16

# LSA_DEBUG_CHECKS=1: attention and decode-step calls first check their tables
# on the device and raise on a violation (synchronises; debugging only)
_DEBUG_CHECKS = os.environ.get("LSA_DEBUG_CHECKS", "0") == "1"


def check_tables(shape: ProblemShape, chunk_off, sel_off, tok_off=None, sel_idx=None,
                 kept_ascending: bool = True, flags=None, stream=None) -> int:
    """lsa_check_tables: OR of the TABLE_ERR_* bits of every stream (0: the
    device-side preconditions hold).  Synchronises the stream to read the
    flag back; a debugging aid, not for the hot path."""
    _dev(chunk_off, "chunk_off", torch.int32, 1)
    _dev(sel_off, "sel_off", torch.int32, 1)
    if tok_off is not None:
        _dev(tok_off, "tok_off", torch.int64, 1)
    if sel_idx is not None:
        _dev(sel_idx, "sel_idx", torch.int32, 1)
    if flags is None:
        flags = torch.empty(1, dtype=torch.int32, device=chunk_off.device)
    _dev(flags, "flags", torch.int32)
    _check(library().lsa_check_tables(ctypes.byref(shape.c()), _ptr(tok_off), _ptr(chunk_off),
                                      _ptr(sel_off), _ptr(sel_idx), int(bool(kept_ascending)),
                                      _ptr(flags), _stream(stream)), "lsa_check_tables")
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    return int(flags[0].item())


def _debug_check(shape, chunk_off, sel_off, tok_off, sel_idx, where):
    if chunk_off is None:  # attention calls carry no chunk table: rebuild it from the shape
        return
    bad = check_tables(shape, chunk_off, sel_off, tok_off, sel_idx, kept_ascending=False)
    if bad:
        raise ValueError(f"{where}: device tables violate the preconditions (flags {bad:#x})")


def _event_ptr(ev):
    if ev is None:
        return None
    if not ev.cuda_event:  # torch creates the HIP event lazily on first record
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def _step_args(shape: ProblemShape, q_idx, emb, chunk_off, scores, sel_off, sel_idx, q,
               k_store, v_store, tok_off, out, lse, reindex, materialize_pool, k_pool, v_pool,
               ev_attn_begin, ev_attn_end, step, reindex_every, where) -> StepArgs:
    if reindex_every < 0 or (reindex_every > 0 and step < 0):
        raise ValueError("reindex_every must be >= 0 and step >= 0")
    # with the schedule in the library's hands every step may re-index: the
    # scoring inputs are always checked and passed
    scoring = bool(reindex) or reindex_every > 0
    if _DEBUG_CHECKS:
        due = reindex_due(step, reindex_every) if reindex_every > 0 else bool(reindex)
        _debug_check(shape, chunk_off, sel_off, tok_off, None if due else sel_idx, where)
    for name, t, dt in [("q", q, shape.dtype), ("k_store", k_store, shape.dtype),
                        ("tok_off", tok_off, torch.int64), ("sel_off", sel_off, torch.int32),
                        ("sel_idx", sel_idx, torch.int32), ("out", out, torch.float32)]:
        _dev(t, name, dt)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if scoring:
        for name, t, dt in [("q_idx", q_idx, shape.dtype), ("emb", emb, shape.dtype),
                            ("chunk_off", chunk_off, torch.int32),
                            ("scores", scores, torch.float32)]:
            _dev(t, name, dt)
    return StepArgs(
        _ptr(q_idx) if scoring else None, _ptr(emb) if scoring else None,
        _ptr(chunk_off) if scoring else None, _ptr(scores) if scoring else None,
        _ptr(sel_off), _ptr(sel_idx), _ptr(q), _ptr(k_store), _ptr(v_store), _ptr(tok_off),
        _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse), int(bool(reindex)),
        int(bool(materialize_pool)), _event_ptr(ev_attn_begin), _event_ptr(ev_attn_end),
        int(reindex_every), 0, int(step))


class PreparedStep:
    """The arguments of lsa_decode_step (or, static=True, of
    lsa_decode_step_static) checked and marshalled once, for a decode loop
    that issues a step over the same buffers again and again: run() only sets
    the step number, the decode queries and the optional events, then calls
    the library (the re-index schedule, reindex_every >= 1, stays the
    library's).  Argument marshalling only, as everywhere in this module."""

    def __init__(self, shape: ProblemShape, *, q_idx, emb, chunk_off, scores, sel_off, sel_idx,
                 q, k_store, v_store, tok_off, out, lse, workspace=None,
                 materialize_pool: bool = False, k_pool=None, v_pool=None,
                 reindex_every: int = 1, static: bool = False):
        if reindex_every < 1:
            raise ValueError("a prepared step runs the library's schedule: reindex_every >= 1")
        self.shape = shape
        self._args = _step_args(shape, q_idx, emb, chunk_off, scores, sel_off, sel_idx, q,
                                k_store, v_store, tok_off, out, lse, True, materialize_pool,
                                k_pool, v_pool, None, None, 0, reindex_every,
                                "lsa_decode_step")
        self._tables = (chunk_off, sel_off, tok_off, sel_idx)
        self._keep = [q_idx, emb, scores, q, k_store, v_store, out, lse, k_pool, v_pool,
                      workspace]
        self._shape_c = shape.c()
        self._shape_ref = ctypes.byref(self._shape_c)
        self._args_ref = ctypes.byref(self._args)
        self._static = static
        if static:
            self._fn = library().lsa_decode_step_static
        else:
            _dev(workspace, "workspace", torch.uint8)
            self._fn = library().lsa_decode_step
            self._ws = ctypes.c_void_p(workspace.data_ptr())
            self._ws_n = workspace.numel()
        self._q = q

    def run(self, step: int, q=None, ev_attn_begin=None, ev_attn_end=None, stream=None):
        a = self._args
        if step < 0:
            raise ValueError("step must be >= 0")
        a.step = step
        if q is not None and q is not self._q:
            if not q.is_cuda or q.dtype != self.shape.dtype or not q.is_contiguous():
                raise ValueError("q must be a contiguous device tensor of the shape's dtype")
            a.q_dev = q.data_ptr()
            self._q = q
        a.ev_attn_begin = _event_ptr(ev_attn_begin)
        a.ev_attn_end = _event_ptr(ev_attn_end)
        if _DEBUG_CHECKS:
            co, so, to, si = self._tables
            due = reindex_due(step, a.reindex_every)
            _debug_check(self.shape, co, so, to, None if due else si, "PreparedStep.run")
        if self._static:
            st = self._fn(self._shape_ref, self._args_ref, _stream(stream))
        else:
            st = self._fn(self._shape_ref, self._args_ref, self._ws, self._ws_n, _stream(stream))
        if st != LSA_OK:
            raise LsaError(st, "lsa_decode_step_static" if self._static else "lsa_decode_step")


def decode_step(shape: ProblemShape, *, q_idx, emb, chunk_off, scores, sel_off, sel_idx, q,
                k_store, v_store, tok_off, out, lse, workspace, reindex: bool = True,
                materialize_pool: bool = False, k_pool=None, v_pool=None,
                ev_attn_begin=None, ev_attn_end=None, stream=None, step: int = 0,
                reindex_every: int = 0) -> None:
    """lsa_decode_step: one whole decode step (score -> select -> [gather] ->
    attention -> merge) enqueued by one call; outputs written in place.

    reindex_every > 0 hands the schedule to the library (re-index iff
    step % reindex_every == 0, ``reindex`` ignored); 0 leaves it to
    ``reindex``."""
    args = _step_args(shape, q_idx, emb, chunk_off, scores, sel_off, sel_idx, q, k_store,
                      v_store, tok_off, out, lse, reindex, materialize_pool, k_pool, v_pool,
                      ev_attn_begin, ev_attn_end, step, reindex_every, "lsa_decode_step")
    _dev(workspace, "workspace", torch.uint8)
    _check(library().lsa_decode_step(ctypes.byref(shape.c()), ctypes.byref(args),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "lsa_decode_step")


STATIC_SCRATCH_BYTES = 64 << 20  # LSA_STATIC_SCRATCH_BYTES


def decode_step_static(shape: ProblemShape, *, q_idx, emb, chunk_off, scores, sel_off, sel_idx,
                       q, k_store, v_store, tok_off, out, lse, reindex: bool = True,
                       materialize_pool: bool = False, k_pool=None, v_pool=None,
                       ev_attn_begin=None, ev_attn_end=None, stream=None, step: int = 0,
                       reindex_every: int = 0) -> None:
    """lsa_decode_step_static: lsa_decode_step with no workspace argument (the
    library's static per-device scratch holds the split partials); allocates
    nothing.  Calls on one device must not overlap."""
    args = _step_args(shape, q_idx, emb, chunk_off, scores, sel_off, sel_idx, q, k_store,
                      v_store, tok_off, out, lse, reindex, materialize_pool, k_pool, v_pool,
                      ev_attn_begin, ev_attn_end, step, reindex_every, "lsa_decode_step_static")
    _check(library().lsa_decode_step_static(ctypes.byref(shape.c()), ctypes.byref(args),
                                            _stream(stream)), "lsa_decode_step_static")


def reindex_due(step: int, reindex_every: int) -> bool:
    """lsa_reindex_due: whether decode step `step` re-scores and re-selects."""
    r = library().lsa_reindex_due(int(step), int(reindex_every))
    if r < 0:
        raise ValueError(f"invalid schedule: step={step}, reindex_every={reindex_every}")
    return bool(r)


def bench_attention_partial(shape: ProblemShape, q, k_base, v_base, tok_off, sel_idx, sel_off,
                            kv_mode: int, workspace, stream=None) -> None:
    """lsa_bench_attention_partial: the split-KV partial kernel alone (timing)."""
    _dev(q, "q", shape.dtype, 3)
    _dev(workspace, "workspace", torch.uint8, 1)
    _check(library().lsa_bench_attention_partial(
        ctypes.byref(shape.c()), int(kv_mode), _ptr(q), _ptr(k_base), _ptr(v_base),
        _ptr(tok_off), _ptr(sel_idx), _ptr(sel_off), _ptr(workspace), workspace.numel(),
        _stream(stream)), "lsa_bench_attention_partial")


def bench_copy(dst: torch.Tensor, src: torch.Tensor, nbytes: int, stream=None) -> None:
    _check(library().lsa_bench_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)),
           "lsa_bench_copy")


BENCH_READ_SINK_BYTES = 256 * 32 * 256 * 4  # LSA_BENCH_READ_SINK_BYTES


def bench_read(src: torch.Tensor, nbytes: int, pattern: int, sink: torch.Tensor,
               stream=None) -> None:
    """lsa_bench_read: stream-read nbytes of src in access pattern 0, 1 or 2."""
    _dev(src, "src")
    _dev(sink, "sink")
    _check(library().lsa_bench_read(_ptr(src), nbytes, int(pattern), _ptr(sink),
                                    sink.numel() * sink.element_size(), _stream(stream)),
           "lsa_bench_read")


def bench_flush(buf: torch.Tensor, stream=None) -> None:
    _check(library().lsa_bench_flush(_ptr(buf), buf.numel() * buf.element_size(),
                                     _stream(stream)), "lsa_bench_flush")
