"""learned_kv_chunk_amd: the Lookahead Sparse Attention decode hot path on MI355X (gfx950).

The binding over the C-ABI library ``liblsa.so`` lives in :mod:`.lsa`; seeded
synthetic inputs live in :mod:`.workloads`.  Importing the package loads
nothing: the HIP library is opened on first use and a missing library raises.
"""
__all__ = ["lsa", "workloads"]
