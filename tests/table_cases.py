"""Offset tables and kept indices that break lsa.h's device-side
preconditions one at a time (every entry still inside the documented array
sizes), with the error bits lsa_check_tables must report.  Shared by the host
build of the checks (tests/test_table_check.py) and the device check
(tests/test_gpu_checks.py)."""
import dataclasses

import numpy as np

CHUNK, SEL, KEEP, TOK, IDX = 1, 2, 4, 8, 16


@dataclasses.dataclass
class Case:
    name: str
    C: int
    max_chunks: int
    max_k: int
    tok_off: list
    chunk_off: list
    sel_off: list
    sel_idx: list
    expect: int
    ascending: bool = True
    uniform: bool = False
    total_chunks: int = -1   # -1: chunk_off[-1]
    total_k: int = -1        # -1: len(sel_idx)

    @property
    def B(self):
        return len(self.chunk_off) - 1

    def totals(self):
        tc = self.chunk_off[-1] if self.total_chunks < 0 else self.total_chunks
        tk = len(self.sel_idx) if self.total_k < 0 else self.total_k
        return tc, tk


# a valid ragged batch: C = 4, lengths 9, 4, 16 -> 3, 1, 4 chunks; keep 2, 1, 2
GOOD = dict(C=4, max_chunks=4, max_k=2, tok_off=[0, 9, 13, 29], chunk_off=[0, 3, 4, 8],
            sel_off=[0, 2, 3, 5], sel_idx=[0, 2, 0, 1, 3])


def _case(name, expect, **kw):
    d = dict(GOOD)
    d.update(kw)
    return Case(name=name, expect=expect, **d)


CASES = [
    _case("valid", 0),
    _case("valid_unordered_pool_table", 0, sel_idx=[2, 0, 0, 3, 1], ascending=False),
    _case("unordered_but_ascending_required", IDX, sel_idx=[2, 0, 0, 3, 1]),
    _case("duplicate_kept_index", IDX, sel_idx=[1, 1, 0, 1, 3]),
    _case("kept_index_past_stream", IDX, sel_idx=[0, 3, 0, 1, 3]),
    _case("negative_kept_index", IDX, sel_idx=[0, 2, -1, 1, 3], ascending=False),
    # stream 1 has -1 chunks (so its kept index 0 is out of range too) and
    # stream 2 six chunks for 16 tokens
    _case("chunk_off_decreasing", CHUNK | KEEP | TOK | IDX, chunk_off=[0, 3, 2, 8],
          max_chunks=6),
    # stream 0: 2 chunks for 9 tokens, and its kept index 2 is past them
    _case("chunk_off_first_not_zero", CHUNK | TOK | IDX, chunk_off=[1, 3, 4, 8]),
    _case("stream_longer_than_max_chunks", CHUNK, max_chunks=3),
    _case("chunk_total_mismatch", CHUNK, total_chunks=9),
    # stream 0 now keeps [0, 2, 0]: not ascending
    _case("sel_off_decreasing", SEL | KEEP | IDX, sel_off=[0, 3, 2, 5], max_k=3),
    _case("sel_off_past_total", SEL | KEEP, sel_off=[0, 2, 6, 5], max_k=4),
    _case("keep_more_than_chunks", KEEP | IDX, sel_off=[0, 1, 3, 5], sel_idx=[0, 0, 1, 1, 3]),
    _case("keep_zero", KEEP, sel_off=[0, 2, 2, 4], sel_idx=[0, 2, 1, 3], max_k=2),
    _case("tok_off_chunk_count_mismatch", TOK, tok_off=[0, 9, 14, 29]),
    _case("tok_off_decreasing", TOK, tok_off=[0, 9, 8, 29]),
    Case("uniform_offsets_wrong", C=4, max_chunks=3, max_k=2, tok_off=[0, 12, 24],
         chunk_off=[0, 2, 6], sel_off=[0, 2, 4], sel_idx=[0, 1, 0, 2], expect=CHUNK | TOK,
         uniform=True),
    Case("uniform_valid", C=4, max_chunks=3, max_k=2, tok_off=[0, 12, 24], chunk_off=[0, 3, 6],
         sel_off=[0, 2, 4], sel_idx=[0, 1, 0, 2], expect=0, uniform=True),
]


def as_arrays(c: Case):
    return (np.array(c.tok_off, np.int64), np.array(c.chunk_off, np.int32),
            np.array(c.sel_off, np.int32), np.array(c.sel_idx, np.int32))
