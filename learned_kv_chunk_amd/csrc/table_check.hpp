// table_check.hpp -- the device-side preconditions of lsa.h's offset tables
// and kept-chunk indices, as checks one stream at a time.
//
// The kernels of the library trust these tables (reading them costs memory
// round trips on the hot path); lsa_check_tables runs the checks below on
// the device for callers that want to catch a bad table before it turns into
// silently wrong output.  The functions only read the table entries the
// documented array sizes guarantee: tok_off / chunk_off / sel_off at b and
// b + 1, and sel_idx inside [sel_off[b], sel_off[b+1]) only when that range
// lies inside [0, total_k].  They are plain C++ so that the same code also
// builds for the host (LSA_HD defined empty), where it is exercised under the
// address and undefined-behaviour sanitizers.
#pragma once

#include <stdint.h>

#include "../../include/lsa.h"

#ifndef LSA_HD
#define LSA_HD __host__ __device__
#endif

namespace lsa {

// Value clamped to [0, cap]: the select kernels rank at most the keys one
// workgroup holds, whatever a violated precondition claims.
LSA_HD inline int32_t select_clamp_keys(int32_t v, int32_t cap) {
  return v < 0 ? 0 : (v > cap ? cap : v);
}

struct TableShape {
  int32_t B, C, max_chunks, max_k;
  int64_t total_chunks, total_k;
  int32_t uniform;  // LSA_SHAPE_UNIFORM set
};

// The stream's own range of kept indices, when it can be read safely.
struct StreamRange {
  int32_t s0, k, n;  // sel_off[b], k_b (0 when unreadable), N_b (>= 0)
};

// Checks of stream b's offset entries; tok_off may be null (not checked).
LSA_HD inline uint32_t table_check_offsets(const TableShape& s, int32_t b, const int64_t* tok_off,
                                           const int32_t* chunk_off, const int32_t* sel_off,
                                           StreamRange* range) {
  uint32_t e = 0;
  const int32_t c0 = chunk_off[b], c1 = chunk_off[b + 1];
  const int32_t s0 = sel_off[b], s1 = sel_off[b + 1];
  if (b == 0 && c0 != 0) e |= LSA_TABLE_ERR_CHUNK_OFF;
  if (b == 0 && s0 != 0) e |= LSA_TABLE_ERR_SEL_OFF;
  if (b == s.B - 1 && c1 != s.total_chunks) e |= LSA_TABLE_ERR_CHUNK_OFF;
  if (b == s.B - 1 && s1 != s.total_k) e |= LSA_TABLE_ERR_SEL_OFF;
  if (c0 < 0 || c1 < c0 || c1 > s.total_chunks ||
      static_cast<int64_t>(c1) - c0 > s.max_chunks)
    e |= LSA_TABLE_ERR_CHUNK_OFF;
  if (s0 < 0 || s1 < s0 || s1 > s.total_k || static_cast<int64_t>(s1) - s0 > s.max_k)
    e |= LSA_TABLE_ERR_SEL_OFF;
  if (s.uniform) {  // the offsets the kernels then compute instead of reading
    if (static_cast<int64_t>(c0) != static_cast<int64_t>(b) * s.max_chunks)
      e |= LSA_TABLE_ERR_CHUNK_OFF;
    if (static_cast<int64_t>(s0) != static_cast<int64_t>(b) * s.max_k) e |= LSA_TABLE_ERR_SEL_OFF;
  }
  const int64_t n = static_cast<int64_t>(c1) - c0;
  const int64_t k = static_cast<int64_t>(s1) - s0;
  if (k < 1 || k > n) e |= LSA_TABLE_ERR_KEEP;
  if (tok_off != nullptr) {
    const int64_t t0 = tok_off[b], t1 = tok_off[b + 1];
    if ((b == 0 && t0 != 0) || t0 < 0 || t1 < t0 ||
        (t1 - t0) / s.C + ((t1 - t0) % s.C != 0 ? 1 : 0) != n)
      e |= LSA_TABLE_ERR_TOK_OFF;
  }
  const bool readable = s0 >= 0 && s1 >= s0 && s1 <= s.total_k;
  range->s0 = readable ? s0 : 0;
  range->k = readable ? s1 - s0 : 0;
  range->n = n > 0 ? static_cast<int32_t>(n < INT32_MAX ? n : INT32_MAX) : 0;
  return e;
}

// Check of the i-th kept index of a stream (0 <= i < r.k): in [0, N_b), and
// above its predecessor when the set must be ascending.
LSA_HD inline uint32_t table_check_index(const int32_t* sel_idx, const StreamRange& r, int32_t i,
                                         bool ascending) {
  const int32_t x = sel_idx[r.s0 + i];
  uint32_t e = 0;
  if (x < 0 || x >= r.n) e |= LSA_TABLE_ERR_SEL_IDX;
  if (ascending && i > 0 && sel_idx[r.s0 + i - 1] >= x) e |= LSA_TABLE_ERR_SEL_IDX;
  return e;
}

}  // namespace lsa
