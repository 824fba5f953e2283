// Host build of the library's table checks (learned_kv_chunk_amd/csrc/
// table_check.hpp, compiled with LSA_HD empty), driven from stdin so that a
// test can run it under the address and undefined-behaviour sanitizers.
// Input: "B C max_chunks max_k total_chunks total_k uniform ascending has_tok
// has_sel", then tok_off (B+1), chunk_off (B+1), sel_off (B+1) and sel_idx
// (total_k values).  Every array is its own heap block of exactly that size,
// so a read outside it is reported by the sanitizer.  Output: the error bits
// of each stream, then their OR.
#include <stdio.h>
#include <stdlib.h>

#define LSA_HD
#include "table_check.hpp"

template <typename T>
static T* read_array(long n, const char* fmt) {
  T* a = static_cast<T*>(malloc(sizeof(T) * (n > 0 ? n : 1)));
  for (long i = 0; i < n; ++i) {
    long long v;
    if (scanf(fmt, &v) != 1) exit(2);
    a[i] = static_cast<T>(v);
  }
  return a;
}

int main() {
  lsa::TableShape s;
  long long tc, tk;
  int ascending, has_tok, has_sel;
  if (scanf("%d %d %d %d %lld %lld %d %d %d %d", &s.B, &s.C, &s.max_chunks, &s.max_k, &tc, &tk,
            &s.uniform, &ascending, &has_tok, &has_sel) != 10)
    return 2;
  s.total_chunks = tc;
  s.total_k = tk;
  int64_t* tok = read_array<int64_t>(s.B + 1, "%lld");
  int32_t* chunk = read_array<int32_t>(s.B + 1, "%lld");
  int32_t* sel_off = read_array<int32_t>(s.B + 1, "%lld");
  int32_t* sel_idx = read_array<int32_t>(tk, "%lld");
  uint32_t all = 0;
  for (int32_t b = 0; b < s.B; ++b) {
    lsa::StreamRange r;
    uint32_t e = lsa::table_check_offsets(s, b, has_tok ? tok : nullptr, chunk, sel_off, &r);
    if (has_sel)
      for (int32_t i = 0; i < r.k; ++i) e |= lsa::table_check_index(sel_idx, r, i, ascending != 0);
    printf("%u ", e);
    all |= e;
  }
  printf("%u\n", all);
  // the select kernels' clamp of key counts
  if (lsa::select_clamp_keys(5000, 4096) != 4096 || lsa::select_clamp_keys(-3, 10) != 0 ||
      lsa::select_clamp_keys(7, 10) != 7)
    return 3;
  free(tok);
  free(chunk);
  free(sel_off);
  free(sel_idx);
  return 0;
}
