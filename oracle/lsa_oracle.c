/*
 * lsa_oracle.c -- plain, slow, double-precision CPU oracle for the LSA decode
 * hot path.  TEST INFRASTRUCTURE ONLY (see lsa_oracle.h): the product path
 * never links or calls it.
 *
 * Each function follows the definition of its step as the pages state it:
 *   oracle_score      dual-encoder inner product per chunk (wiki note
 *                     flowchart + "Key points"; review section 3-2-4; abstract).
 *   oracle_select     top-k keep set per stream (review section 3-2-3 step 5);
 *                     ties go to the lower chunk index, NaN ranks last.
 *   oracle_gather     copy of the kept chunks into a resident pool (wiki note
 *                     flowchart, its resident-chunk node; molayo explainer,
 *                     the paragraph on gathering only the selected chunks).
 *   oracle_attention  softmax attention restricted to the kept chunks' tokens
 *                     (review section 3-2-3 steps 6-7), computed with a full
 *                     max pass then a weighted-sum pass.
 *   oracle_score_fp8mh  the multi-head scorer of float8 compressed-key chunk
 *                     records (review sections 3-2-1, 3-2-2, 4-3): decode
 *                     each key value, dot with every head's query, scale,
 *                     ReLU, weighted sum over heads.
 *   oracle_score_fp8mh_layers  the same per layer, combined by max or mean
 *                     (review section 3-2-2, the layer ensemble).
 *   oracle_select_threshold  threshold keep mask, capped by a top-k, with a
 *                     dense fallback for a stream where no chunk passes
 *                     (review section 3-2-3 step 5, sections 4-3 and 5-1).
 *   oracle_pool_delta  the pool's slot table after a re-index when only the
 *                     newly kept chunks are copied in (wiki note flowchart,
 *                     the swap between GPU and host memory).
 *   oracle_keep_recent  the attention keep set of a context that grew since
 *                     the last re-index: kept chunks, the last scored chunk
 *                     and the chunks not yet scored (the newest max_recent
 *                     of those two kinds when the bound binds).
 */
#include "lsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one stored element to double. */
static double elem(const void* base, int64_t i, int32_t dtype) {
  if (dtype == ORACLE_BF16) {
    uint16_t h = ((const uint16_t*)base)[i];
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

int32_t oracle_keep_count(int32_t n_chunks, int32_t num, int32_t den, int32_t round_up) {
  if (n_chunks <= 0 || num <= 0 || den <= 0) return 0;
  int64_t p = (int64_t)n_chunks * (int64_t)num;
  int64_t k = round_up ? (p + den - 1) / den : p / den;
  if (k < 1) k = 1;
  if (k > n_chunks) k = n_chunks;
  return (int32_t)k;
}

void oracle_score(int32_t B, int32_t D, int32_t dtype, const void* q, const void* emb,
                  const int32_t* chunk_off, double* scores) {
  for (int32_t b = 0; b < B; ++b) {
    for (int64_t row = chunk_off[b]; row < chunk_off[b + 1]; ++row) {
      double s = 0.0;
      for (int32_t j = 0; j < D; ++j)
        s += elem(q, (int64_t)b * D + j, dtype) * elem(emb, row * D + j, dtype);
      scores[row] = s;
    }
  }
}

typedef struct {
  double s;
  int32_t n;
} ranked;

/* Rank order: higher score first; NaN after every number; equal scores (and
 * NaN among NaN) by lower chunk index.  -0.0 and +0.0 compare equal. */
static int rank_cmp(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  int an = isnan(a->s), bn = isnan(b->s);
  if (an != bn) return an ? 1 : -1;
  if (!an) {
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
  }
  return (a->n < b->n) ? -1 : (a->n > b->n);
}

static int int_cmp(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int32_t oracle_select(int32_t B, const double* scores, const int32_t* chunk_off,
                      const int32_t* sel_off, int32_t* sel_idx) {
  for (int32_t b = 0; b < B; ++b) {
    int32_t n = chunk_off[b + 1] - chunk_off[b];
    int32_t k = sel_off[b + 1] - sel_off[b];
    if (k < 0 || k > n) return -1;
    if (k == 0) continue;
    ranked* r = (ranked*)malloc(sizeof(ranked) * (size_t)n);
    for (int32_t i = 0; i < n; ++i) {
      r[i].s = scores[chunk_off[b] + i];
      r[i].n = i;
    }
    qsort(r, (size_t)n, sizeof(ranked), rank_cmp);
    int32_t* out = sel_idx + sel_off[b];
    for (int32_t i = 0; i < k; ++i) out[i] = r[i].n;
    qsort(out, (size_t)k, sizeof(int32_t), int_cmp);
    free(r);
  }
  return 0;
}

void oracle_gather(int32_t B, int32_t C, int64_t row_bytes, const void* store,
                   const int64_t* tok_off, const int32_t* sel_idx, const int32_t* sel_off,
                   void* pool) {
  const unsigned char* src = (const unsigned char*)store;
  unsigned char* dst = (unsigned char*)pool;
  for (int32_t b = 0; b < B; ++b) {
    int64_t len = tok_off[b + 1] - tok_off[b];
    for (int32_t j = sel_off[b]; j < sel_off[b + 1]; ++j) {
      int64_t first = (int64_t)sel_idx[j] * C;
      for (int32_t r = 0; r < C; ++r) {
        unsigned char* d = dst + ((int64_t)j * C + r) * row_bytes;
        if (first + r < len)
          memcpy(d, src + (tok_off[b] + first + r) * row_bytes, (size_t)row_bytes);
        else
          memset(d, 0, (size_t)row_bytes);
      }
    }
  }
}

void oracle_attention(int32_t B, int32_t H, int32_t dqk, int32_t dv, int32_t v_aliases_k,
                      int32_t dtype, int32_t C, double scale, const void* Q, const void* K,
                      const void* V, const int64_t* tok_off, const int32_t* sel_idx,
                      const int32_t* sel_off, double* out, double* lse, int32_t nthreads) {
  const void* vbase = v_aliases_k ? K : V;
  const int64_t vstride = v_aliases_k ? dqk : dv;
  const int64_t pairs = (int64_t)B * H;
  if (nthreads < 1) nthreads = 1;
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (int64_t p = 0; p < pairs; ++p) {
    const int32_t b = (int32_t)(p / H);
    const int32_t h = (int32_t)(p % H);
    const int64_t len = tok_off[b + 1] - tok_off[b];
    const int64_t max_tok = (int64_t)(sel_off[b + 1] - sel_off[b]) * C;
    double* x = (double*)malloc(sizeof(double) * (size_t)(max_tok > 0 ? max_tok : 1));
    int64_t* row = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_tok > 0 ? max_tok : 1));
    int64_t nt = 0;
    /* pass 1: logits of every kept token, and their maximum */
    double m = -INFINITY;
    for (int32_t j = sel_off[b]; j < sel_off[b + 1]; ++j) {
      int64_t first = (int64_t)sel_idx[j] * C;
      for (int64_t t = first; t < first + C && t < len; ++t) {
        int64_t r = tok_off[b] + t;
        double dot = 0.0;
        for (int32_t i = 0; i < dqk; ++i)
          dot += elem(Q, ((int64_t)b * H + h) * dqk + i, dtype) * elem(K, r * dqk + i, dtype);
        x[nt] = scale * dot;
        row[nt] = r;
        if (x[nt] > m) m = x[nt];
        ++nt;
      }
    }
    double* o = out + ((int64_t)b * H + h) * dv;
    for (int32_t c = 0; c < dv; ++c) o[c] = 0.0;
    if (nt == 0) {
      lse[(int64_t)b * H + h] = -INFINITY;
    } else {
      /* pass 2: normaliser and weighted sum of value rows */
      double z = 0.0;
      for (int64_t i = 0; i < nt; ++i) {
        double w = exp(x[i] - m);
        z += w;
        for (int32_t c = 0; c < dv; ++c) o[c] += w * elem(vbase, row[i] * vstride + c, dtype);
      }
      for (int32_t c = 0; c < dv; ++c) o[c] /= z;
      lse[(int64_t)b * H + h] = m + log(z);
    }
    free(x);
    free(row);
  }
}

double oracle_fp8_e4m3(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 15;
  const int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);             /* subnormal: m / 8 * 2^(1 - 7) */
  else
    v = ldexp((double)(8 + m), e - 10);   /* (1 + m / 8) * 2^(e - 7) */
  return sign ? -v : v;
}

void oracle_score_fp8mh(int32_t B, int32_t Hs, int32_t D, int32_t dtype, const void* q,
                        const float* w, const uint8_t* rec, const int32_t* chunk_off,
                        double* scores) {
  const int64_t rec_bytes = (int64_t)D + 4;
  double* k = (double*)malloc(sizeof(double) * (size_t)D);
  for (int32_t b = 0; b < B; ++b) {
    for (int64_t n = chunk_off[b]; n < chunk_off[b + 1]; ++n) {
      const uint8_t* r = rec + n * rec_bytes;
      float cf;
      memcpy(&cf, r + D, sizeof cf);
      for (int32_t d = 0; d < D; ++d) k[d] = oracle_fp8_e4m3(r[d]);
      double x = 0.0;
      for (int32_t h = 0; h < Hs; ++h) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d)
          dot += elem(q, ((int64_t)b * Hs + h) * D + d, dtype) * k[d];
        double a = (double)cf * dot;
        if (a < 0.0) a = 0.0;
        x += (double)w[(int64_t)b * Hs + h] * a;
      }
      scores[n] = x;
    }
  }
  free(k);
}

int32_t oracle_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_score_fp8mh_layers(int32_t L, int32_t combine, int32_t B, int32_t Hs, int32_t D,
                               int32_t dtype, const void* q, const float* w, const uint8_t* rec,
                               const int32_t* chunk_off, double* scores) {
  const int64_t total = chunk_off[B];
  const size_t esize = dtype == ORACLE_BF16 ? 2 : 4;
  double* x = (double*)malloc(sizeof(double) * (size_t)(total > 0 ? total : 1));
  for (int32_t l = 0; l < L; ++l) {
    const char* ql = (const char*)q + (size_t)l * (size_t)B * (size_t)Hs * (size_t)D * esize;
    const float* wl = w + (int64_t)l * B * Hs;
    const uint8_t* rl = rec + (int64_t)l * total * ((int64_t)D + 4);
    oracle_score_fp8mh(B, Hs, D, dtype, ql, wl, rl, chunk_off, x);
    for (int64_t n = 0; n < total; ++n) {
      if (l == 0) scores[n] = x[n];
      else if (combine == ORACLE_COMBINE_MAX) scores[n] = x[n] > scores[n] ? x[n] : scores[n];
      else scores[n] += x[n];
    }
  }
  if (combine == ORACLE_COMBINE_MEAN)
    for (int64_t n = 0; n < total; ++n) scores[n] /= (double)L;
  free(x);
}

void oracle_select_threshold(int32_t B, const double* scores, const int32_t* chunk_off,
                             double tau, int32_t max_keep, int32_t* sel_off, int32_t* sel_idx,
                             int32_t* fallback) {
  sel_off[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = chunk_off[b + 1] - chunk_off[b];
    const double* s = scores + chunk_off[b];
    int32_t* out = sel_idx + sel_off[b];
    int32_t kept = 0;
    for (int32_t i = 0; i < n; ++i)
      if (s[i] >= tau) out[kept++] = i;
    fallback[b] = (kept == 0 && n > 0) ? 1 : 0;
    if (fallback[b]) {
      for (int32_t i = 0; i < n; ++i) out[i] = i;
      kept = n;
    } else if (max_keep > 0 && kept > max_keep) {
      ranked* r = (ranked*)malloc(sizeof(ranked) * (size_t)kept);
      for (int32_t i = 0; i < kept; ++i) {
        r[i].s = s[out[i]];
        r[i].n = out[i];
      }
      qsort(r, (size_t)kept, sizeof(ranked), rank_cmp);
      for (int32_t i = 0; i < max_keep; ++i) out[i] = r[i].n;
      qsort(out, (size_t)max_keep, sizeof(int32_t), int_cmp);
      free(r);
      kept = max_keep;
    }
    sel_off[b + 1] = sel_off[b] + kept;
  }
}

void oracle_pool_delta(int32_t B, const int32_t* chunk_off, const int32_t* sel_idx,
                       const int32_t* sel_off, const int32_t* table_in, int32_t* table_out,
                       int32_t* loads, int32_t* load_count) {
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = chunk_off[b + 1] - chunk_off[b];
    const int32_t s0 = sel_off[b], k = sel_off[b + 1] - sel_off[b];
    unsigned char* wanted = (unsigned char*)calloc((size_t)(n > 0 ? n : 1), 1);
    unsigned char* held = (unsigned char*)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int32_t j = 0; j < k; ++j) wanted[sel_idx[s0 + j]] = 1;
    /* slots keeping a still-wanted chunk; every other slot is free */
    int32_t n_free = 0;
    int32_t* free_slots = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
    for (int32_t p = 0; p < k; ++p) {
      const int32_t c = table_in[s0 + p];
      if (c >= 0 && c < n && wanted[c] && !held[c]) {
        held[c] = 1;
        table_out[s0 + p] = c;
      } else {
        free_slots[n_free++] = s0 + p;
      }
    }
    /* newly kept chunks, ascending, into the free slots, ascending */
    int32_t n_load = 0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t c = sel_idx[s0 + j];
      if (held[c]) continue;
      const int32_t slot = free_slots[n_load];
      table_out[slot] = c;
      loads[s0 + n_load] = slot;
      ++n_load;
    }
    for (int32_t i = n_load; i < n_free; ++i) table_out[free_slots[i]] = -1;
    load_count[b] = n_load;
    free(free_slots);
    free(held);
    free(wanted);
  }
}

void oracle_keep_recent(int32_t B, int32_t C, const int64_t* seq_len, const int32_t* chunk_off,
                        const int32_t* sel_idx, const int32_t* sel_off, int32_t max_recent,
                        int32_t* out_idx, int32_t* out_off) {
  out_off[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t m = chunk_off[b + 1] - chunk_off[b];
    const int32_t k = sel_off[b + 1] - sel_off[b];
    const int64_t len = seq_len[b];
    const int32_t total = (int32_t)((len + C - 1) / C);
    int32_t* out = out_idx + out_off[b];
    int32_t n = 0;
    int32_t last_kept = 0;
    for (int32_t i = 0; i < k; ++i) {
      out[n++] = sel_idx[sel_off[b] + i];
      if (sel_idx[sel_off[b] + i] == m - 1) last_kept = 1;
    }
    /* the chunks beyond the kept ones, oldest first: the last scored chunk
     * (unless kept), then every unscored chunk; when there are more than
     * max_recent of them the newest max_recent are the ones attended, since
     * they hold the tokens written most recently, the current one included */
    int32_t first = (m > 0 && !last_kept) ? m - 1 : m;
    if (total - first > max_recent) first = total - max_recent;
    for (int32_t c = first; c < total; ++c) out[n++] = c;
    out_off[b + 1] = out_off[b] + n;
  }
}
