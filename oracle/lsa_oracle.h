/*
 * lsa_oracle.h -- CPU oracle for the Lookahead Sparse Attention (LSA) decode
 * hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or helper with the HIP
 * library, and it never reads anything the HIP library wrote except where a
 * test deliberately hands it the GPU's own fp32 scores to rank.
 *
 * Everything is plain C99, accumulates in double precision and follows the
 * method's definitions directly, with no blocking, splitting or fusion:
 *
 *   score      -- dual-encoder relevance: one inner product between a stream's
 *                 indexer query embedding and each of its chunk embeddings
 *                 (the bayesiansapien wiki note on FlashMemory-DeepSeek-V4
 *                 LSA, its flowchart and its "Key points"; dimensionstp review
 *                 section 3-2-4; arXiv abstract v2).
 *   select     -- keep the k highest-scoring chunks of each stream (review
 *                 section 3-2-3, step 5, the top-k keep mask).
 *   gather     -- copy the kept chunks into a resident pool (wiki note
 *                 flowchart, its resident-chunk node; molayo explainer, the
 *                 paragraph on gathering only the selected chunks).
 *   attention  -- softmax attention of each query head restricted to the
 *                 tokens of the kept chunks (review section 3-2-3, steps 6-7).
 *   score_fp8mh -- the released retriever's multi-head scorer over float8
 *                 compressed-key chunk records (review sections 3-2-1, 3-2-2
 *                 and 4-3).
 *
 * Element encodings: ORACLE_F32 arrays hold IEEE-754 binary32 values;
 * ORACLE_BF16 arrays hold bfloat16 bit patterns (the upper 16 bits of a
 * binary32), which are widened exactly.
 */
#ifndef LSA_ORACLE_H
#define LSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Number of chunks kept out of n_chunks at keep ratio num/den: floor or
 * ceiling of n_chunks*num/den in exact integer arithmetic, clamped to
 * [1, n_chunks].  Returns 0 for n_chunks <= 0 or a bad ratio. */
int32_t oracle_keep_count(int32_t n_chunks, int32_t num, int32_t den, int32_t round_up);

/* scores[chunk_off[b] + n] = sum_j q[b][j] * emb[chunk_off[b] + n][j]
 * q: [B][D], emb: [chunk_off[B]][D], both of element type dtype. */
void oracle_score(int32_t B, int32_t D, int32_t dtype, const void* q, const void* emb,
                  const int32_t* chunk_off, double* scores);

/* For each stream b keep k_b = sel_off[b+1]-sel_off[b] chunks: rank the
 * stream's chunks by (score descending, chunk index ascending) with NaN
 * ranked below every number, keep the first k_b and write their indices in
 * ascending order to sel_idx[sel_off[b] ...].  Returns 0, or -1 when some
 * k_b is outside [0, N_b]. */
int32_t oracle_select(int32_t B, const double* scores, const int32_t* chunk_off,
                      const int32_t* sel_off, int32_t* sel_idx);

/* Byte copy of the kept chunks into a pool: slot sel_off[b]+j receives the
 * rows of chunk sel_idx[sel_off[b]+j] of stream b (row r of the slot is token
 * n*C + r); rows at or beyond the stream's length are written as zeros.
 * row_bytes is the size of one token row of the store. */
void oracle_gather(int32_t B, int32_t C, int64_t row_bytes, const void* store,
                   const int64_t* tok_off, const int32_t* sel_idx, const int32_t* sel_off,
                   void* pool);

/* Sparse decode attention, two passes per (stream, head), no splitting.
 * Q: [B][H][dqk].  K rows: K[tok_off[b] + t][0..dqk).  V rows: if
 * v_aliases_k, V[t][c] = K[t][c] for c < dv, else V[tok_off[b]+t][0..dv).
 * Tokens taken: every t in [n*C, min(n*C+C, L_b)) for each kept chunk n of
 * stream b, L_b = tok_off[b+1]-tok_off[b].
 *   x_t = scale * <Q[b][h], K_t>,  m = max x_t,  w_t = exp(x_t - m),
 *   out[b][h][:] = sum_t w_t V_t / sum_t w_t,  lse[b][h] = m + log(sum_t w_t).
 * A stream with no token gets out = 0 and lse = -inf.
 * nthreads > 1 spreads (stream, head) pairs over OpenMP threads; the
 * arithmetic of each pair does not depend on it. */
void oracle_attention(int32_t B, int32_t H, int32_t dqk, int32_t dv, int32_t v_aliases_k,
                      int32_t dtype, int32_t C, double scale, const void* Q, const void* K,
                      const void* V, const int64_t* tok_off, const int32_t* sel_idx,
                      const int32_t* sel_off, double* out, double* lse, int32_t nthreads);

/* Value of one float8 e4m3 code (the OCP E4M3 encoding with no infinities:
 * sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes
 * m * 2^-9; the all-ones exponent and mantissa encode NaN), exactly. */
double oracle_fp8_e4m3(uint8_t code);

/* Multi-head relevance of compressed-key chunk records (dimensionstp review,
 * section 3-2-1 record table and section 3-2-2 scorer; section 4-3 shapes).
 * Record n of the table, rec_bytes = D + 4 bytes: D float8 e4m3 key values
 * k[0..D) followed by a little-endian float32 dequantisation scale c.  For
 * stream b and each of its chunks:
 *   x = sum_h w[b][h] * max(0, c * sum_d q[b][h][d] * k[d])
 * q: [B][Hs][D] of element type dtype; w: [B][Hs] float32.  The sigmoid of
 * the pages' formula is monotone and is not applied: x is the ranking score. */
void oracle_score_fp8mh(int32_t B, int32_t Hs, int32_t D, int32_t dtype, const void* q,
                        const float* w, const uint8_t* rec, const int32_t* chunk_off,
                        double* scores);

/* Multi-layer ensemble of the multi-head scorer (dimensionstp review,
 * section 3-2-2: the released retriever scores chunks in several CSA layers,
 * each with its own weights, and combines the per-layer scores by max or
 * mean).  Layer l has its own q [B][Hs][D], w [B][Hs] and record table
 * [total][D + 4], stored layer after layer (q, w and rec point at layer 0).
 * combine ORACLE_COMBINE_MAX: x = max_l x_l; ORACLE_COMBINE_MEAN: x = (sum_l
 * x_l) / L, each x_l as oracle_score_fp8mh computes it. */
#define ORACLE_COMBINE_MAX 0
#define ORACLE_COMBINE_MEAN 1
void oracle_score_fp8mh_layers(int32_t L, int32_t combine, int32_t B, int32_t Hs, int32_t D,
                               int32_t dtype, const void* q, const float* w, const uint8_t* rec,
                               const int32_t* chunk_off, double* scores);

/* Threshold keep mask with a dense fallback (dimensionstp review, section
 * 3-2-3 step 5: the keep mask comes from a top-k or a threshold; sections 4-3
 * and 5-1: exact-retrieval tasks need a threshold fallback).  Per stream b:
 *   pass_b = { n : scores[n] >= tau }            (NaN never passes)
 *   if pass_b is empty: keep every chunk of the stream, fallback[b] = 1
 *   else if max_keep > 0 and |pass_b| > max_keep: keep the max_keep chunks of
 *        pass_b ranked first by (score descending, index ascending)
 *   else keep pass_b; fallback[b] = 0.
 * Kept indices are written ascending to sel_idx[sel_off[b] ..), with sel_off
 * [B+1] the running totals of the kept counts (sel_off[0] = 0); sel_idx needs
 * room for chunk_off[B] entries. */
void oracle_select_threshold(int32_t B, const double* scores, const int32_t* chunk_off,
                             double tau, int32_t max_keep, int32_t* sel_off, int32_t* sel_idx,
                             int32_t* fallback);

/* Delta residency of the chunk pool (wiki note flowchart: only the selected
 * chunks stay on the GPU, the rest live in host memory and are swapped in
 * when needed; dimensionstp review section 3-2-5: that offload engine is
 * unreleased, so the rule below is the plainest one that fits).  Stream b
 * owns the k_b pool slots sel_off[b] .. sel_off[b+1]-1; table[slot] is the
 * chunk a slot holds (-1: none).  Given the new kept set sel_idx (ascending,
 * k_b chunks per stream) and the old table:
 *   a slot whose chunk is still kept keeps it (no copy);
 *   the other slots are free; the new chunks not held by any slot are loaded,
 *   the i-th of them (ascending chunk index) into the i-th free slot
 *   (ascending slot index); free slots left over hold -1.
 * Writes the new table to table_out, the slots loaded to loads[sel_off[b] ..
 * sel_off[b] + load_count[b]) in load order, and their number to load_count. */
void oracle_pool_delta(int32_t B, const int32_t* chunk_off, const int32_t* sel_idx,
                       const int32_t* sel_off, const int32_t* table_in, int32_t* table_out,
                       int32_t* loads, int32_t* load_count);

/* Attention keep set of a growing context (dimensionstp review section
 * 3-2-3 steps 2 and 7: history goes to the cache and decode attends to the
 * kept chunks; the pages say nothing of tokens added after the last
 * re-index, so this is the plainest rule that fits): the chunks of the last
 * selection (ascending, all below M_b = chunk_off[b+1]-chunk_off[b], the
 * chunks the indexer has scored), plus the last scored chunk M_b-1 when it
 * was not kept (it was the partial tail when scored and may have grown
 * since), plus every chunk from M_b to ceil(seq_len[b]/C)-1 (not yet
 * scored).  At most max_recent chunks beyond the kept ones per stream: when
 * there are more, the newest max_recent of them (the highest indices, which
 * hold the most recent tokens).  Writes the ascending union to
 * out_idx[out_off[b] ..] with out_off[B+1] its running totals. */
void oracle_keep_recent(int32_t B, int32_t C, const int64_t* seq_len, const int32_t* chunk_off,
                        const int32_t* sel_idx, const int32_t* sel_off, int32_t max_recent,
                        int32_t* out_idx, int32_t* out_off);

/* Threads an OpenMP region may use here (1 when built without OpenMP). */
int32_t oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
