/*
 * lsa.h -- C ABI of the Lookahead Sparse Attention (LSA) decode hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("FlashMemory-DeepSeek-V4: Lightning Index Ultra-Long Context via
 * Lookahead Sparse Attention"): for each decode stream a neural memory indexer
 * scores every historical KV chunk, only the highest-scoring chunks stay
 * resident, and attention runs over those chunks alone.  The pages describe
 * the decode loop in the dimensionstp review, section 3-2-3 ("Lookahead Sparse
 * Attention", steps 1-7): dense prefill, the K/V history kept as chunks, the
 * retriever re-scoring all chunks every ~64 decode steps, a top-k or threshold
 * keep mask, and sparse attention over the kept chunks until the next
 * re-scoring.  This library implements steps 4-7 on the GPU.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer.  Pointers named *_dev are device
 *   (HBM) pointers; the lsa_shape / lsa_step_args structs themselves are read
 *   on the host during the call and may be freed when it returns.  The library
 *   never allocates device or host memory and is reentrant; scratch memory is
 *   the caller's workspace, except for lsa_decode_step_static, whose scratch
 *   is a static device array.
 * Asynchrony: a call validates its arguments on the host, enqueues kernels on
 *   `hip_stream` (a hipStream_t; NULL means the legacy null stream) and
 *   returns.  Results are valid once the stream reaches that point.  No call
 *   synchronises or copies device data to the host.
 * Errors: every precondition the host can check is checked before anything
 *   is enqueued; on failure the call returns a non-zero lsa_status, enqueues
 *   nothing and leaves every output untouched.  Launch failures are reported
 *   as LSA_ERR_HIP (the thread's pending HIP error is cleared on entry).
 *   Device-side preconditions (offset tables monotone and consistent with the
 *   stated totals, 1 <= k_b <= N_b, kept indices in [0, N_b)) cannot be checked
 *   without reading device memory; kernels clamp so that a violation never
 *   writes outside the documented output ranges, but results are then
 *   unspecified.  lsa_check_tables checks them on the device (a debug aid,
 *   not called by any other entry point).
 * Layout: all tensors are dense row-major.  Ragged per-stream data is packed
 *   back to back and described by CSR offset arrays of B+1 entries whose first
 *   entry is 0:
 *     tok_off[B+1]   int64  tokens: stream b owns rows [tok_off[b], tok_off[b+1])
 *                           of the K/V history; L_b = tok_off[b+1]-tok_off[b].
 *     chunk_off[B+1] int32  chunks: N_b = chunk_off[b+1]-chunk_off[b] must equal
 *                           ceil(L_b / C).  Chunk n of stream b covers tokens
 *                           [n*C, min(n*C+C, L_b)); the last one may be partial.
 *     sel_off[B+1]   int32  kept chunks: k_b = sel_off[b+1]-sel_off[b].
 * Element types: LSA_DTYPE_F32 (IEEE binary32) or LSA_DTYPE_BF16 (bfloat16);
 *   one dtype covers q_idx, chunk embeddings, Q, K and V.  Scores, outputs and
 *   log-sum-exps are always fp32; arithmetic accumulates in fp32.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lsa_status;
#define LSA_OK 0
#define LSA_ERR_INVALID_ARGUMENT 1
#define LSA_ERR_UNSUPPORTED 2
#define LSA_ERR_WORKSPACE_TOO_SMALL 3
#define LSA_ERR_HIP 4

enum { LSA_DTYPE_F32 = 0, LSA_DTYPE_BF16 = 1 };
enum { LSA_KV_STORE = 0, LSA_KV_POOL = 1 };

/* Problem shape.  Every field is read on the host. */
typedef struct lsa_shape {
  int32_t batch;          /* B >= 1 decode streams */
  int32_t chunk_size;     /* C tokens per chunk, 1..1024 */
  int32_t index_dim;      /* D, indexer embedding width */
  int32_t num_q_heads;    /* H query heads, all sharing one KV head */
  int32_t head_dim_qk;    /* key / query width */
  int32_t head_dim_v;     /* value / output width */
  int32_t v_aliases_k;    /* 1: V rows are the first head_dim_v columns of the
                             K rows (absorbed multi-head latent attention);
                             0: V is its own [sum L, head_dim_v] tensor */
  int32_t dtype;          /* LSA_DTYPE_* */
  float softmax_scale;    /* logits = softmax_scale * <q_h, k_t> */
  int32_t max_chunks;     /* >= max_b N_b */
  int32_t max_k;          /* >= max_b k_b */
  int64_t total_chunks;   /* = sum_b N_b = chunk_off[B] */
  int64_t total_k;        /* = sum_b k_b = sel_off[B] */
  int32_t attn_tiles_per_block; /* split-KV granularity: 32-token tiles handled
                             by one attention workgroup (values above
                             1022 * ceil(chunk_size / 32) act as that bound);
                             0 picks a default for the shape.  Changing it
                             changes results only by
                             rounding (bf16 inputs: the attention weights are
                             rounded to bf16 relative to each split's running
                             maximum, about 2^-9 relative). */
  int32_t flags;          /* 0, or LSA_SHAPE_UNIFORM */
} lsa_shape;

/* lsa_shape.flags: every stream has exactly max_chunks chunks and keeps
 * exactly max_k of them, so chunk_off[b] = b * max_chunks and
 * sel_off[b] = b * max_k (checked on the host against total_chunks and
 * total_k; the offset arrays are still passed and must hold these values).
 * The kernels then derive those offsets instead of reading them, which takes
 * one dependent memory round trip out of the score, select, gather,
 * attention and merge launches.  Leave it 0 for ragged batches and for keep
 * sets whose sizes are known on the device only (lsa_select_threshold,
 * lsa_keep_recent), whose shapes carry bounds. */
#define LSA_SHAPE_UNIFORM 1

/* Human-readable name of a status code (static storage). */
const char* lsa_status_string(lsa_status status);

/* Version of this ABI (incremented on incompatible change). */
int32_t lsa_abi_version(void);

/* Kept chunks out of n_chunks at keep ratio ratio_num/ratio_den: the floor
 * (round_up = 0) or ceiling (round_up = 1) of n_chunks*ratio_num/ratio_den in
 * exact integer arithmetic, clamped to [1, n_chunks].  The wiki note and the
 * abstract quote an average footprint of 13.5% of the full context and more
 * than 90% reduction at 500K tokens; those are keep ratios of this form.
 * Returns 0 when n_chunks <= 0 or the ratio is not positive. */
int32_t lsa_keep_count(int32_t n_chunks, int32_t ratio_num, int32_t ratio_den,
                       int32_t round_up);

/* Bytes of workspace lsa_sparse_decode_attn / lsa_decode_step need for this
 * shape (0 if the shape is invalid).  Monotone in batch, total_k, max_k,
 * num_q_heads and head_dim_v; any buffer at least this large works.  The
 * buffer must be zero-filled once before its first use (it holds one arrival
 * counter per stream); every call leaves it zero-filled again, so a workspace
 * is zeroed once when allocated, not per call. */
size_t lsa_workspace_bytes(const lsa_shape* shape);

/* How lsa_sparse_decode_attn / lsa_decode_step would run attention for this
 * shape on the current device (a description for measurement and
 * diagnostics; nothing is enqueued).  Wiki note "Key points": the cost of
 * decode is the KV traffic; this names the kernel that streams it and
 * whether its split-KV partials are merged by a separate launch. */
enum { LSA_ATTN_KERNEL_MQA = 0, LSA_ATTN_KERNEL_MLA = 1, LSA_ATTN_KERNEL_VECTOR = 2 };
typedef struct {
  int64_t grid;             /* workgroups of the attention launch (an upper bound
                               of the ones that do work) */
  int64_t partial_rows;     /* split-KV partial results the workspace holds */
  int32_t kernel;           /* LSA_ATTN_KERNEL_* */
  int32_t tiles_per_chunk;  /* 32-token tiles per chunk */
  int32_t merge_in_kernel;  /* 1: each stream's last workgroup merges its
                               partials (no merge launch); 0: a merge launch */
  int32_t split_heads;      /* 1: the vector-ALU kernel's split-heads form */
  int32_t select_in_kernel; /* 1: a re-indexing lsa_decode_step over the store
                               ranks the kept chunks inside the attention
                               kernel (no select launch) */
  int32_t reserved;         /* 0 */
} lsa_attn_plan_info;

/* Fills *info; LSA_ERR_INVALID_ARGUMENT for a null pointer or a shape
 * lsa_sparse_decode_attn would refuse, LSA_ERR_UNSUPPORTED for an
 * unsupported one (then *info is untouched). */
lsa_status lsa_attention_plan(const lsa_shape* shape, lsa_attn_plan_info* info);

/* ---------------------------------------------------------------------------
 * Chunk scoring (dual-encoder relevance).  Wiki note flowchart and "Key
 * points"; dimensionstp review sections 2-1 and 3-2-4; abstract v2: the
 * indexer is a standard dual encoder, so a chunk's relevance is the inner
 * product of the stream's query embedding with the chunk's embedding.
 *   scores_dev[chunk_off[b] + n] = sum_j q_idx[b][j] * emb[chunk_off[b] + n][j]
 * q_idx_dev: [B][D]; emb_dev: [total_chunks][D]; scores_dev: [total_chunks] fp32.
 * No normalisation and no sigmoid are applied (inputs are expected to be
 * normalised already; a monotone squashing never changes a top-k).
 * Supported when a row of D elements is 16-byte vectors in a power-of-two
 * count from 4 to 128 (bf16: D = 32, 64, ..., 1024; fp32: D = 16, 32, ..., 512);
 * other D return LSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
lsa_status lsa_score(const lsa_shape* shape, const void* q_idx_dev, const void* emb_dev,
                     const int32_t* chunk_off_dev, float* scores_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Multi-head relevance of float8 compressed-key chunk records.  Dimensionstp
 * review, section 3-2-1 (the compressed-key record: head_dim float8 e4m3 key
 * values followed by a float32 per-chunk dequantisation scale, 132 bytes for
 * head_dim 128), section 3-2-2 (the released retriever's scorer) and section
 * 4-3 (128 heads of dimension 128).  For stream b and each of its chunks:
 *   scores_dev[chunk_off[b] + n] =
 *       sum_h head_w[b][h] * max(0, scale_n * sum_d q_heads[b][h][d] * k_n[d])
 * where k_n[d] is the d-th float8 e4m3 value of record chunk_off[b] + n (the
 * OCP E4M3 encoding: no infinities, 0x7f / 0xff are NaN) and scale_n its
 * float32 scale (little-endian).  The sigmoid of the pages' formula is
 * monotone and is not applied; the result ranks chunks for lsa_select_topk.
 * q_heads_dev: [B][num_heads][head_dim] bf16 (shape->dtype must be bf16),
 * 16-byte aligned; head_w_dev: [B][num_heads] fp32; records_dev:
 * [total_chunks][head_dim + 4] bytes, 4-byte aligned; scores_dev:
 * [total_chunks] fp32.  Only batch, chunk_size, max_chunks and the totals of
 * the shape are used.  Supported: head_dim 64 or 128 and num_heads 16, 32, 64
 * or 128 (LSA_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------- */
lsa_status lsa_score_fp8_multihead(const lsa_shape* shape, int32_t num_heads, int32_t head_dim,
                                   const void* q_heads_dev, const float* head_w_dev,
                                   const void* records_dev, const int32_t* chunk_off_dev,
                                   float* scores_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Layer ensemble of the multi-head scorer.  Dimensionstp review, section
 * 3-2-2: the released retriever scores chunks in several CSA layers, each
 * with its own weights and compressed keys, and combines the per-layer scores
 * by max (close to a union of the layers' choices) or by mean.  Layer l's
 * score x_l is what lsa_score_fp8_multihead computes from layer l's inputs:
 *   combine LSA_COMBINE_MAX:  scores_dev[i] = max_l x_l[i]
 *   combine LSA_COMBINE_MEAN: scores_dev[i] = (x_0[i] + ... + x_{L-1}[i]) / L
 *                             (fp32 sum in layer order, then one division)
 * The inputs are stored layer after layer: q_heads_dev
 * [num_layers][B][num_heads][head_dim] bf16, head_w_dev
 * [num_layers][B][num_heads] fp32, records_dev
 * [num_layers][total_chunks][head_dim + 4] bytes; alignment, shapes and
 * support as for lsa_score_fp8_multihead.  1 <= num_layers <= 16, else
 * LSA_ERR_INVALID_ARGUMENT; a combine other than the two above is
 * LSA_ERR_INVALID_ARGUMENT.  With num_layers = 1 the result equals
 * lsa_score_fp8_multihead's bit for bit.  All layers are read in one pass.
 * ------------------------------------------------------------------------- */
enum { LSA_COMBINE_MAX = 0, LSA_COMBINE_MEAN = 1 };

lsa_status lsa_score_fp8_multihead_layers(const lsa_shape* shape, int32_t num_layers,
                                          int32_t combine, int32_t num_heads, int32_t head_dim,
                                          const void* q_heads_dev, const float* head_w_dev,
                                          const void* records_dev, const int32_t* chunk_off_dev,
                                          float* scores_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Top-k keep set.  Dimensionstp review section 3-2-3 step 5 (top-k keep
 * mask).  For each stream, keeps the k_b chunks ranked first by (score
 * descending, chunk index ascending); NaN ranks below every number and -0.0
 * equals +0.0.  Writes their chunk indices (0-based within the stream) in
 * ascending order to sel_idx_dev[sel_off[b] .. sel_off[b+1]).
 * scores_dev: [total_chunks] fp32; sel_idx_dev: [total_k] int32.
 * Requires max_chunks <= 65536.  The result is a deterministic function of the
 * fp32 scores (bit-identical across runs).
 * ------------------------------------------------------------------------- */
lsa_status lsa_select_topk(const lsa_shape* shape, const float* scores_dev,
                           const int32_t* chunk_off_dev, const int32_t* sel_off_dev,
                           int32_t* sel_idx_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Threshold keep set with a dense fallback.  Dimensionstp review section
 * 3-2-3 step 5 (the keep mask comes from a top-k or from a threshold);
 * sections 4-3 and 5-1 (exact-retrieval tasks need a threshold fallback).
 * For each stream b:
 *   pass_b = { n : scores[chunk_off[b] + n] >= threshold }  (fp32 compare;
 *            NaN never passes, -0.0 == +0.0)
 *   pass_b empty (and N_b > 0): keep all N_b chunks -- dense attention for
 *            that stream -- and set fallback_dev[b] = 1;
 *   otherwise, when max_keep > 0 and |pass_b| > max_keep: keep the max_keep
 *            chunks of pass_b ranked first by (score descending, index
 *            ascending), as lsa_select_topk would; else keep pass_b;
 *            fallback_dev[b] = 0.
 * Writes the kept counts' running totals to sel_off_dev[0 .. B] (sel_off[0]
 * = 0; a CSR table lsa_sparse_decode_attn and lsa_gather_chunks accept) and
 * the kept indices, ascending within each stream, to sel_idx_dev
 * [sel_off[b] .. sel_off[b+1]).  sel_idx_dev must hold total_chunks int32
 * (every chunk may be kept); fallback_dev [B] int32 may be NULL.  Calls that
 * consume this keep set take a shape whose total_k / max_k are the bounds
 * total_chunks / max_chunks, since the counts are known on the device only.
 * workspace_dev: at least lsa_select_threshold_workspace_bytes(shape) bytes,
 * 256-byte aligned (else LSA_ERR_WORKSPACE_TOO_SMALL / INVALID_ARGUMENT);
 * threshold must not be NaN and max_keep must be >= 0 (else
 * LSA_ERR_INVALID_ARGUMENT).  Requires max_chunks <= 65536.  Two kernels:
 * the per-stream counts, then the offsets and the indices.
 * ------------------------------------------------------------------------- */
size_t lsa_select_threshold_workspace_bytes(const lsa_shape* shape);

lsa_status lsa_select_threshold(const lsa_shape* shape, const float* scores_dev,
                                const int32_t* chunk_off_dev, float threshold, int32_t max_keep,
                                int32_t* sel_off_dev, int32_t* sel_idx_dev, int32_t* fallback_dev,
                                void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Resident chunk pool.  Wiki note flowchart (its resident-chunk node); molayo
 * explainer (gather the chunks a query needs instead of sweeping the whole
 * cache).  Copies each kept chunk into
 * its pool slot: slot s = sel_off[b] + j receives chunk n = sel_idx[s] of
 * stream b, row r of the slot being token n*C + r; rows with n*C + r >= L_b
 * are zero-filled.
 * k_store_dev: [sum L][head_dim_qk]; k_pool_dev: [total_k][C][head_dim_qk].
 * v_store_dev / v_pool_dev: [sum L][head_dim_v] / [total_k][C][head_dim_v];
 * both must be NULL when v_aliases_k (the K pool then carries V too).
 * A bit-exact copy.
 * ------------------------------------------------------------------------- */
lsa_status lsa_gather_chunks(const lsa_shape* shape, const void* k_store_dev,
                             const void* v_store_dev, const int64_t* tok_off_dev,
                             const int32_t* sel_idx_dev, const int32_t* sel_off_dev,
                             void* k_pool_dev, void* v_pool_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Decode-time growth of the context.  Dimensionstp review section 3-2-3,
 * steps 2 and 7: new history goes to the cache and decode attends to the
 * kept chunks.  The stores use a capacity layout: stream b owns rows
 * base_off[b] .. base_off[b+1]-1 (int64 [B+1], base_off[0] = 0) of which the
 * first seq_len[b] (int64 [B], device) hold tokens.
 * lsa_append_kv: writes k_new[b] ([B][head_dim_qk]) and v_new[b]
 *   ([B][head_dim_v]; NULL when v_aliases_k) as row seq_len[b] of stream b
 *   and increments seq_len[b]; a stream whose rows are all used is left
 *   unchanged.  Rows must be multiples of 16 bytes (else UNSUPPORTED); all
 *   pointers 16-byte aligned (offsets 8).
 * lsa_keep_recent: the keep set attention needs once the context grew after
 *   the last re-index (the pages are silent on those tokens; this library's
 *   reading): per stream, the kept chunks sel_idx (ascending, all below M_b =
 *   chunk_off[b+1]-chunk_off[b], the chunks the indexer scored), then the
 *   last scored chunk M_b-1 unless kept (it was the partial tail when scored
 *   and may have grown since), then every chunk from M_b to
 *   ceil(seq_len[b]/C)-1; at most max_recent chunks beyond the kept ones,
 *   the newest max_recent when more qualify (so the chunk holding the
 *   latest token is always attended when max_recent >= 1).
 *   Writes the ascending union to out_sel_idx_dev (room for total_k +
 *   B*max_recent) and its CSR offsets to out_sel_off_dev [B+1], computed on
 *   the device.  Attention over it takes a shape whose total_k / max_k are
 *   the bounds total_k + B*max_recent / max_k + max_recent and whose chunk
 *   bounds cover the capacity.
 * lsa_sparse_decode_attn_varlen: lsa_sparse_decode_attn over the capacity
 *   layout: rows of stream b start at base_off[b] and L_b = seq_len[b]
 *   (clamped to the capacity).  Same kernels, same workspace.
 * ------------------------------------------------------------------------- */
lsa_status lsa_append_kv(const lsa_shape* shape, const void* k_new_dev, const void* v_new_dev,
                         const int64_t* base_off_dev, int64_t* seq_len_dev, void* k_store_dev,
                         void* v_store_dev, void* hip_stream);

lsa_status lsa_keep_recent(const lsa_shape* shape, const int64_t* seq_len_dev,
                           const int32_t* chunk_off_dev, const int32_t* sel_idx_dev,
                           const int32_t* sel_off_dev, int32_t max_recent,
                           int32_t* out_sel_idx_dev, int32_t* out_sel_off_dev, void* hip_stream);

lsa_status lsa_sparse_decode_attn_varlen(const lsa_shape* shape, int32_t kv_mode,
                                         const void* q_dev, const void* k_base_dev,
                                         const void* v_base_dev, const int64_t* base_off_dev,
                                         const int64_t* seq_len_dev, const int32_t* sel_idx_dev,
                                         const int32_t* sel_off_dev, float* out_dev,
                                         float* lse_dev, void* workspace_dev,
                                         size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Delta residency of the chunk pool over a host-memory backing store.  Wiki
 * note flowchart: only the selected chunks stay resident on the GPU, the rest
 * of the cache lives in host memory and chunks are swapped in as the
 * selection changes (dimensionstp review section 3-2-5: that engine is
 * unreleased; the slot rule below is this library's).  Stream b owns pool
 * slots sel_off[b] .. sel_off[b+1]-1 and table_dev[slot] names the chunk a
 * slot holds (-1: none; start from all -1).  Given the new kept set
 * sel_idx_dev (ascending, k_b chunks per stream, as lsa_select_topk writes):
 *   a slot whose chunk is still kept keeps it and is not copied;
 *   the other slots are freed; the newly kept chunks, in ascending order, are
 *   copied from the host store into the freed slots, in ascending slot order
 *   (rows past the end of the stream zero-filled); freed slots left over
 *   hold -1.
 * Outputs: table_dev [total_k] (updated in place), loads_dev [total_k] (the
 * slots written, stream b's in loads[sel_off[b] .. sel_off[b] +
 * load_count[b])), load_count_dev [B].  k_pool_dev / v_pool_dev as for
 * lsa_gather_chunks, except that slot s holds chunk table[s]: attention then
 * reads the pool with kv_mode LSA_KV_POOL and sel_idx = table (any order of a
 * stream's chunks gives the same result up to rounding).
 * k_host / v_host: the K and V history [sum L][head_dim] in page-locked host
 * memory (hipHostMalloc or a pinned torch tensor), 16-byte aligned; v_host
 * NULL when v_aliases_k.  Memory that is not page-locked host memory is
 * LSA_ERR_INVALID_ARGUMENT (checked with hipPointerGetAttributes).  Rows must
 * be multiples of 16 bytes and max_chunks <= 65536 (else LSA_ERR_UNSUPPORTED).
 * Preconditions on the device: k_b is the same as when the table was written,
 * and a stream's table entries are distinct.  Two kernels; only the loaded
 * chunks cross the host link.
 * ------------------------------------------------------------------------- */
lsa_status lsa_pool_delta_update(const lsa_shape* shape, const void* k_host, const void* v_host,
                                 const int64_t* tok_off_dev, const int32_t* chunk_off_dev,
                                 const int32_t* sel_idx_dev, const int32_t* sel_off_dev,
                                 int32_t* table_dev, int32_t* loads_dev, int32_t* load_count_dev,
                                 void* k_pool_dev, void* v_pool_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Sparse decode attention over the kept chunks.  Dimensionstp review section
 * 3-2-3 steps 6-7: unselected chunks are masked out and attention runs over
 * the kept ones.  For every stream b and head h, over the tokens t of the
 * kept chunks (t < L_b):
 *   x_t = softmax_scale * <q[b][h], K_t>
 *   out[b][h][:] = sum_t exp(x_t) V_t / sum_t exp(x_t)
 *   lse[b][h]    = log(sum_t exp(x_t))          (natural log)
 * computed split-KV: workgroups own runs of 32-token tiles, keep an fp32
 * online softmax, and their partial (max, sum, output) results are combined
 * by log-sum-exp (by the last workgroup of each stream to finish, or by a
 * merge pass).  For absorbed latent attention the partial output rows are
 * stored rounded to bf16 (at most 2^-9 relative per element); the maxima,
 * the sums and the combination stay fp32.
 * q_dev: [B][H][head_dim_qk].  kv_mode LSA_KV_STORE: k_base/v_base are the
 * stores ([sum L][d]) and chunk sel_idx[s] of stream b is read in place.
 * kv_mode LSA_KV_POOL: k_base/v_base are pools written by lsa_gather_chunks
 * and slot s is read (sel_idx is still needed for the valid-token count of
 * partial chunks).  A stream's kept indices may come in any order (the
 * select writes them ascending): the order changes only how the sums are
 * split and rounded.  v_base must be NULL when v_aliases_k.
 * out_dev: [B][H][head_dim_v] fp32; lse_dev: [B][H] fp32 (may be NULL).
 * workspace_dev: >= lsa_workspace_bytes(shape) bytes, 256-byte aligned,
 * zero-filled before its first use (see lsa_workspace_bytes); it holds the
 * split partial results and the per-stream arrival counters of the kernels
 * that merge a stream in its last workgroup (the multi-query and vector-ALU
 * kernels, for shapes whose streams have few workgroups; otherwise, and for
 * absorbed latent attention, a separate merge pass runs); calls that share a
 * workspace must not run concurrently.
 * Supported: bf16 with num_q_heads <= 64 and head_dim_qk == head_dim_v in
 * {64, 128} (multi-query); bf16 with head_dim_qk 576, head_dim_v 512,
 * v_aliases_k = 1 and 1 to 64 query heads (absorbed latent attention); fp32
 * or bf16 with num_q_heads <= 16 and head dims <= 256 (portable kernel).
 * Anything else returns LSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
lsa_status lsa_sparse_decode_attn(const lsa_shape* shape, int32_t kv_mode, const void* q_dev,
                                  const void* k_base_dev, const void* v_base_dev,
                                  const int64_t* tok_off_dev, const int32_t* sel_idx_dev,
                                  const int32_t* sel_off_dev, float* out_dev, float* lse_dev,
                                  void* workspace_dev, size_t workspace_bytes,
                                  void* hip_stream);

/* ---------------------------------------------------------------------------
 * One decode step of the whole path in one call: on a re-index step, score ->
 * select (-> gather into the pool when materialize_pool); then sparse
 * attention (from the pool when materialize_pool, else in place from the
 * store).  On other steps the previous sel_idx (and pool) are reused.  This is
 * the lookahead schedule of the review (section 3-2-3 steps 4-7; section 3-1
 * table and section 4-3: re-score about every 64 decode steps): with
 * reindex_every = R > 0 the call re-indexes exactly when step % R == 0
 * (lsa_reindex_due) and `reindex` is ignored; with reindex_every = 0 the
 * caller decides through `reindex` (non-zero: re-index).  A re-index step
 * scores q_idx_dev as it is at that step, so a caller whose indexer query
 * changes every step passes the current one.  Every phase is one grid over
 * all streams; nothing returns to the host between phases.  Over the store,
 * the multi-query kernel and the vector-ALU kernel on short inputs rank each
 * stream's kept chunks in their own prologue (same keys, rule and algorithm
 * as lsa_select_topk, so the same sel_idx, which the stream's first
 * workgroup writes) instead of a select launch; lsa_attention_plan reports
 * which.
 * reindex_every < 0, or step < 0 with reindex_every > 0, is
 * LSA_ERR_INVALID_ARGUMENT.
 * ev_attn_begin / ev_attn_end: optional hipEvent_t recorded on hip_stream
 * right before and right after the split-KV attention kernel (the merge pass
 * runs after ev_attn_end; NULL to skip), so a caller can time that kernel
 * inside the step.
 * ------------------------------------------------------------------------- */
typedef struct lsa_step_args {
  const void* q_idx_dev;        /* [B][D] indexer query embeddings */
  const void* emb_dev;          /* [total_chunks][D] chunk embeddings */
  const int32_t* chunk_off_dev; /* [B+1] */
  float* scores_dev;            /* [total_chunks] fp32, written when reindex */
  const int32_t* sel_off_dev;   /* [B+1] */
  int32_t* sel_idx_dev;         /* [total_k], written when reindex, else read */
  const void* q_dev;            /* [B][H][head_dim_qk] decode queries */
  const void* k_store_dev;      /* [sum L][head_dim_qk] */
  const void* v_store_dev;      /* [sum L][head_dim_v], NULL when v_aliases_k */
  const int64_t* tok_off_dev;   /* [B+1] */
  void* k_pool_dev;             /* [total_k][C][head_dim_qk] when materialize_pool */
  void* v_pool_dev;             /* [total_k][C][head_dim_v] when materialize_pool
                                   and not v_aliases_k, else NULL */
  float* out_dev;               /* [B][H][head_dim_v] fp32 */
  float* lse_dev;               /* [B][H] fp32 or NULL */
  int32_t reindex;              /* non-zero: re-score and re-select this step */
  int32_t materialize_pool;     /* non-zero: gather kept chunks into the pool */
  void* ev_attn_begin;          /* hipEvent_t or NULL */
  void* ev_attn_end;            /* hipEvent_t or NULL */
  int32_t reindex_every;        /* R > 0: re-index iff step % R == 0; 0: use `reindex` */
  int32_t reserved;             /* 0 */
  int64_t step;                 /* decode step number, counted from 0 */
} lsa_step_args;

/* 1 when decode step `step` re-scores and re-selects under re-index interval
 * reindex_every (step % reindex_every == 0), else 0; -1 for reindex_every < 1
 * or step < 0.  The schedule lsa_decode_step applies when its args carry
 * reindex_every > 0. */
int32_t lsa_reindex_due(int64_t step, int32_t reindex_every);

lsa_status lsa_decode_step(const lsa_shape* shape, const lsa_step_args* args,
                           void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * lsa_decode_step without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, kernels and
 * results as lsa_decode_step; the split-KV partials go to a static device
 * array of LSA_STATIC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends.  A shape whose lsa_workspace_bytes
 * exceeds that size returns LSA_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued.  The call allocates nothing.  All calls on one device share that
 * device's array: calls that overlap on one device (concurrent streams, or
 * host threads) race and must be serialised by the caller.  The first call
 * on a device looks up the array's device address (LSA_ERR_HIP if that
 * fails) and enqueues, ahead of its step, a fill kernel that zeroes the
 * array's per-stream arrival counters (a kernel, not a memset, so that the
 * call can be captured in a graph); every step leaves them at zero.
 * ------------------------------------------------------------------------- */
#define LSA_STATIC_SCRATCH_BYTES (64u << 20)

lsa_status lsa_decode_step_static(const lsa_shape* shape, const lsa_step_args* args,
                                  void* hip_stream);

/* ---------------------------------------------------------------------------
 * Debug check of the device-side preconditions (off the hot path; nothing
 * else calls it).  The kernels read the offset tables and kept indices
 * without checking them; a caller that wants a bad table reported instead of
 * silently wrong results runs this first.  For every stream b it checks:
 *   LSA_TABLE_ERR_CHUNK_OFF  chunk_off[0] == 0, chunk_off[B] == total_chunks,
 *                            0 <= chunk_off[b] <= chunk_off[b+1] <= total_chunks,
 *                            N_b <= max_chunks (and chunk_off[b] = b * max_chunks
 *                            for a LSA_SHAPE_UNIFORM shape);
 *   LSA_TABLE_ERR_SEL_OFF    the same of sel_off against total_k and max_k;
 *   LSA_TABLE_ERR_KEEP       1 <= k_b <= N_b;
 *   LSA_TABLE_ERR_TOK_OFF    tok_off[0] == 0, tok_off non-decreasing and
 *                            N_b == ceil(L_b / C) (skipped when tok_off_dev is
 *                            NULL);
 *   LSA_TABLE_ERR_SEL_IDX    every kept index in [0, N_b), and strictly
 *                            ascending within a stream when kept_ascending is
 *                            non-zero (lsa_select_topk's output; a pool table
 *                            of lsa_pool_delta_update is not ascending)
 *                            (skipped when sel_idx_dev is NULL).
 * *error_flags_dev (one int32 in device memory) receives the OR of the bits
 * of every stream: 0 when every precondition holds.  Only entries inside the
 * documented array sizes are read (sel_idx only where sel_off's range lies
 * in [0, total_k]).  Two kernels: one clears the flag, one checks.
 * ------------------------------------------------------------------------- */
#define LSA_TABLE_ERR_CHUNK_OFF 1
#define LSA_TABLE_ERR_SEL_OFF 2
#define LSA_TABLE_ERR_KEEP 4
#define LSA_TABLE_ERR_TOK_OFF 8
#define LSA_TABLE_ERR_SEL_IDX 16

lsa_status lsa_check_tables(const lsa_shape* shape, const int64_t* tok_off_dev,
                            const int32_t* chunk_off_dev, const int32_t* sel_off_dev,
                            const int32_t* sel_idx_dev, int32_t kept_ascending,
                            int32_t* error_flags_dev, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not part of the method).
 * lsa_bench_copy: streaming device copy of `bytes` (a multiple of 16, both
 *   pointers 16-byte aligned); the reference kernel against which HBM counters
 *   and achievable bandwidth are calibrated.
 * lsa_bench_read: reads `bytes` of a device buffer without writing it (the
 *   reference for the HBM read counters): pattern 0 plain 16-byte loads,
 *   each wave instruction covering 1 KiB of consecutive bytes; 1 the same
 *   with the non-temporal hint; 2 the multi-query attention kernel's K
 *   operand pattern (256-byte rows in blocks of 16, one instruction covering
 *   64 bytes of each of 16 rows, non-temporal).  bytes: a multiple of 16
 *   (4096 for pattern 2).  sink_dev: one uint32 per thread of the launch,
 *   LSA_BENCH_READ_SINK_BYTES bytes (else LSA_ERR_WORKSPACE_TOO_SMALL).
 * lsa_bench_flush: overwrites `bytes` of a caller buffer (multiple of 16) so
 *   that caches hold none of a workload's data afterwards.
 * lsa_bench_attention_partial: enqueues only the split-KV partial kernel of
 *   lsa_sparse_decode_attn (same arguments and checks, no outputs: the
 *   partial results land in the workspace and are not merged), so that the
 *   kernel can be timed back to back without anything recorded between
 *   launches.
 * ------------------------------------------------------------------------- */
lsa_status lsa_bench_copy(void* dst_dev, const void* src_dev, size_t bytes, void* hip_stream);
#define LSA_BENCH_READ_SINK_BYTES (256u * 32u * 256u * 4u)
lsa_status lsa_bench_read(const void* src_dev, size_t bytes, int32_t pattern, void* sink_dev,
                          size_t sink_bytes, void* hip_stream);
lsa_status lsa_bench_flush(void* buf_dev, size_t bytes, void* hip_stream);
lsa_status lsa_bench_attention_partial(const lsa_shape* shape, int32_t kv_mode, const void* q_dev,
                                       const void* k_base_dev, const void* v_base_dev,
                                       const int64_t* tok_off_dev, const int32_t* sel_idx_dev,
                                       const int32_t* sel_off_dev, void* workspace_dev,
                                       size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
