// capi.hip -- the extern "C" entry points of lsa.h: host-side validation of
// every argument, workspace sizing, and kernel enqueueing on the caller's
// stream.  No entry point allocates, synchronises or reads device memory.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int32_t kMaxChunkSize = 1024;
constexpr int32_t kMaxChunksPerStream = 65536;
constexpr int32_t kMaxScoreLayers = 16;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t elem_bytes(const lsa_shape& s) { return s.dtype == LSA_DTYPE_BF16 ? 2 : 4; }

// Checks shared by every entry point: batch, chunking and the CSR totals.
lsa_status check_common(const lsa_shape* s) {
  if (s == nullptr) return LSA_ERR_INVALID_ARGUMENT;
  if (s->batch < 1 || s->chunk_size < 1 || s->chunk_size > kMaxChunkSize) return LSA_ERR_INVALID_ARGUMENT;
  if (s->dtype != LSA_DTYPE_F32 && s->dtype != LSA_DTYPE_BF16) return LSA_ERR_INVALID_ARGUMENT;
  if ((s->flags & ~LSA_SHAPE_UNIFORM) != 0 || s->attn_tiles_per_block < 0)
    return LSA_ERR_INVALID_ARGUMENT;
  if (s->max_chunks < 1 || s->max_k < 1 || s->max_k > s->max_chunks) return LSA_ERR_INVALID_ARGUMENT;
  if (s->total_chunks < s->batch || s->total_chunks > static_cast<int64_t>(s->batch) * s->max_chunks ||
      s->total_chunks > INT32_MAX)
    return LSA_ERR_INVALID_ARGUMENT;
  if (s->total_k < s->batch || s->total_k > static_cast<int64_t>(s->batch) * s->max_k ||
      s->total_k > s->total_chunks)
    return LSA_ERR_INVALID_ARGUMENT;
  if ((s->flags & LSA_SHAPE_UNIFORM) &&
      (s->total_chunks != static_cast<int64_t>(s->batch) * s->max_chunks ||
       s->total_k != static_cast<int64_t>(s->batch) * s->max_k))
    return LSA_ERR_INVALID_ARGUMENT;
  return LSA_OK;
}

lsa_status check_score(const lsa_shape* s) {
  lsa_status st = check_common(s);
  if (st != LSA_OK) return st;
  if (s->index_dim < 1) return LSA_ERR_INVALID_ARGUMENT;
  if (!score_supported(*s)) return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

lsa_status check_select(const lsa_shape* s) {
  lsa_status st = check_common(s);
  if (st != LSA_OK) return st;
  if (s->max_chunks > kMaxChunksPerStream) return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

lsa_status check_attn_shape(const lsa_shape* s) {
  lsa_status st = check_common(s);
  if (st != LSA_OK) return st;
  if (s->num_q_heads < 1 || s->head_dim_qk < 1 || s->head_dim_v < 1) return LSA_ERR_INVALID_ARGUMENT;
  if (s->v_aliases_k != 0 && s->v_aliases_k != 1) return LSA_ERR_INVALID_ARGUMENT;
  if (s->v_aliases_k && s->head_dim_v > s->head_dim_qk) return LSA_ERR_INVALID_ARGUMENT;
  if (!(s->softmax_scale > 0.f) || !isfinite(s->softmax_scale)) return LSA_ERR_INVALID_ARGUMENT;
  if ((s->head_dim_qk * elem_bytes(*s)) % 16 != 0 || (s->head_dim_v * elem_bytes(*s)) % 16 != 0)
    return LSA_ERR_UNSUPPORTED;
  if (!mqa_attn_supported(*s) && !mla_attn_supported(*s) && !portable_attn_supported(*s))
    return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

lsa_status hip_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_ERR_HIP; }

// Enqueue the attention partial kernel and the merge; arguments validated.
// ev_begin / ev_end (may be null) bracket the partial kernel.
// Whether the attention kernel merges each stream's partials in the stream's
// last workgroup (no merge launch): the multi-query and vector-ALU kernels
// can, when streams average at most eight workgroups (so a last workgroup
// reads few partials) and its threads hold the output row in one pass
// (H * dv <= 8 * threads, dv a multiple of 8); otherwise the merge launch
// reads the partials with many workgroups in parallel.  Measured: 32 ragged
// streams (eight workgroups each on average) 82.1 -> 79.2 us per step fused,
// their merges overlapping other streams' tiles; 16 x 128K (sixteen each,
// all streams ending together) 42.9 -> 45.2 us fused, so that shape keeps
// the merge launch.
bool fuse_merge_in_kernel(const lsa_shape& s, const AttnPlan& plan) {
  if (mla_attn_supported(s) || s.batch > kCounterStreams || s.head_dim_v % 8 != 0) return false;
  int32_t threads = 256;
  if (!mqa_attn_supported(s)) {  // vector-ALU kernel: four waves up to 256-byte rows, else two
    const int32_t es = s.dtype == LSA_DTYPE_BF16 ? 2 : 4;
    const int32_t rb = (s.head_dim_qk > s.head_dim_v ? s.head_dim_qk : s.head_dim_v) * es;
    threads = rb <= 256 ? 256 : 128;
  }
  if (s.num_q_heads * s.head_dim_v > 8 * threads) return false;
  const int64_t wgs_expected =
      plan.per > 0 ? (s.total_k * plan.tiles_per_chunk + plan.per - 1) / plan.per : plan.target;
  // the split-heads form has one tile per workgroup and small partials: its
  // last workgroup merges up to 32 per stream on average
  const int64_t per_stream = plan.split_heads ? 32 : 8;
  return wgs_expected <= per_stream * static_cast<int64_t>(s.batch);
}

// Whether a re-indexing decode step over the store ranks the kept chunks in
// the attention kernel's prologue (no select launch, no kept-index round
// trip): the multi-query kernel and the split-heads vector-ALU kernel can.
bool select_in_attention_kernel(const lsa_shape& s, const AttnPlan& plan) {
  if (mla_attn_supported(s)) return false;
  return mqa_attn_supported(s) ? mqa_select_in_kernel_supported(s)
                               : portable_select_in_kernel_supported(s, plan);
}

// The split-KV plan of a validated attention shape on the current device and
// the workspace layout it implies (computed once per call).
struct AttnSetup {
  AttnPlan plan;
  PartialLayout layout;
};

AttnSetup attn_setup(const lsa_shape& s) {
  AttnSetup x;
  x.plan = make_attn_plan(s, device_cu_count());
  x.layout = partial_layout(s, x.plan);
  return x;
}

lsa_status enqueue_attention(const lsa_shape& s, const AttnSetup& setup, int32_t kv_mode,
                             const void* q, const void* kbase, const void* vbase,
                             const int64_t* tok_off, const int32_t* sel_idx,
                             const int32_t* sel_off, float* out, float* lse, void* ws,
                             hipStream_t st, void* ev_begin = nullptr, void* ev_end = nullptr,
                             const int64_t* seq_len = nullptr, bool partial_only = false,
                             const float* sel_scores = nullptr,
                             const int32_t* chunk_off = nullptr) {
  const AttnPlan& plan = setup.plan;
  const PartialLayout& pl = setup.layout;
  AttnArgs a;
  // sel_scores non-null: the attention kernel ranks the kept chunks itself and
  // writes them to sel_idx (which it then does not read)
  a.sel_scores = sel_scores;
  a.chunk_off = chunk_off;
  a.sel_idx_out = const_cast<int32_t*>(sel_idx);
  a.uni_n = (s.flags & LSA_SHAPE_UNIFORM) ? s.max_chunks : 0;
  a.q = q;
  a.k = kbase;
  a.v = s.v_aliases_k ? kbase : vbase;
  a.tok_off = tok_off;
  a.seq_len = seq_len;
  a.sel_idx = sel_idx;
  a.sel_off = sel_off;
  a.out = out;
  a.lse = lse;
  a.ws_m = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.m_off);
  a.ws_l = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.l_off);
  a.ws_o = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.o_off);
  a.o_bf16 = partial_o_bf16(s) ? 1 : 0;
  a.counters = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.cnt_off);
  // in-kernel merge, or the merge launch after the partial kernel
  const bool fused = !partial_only && fuse_merge_in_kernel(s, plan);
  a.fuse_merge = fused ? 1 : 0;
  a.B = s.batch;
  a.H = s.num_q_heads;
  a.dqk = s.head_dim_qk;
  a.dv = s.head_dim_v;
  a.C = s.chunk_size;
  a.k_row = s.head_dim_qk;
  a.v_row = s.v_aliases_k ? s.head_dim_qk : s.head_dim_v;
  a.pool = kv_mode == LSA_KV_POOL ? 1 : 0;
  a.tiles_per_chunk = plan.tiles_per_chunk;
  a.per = plan.per;
  a.target = plan.target;
  a.uni_k = (s.flags & LSA_SHAPE_UNIFORM) ? s.max_k : 0;
  a.uni_wgs = 0;
  a.uni_per = 1;
  if (a.uni_k > 0) {  // the split every stream of a uniform batch takes
    const int32_t t = s.max_k * plan.tiles_per_chunk;
    const int32_t total = static_cast<int32_t>(s.total_k) * plan.tiles_per_chunk;
    const StreamSplit sp =
        split_of_tiles(t, plan.tiles_per_chunk, plan.per, plan.target, total,
                       uniform_balanced_run(s.batch, t, plan.per, plan.target));
    a.uni_wgs = sp.wgs;
    a.uni_per = sp.per;
  }
  a.split_heads = plan.split_heads;
  a.scale_log2 = s.softmax_scale * 1.4426950408889634f;
  if (ev_begin && hipEventRecord(static_cast<hipEvent_t>(ev_begin), st) != hipSuccess)
    return LSA_ERR_HIP;
  hipError_t e;
  if (mla_attn_supported(s)) e = launch_attn_mla(s, a, plan.grid, st);
  else if (mqa_attn_supported(s)) e = launch_attn_mqa(s, a, plan.grid, st);
  else e = launch_attn_portable(s, a, plan.grid, st);
  if (e != hipSuccess) return LSA_ERR_HIP;
  if (ev_end && hipEventRecord(static_cast<hipEvent_t>(ev_end), st) != hipSuccess)
    return LSA_ERR_HIP;
  if (partial_only || fused) return LSA_OK;
  return hip_status(launch_attn_merge(s, a, plan, st));
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" {

const char* lsa_status_string(lsa_status status) {
  switch (status) {
    case LSA_OK: return "LSA_OK";
    case LSA_ERR_INVALID_ARGUMENT: return "LSA_ERR_INVALID_ARGUMENT";
    case LSA_ERR_UNSUPPORTED: return "LSA_ERR_UNSUPPORTED";
    case LSA_ERR_WORKSPACE_TOO_SMALL: return "LSA_ERR_WORKSPACE_TOO_SMALL";
    case LSA_ERR_HIP: return "LSA_ERR_HIP";
    default: return "LSA_ERR_UNKNOWN";
  }
}

int32_t lsa_abi_version(void) { return 4; }

int32_t lsa_reindex_due(int64_t step, int32_t reindex_every) {
  if (reindex_every < 1 || step < 0) return -1;
  return step % reindex_every == 0 ? 1 : 0;
}

int32_t lsa_keep_count(int32_t n_chunks, int32_t ratio_num, int32_t ratio_den, int32_t round_up) {
  if (n_chunks <= 0 || ratio_num <= 0 || ratio_den <= 0) return 0;
  const int64_t prod = static_cast<int64_t>(n_chunks) * ratio_num;
  int64_t k = round_up ? (prod + ratio_den - 1) / ratio_den : prod / ratio_den;
  if (k < 1) k = 1;
  if (k > n_chunks) k = n_chunks;
  return static_cast<int32_t>(k);
}

size_t lsa_workspace_bytes(const lsa_shape* shape) {
  if (check_attn_shape(shape) != LSA_OK) return 0;
  return partial_layout(*shape, make_attn_plan(*shape, device_cu_count())).total;
}

lsa_status lsa_attention_plan(const lsa_shape* shape, lsa_attn_plan_info* info) {
  if (info == nullptr) return LSA_ERR_INVALID_ARGUMENT;
  const lsa_status st = check_attn_shape(shape);
  if (st != LSA_OK) return st;
  const lsa_shape& s = *shape;
  const AttnPlan plan = make_attn_plan(s, device_cu_count());
  lsa_attn_plan_info r;
  r.grid = plan.grid;
  r.partial_rows = plan.ws_rows;
  r.kernel = mla_attn_supported(s)   ? LSA_ATTN_KERNEL_MLA
             : mqa_attn_supported(s) ? LSA_ATTN_KERNEL_MQA
                                     : LSA_ATTN_KERNEL_VECTOR;
  r.tiles_per_chunk = plan.tiles_per_chunk;
  r.merge_in_kernel = fuse_merge_in_kernel(s, plan) ? 1 : 0;
  r.split_heads = plan.split_heads;
  r.select_in_kernel = select_in_attention_kernel(s, plan) ? 1 : 0;
  r.reserved = 0;
  *info = r;
  return LSA_OK;
}

lsa_status lsa_score(const lsa_shape* shape, const void* q_idx_dev, const void* emb_dev,
                     const int32_t* chunk_off_dev, float* scores_dev, void* hip_stream) {
  lsa_status st = check_score(shape);
  if (st != LSA_OK) return st;
  if (!q_idx_dev || !emb_dev || !chunk_off_dev || !scores_dev) return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(q_idx_dev, 16) || !aligned(emb_dev, 16) || !aligned(chunk_off_dev, 4) ||
      !aligned(scores_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_score(*shape, q_idx_dev, emb_dev, chunk_off_dev, scores_dev,
                                 static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_score_fp8_multihead_layers(const lsa_shape* shape, int32_t num_layers,
                                          int32_t combine, int32_t num_heads, int32_t head_dim,
                                          const void* q_heads_dev, const float* head_w_dev,
                                          const void* records_dev, const int32_t* chunk_off_dev,
                                          float* scores_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  if (num_layers < 1 || num_layers > kMaxScoreLayers) return LSA_ERR_INVALID_ARGUMENT;
  if (combine != LSA_COMBINE_MAX && combine != LSA_COMBINE_MEAN) return LSA_ERR_INVALID_ARGUMENT;
  if (num_heads < 1 || head_dim < 1) return LSA_ERR_INVALID_ARGUMENT;
  if (shape->dtype != LSA_DTYPE_BF16 || !score_mh_supported(num_heads, head_dim))
    return LSA_ERR_UNSUPPORTED;
  if (!q_heads_dev || !head_w_dev || !records_dev || !chunk_off_dev || !scores_dev)
    return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(q_heads_dev, 16) || !aligned(head_w_dev, 4) || !aligned(records_dev, 4) ||
      !aligned(chunk_off_dev, 4) || !aligned(scores_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_score_mh(*shape, num_layers, combine, num_heads, head_dim, q_heads_dev,
                                    head_w_dev, records_dev, chunk_off_dev, scores_dev,
                                    static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_score_fp8_multihead(const lsa_shape* shape, int32_t num_heads, int32_t head_dim,
                                   const void* q_heads_dev, const float* head_w_dev,
                                   const void* records_dev, const int32_t* chunk_off_dev,
                                   float* scores_dev, void* hip_stream) {
  return lsa_score_fp8_multihead_layers(shape, 1, LSA_COMBINE_MAX, num_heads, head_dim,
                                        q_heads_dev, head_w_dev, records_dev, chunk_off_dev,
                                        scores_dev, hip_stream);
}

size_t lsa_select_threshold_workspace_bytes(const lsa_shape* shape) {
  if (check_select(shape) != LSA_OK) return 0;
  return align256(static_cast<size_t>(shape->batch) * sizeof(int32_t));
}

lsa_status lsa_select_threshold(const lsa_shape* shape, const float* scores_dev,
                                const int32_t* chunk_off_dev, float threshold, int32_t max_keep,
                                int32_t* sel_off_dev, int32_t* sel_idx_dev, int32_t* fallback_dev,
                                void* workspace_dev, size_t workspace_bytes, void* hip_stream) {
  lsa_status st = check_select(shape);
  if (st != LSA_OK) return st;
  if (isnan(threshold) || max_keep < 0) return LSA_ERR_INVALID_ARGUMENT;
  if (!scores_dev || !chunk_off_dev || !sel_off_dev || !sel_idx_dev || !workspace_dev)
    return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(scores_dev, 4) || !aligned(chunk_off_dev, 4) || !aligned(sel_off_dev, 4) ||
      !aligned(sel_idx_dev, 4) || (fallback_dev && !aligned(fallback_dev, 4)) ||
      !aligned(workspace_dev, 256))
    return LSA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < lsa_select_threshold_workspace_bytes(shape))
    return LSA_ERR_WORKSPACE_TOO_SMALL;
  (void)hipGetLastError();
  return hip_status(launch_select_threshold(*shape, scores_dev, chunk_off_dev, threshold, max_keep,
                                            sel_off_dev, sel_idx_dev, fallback_dev,
                                            static_cast<int32_t*>(workspace_dev),
                                            static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_select_topk(const lsa_shape* shape, const float* scores_dev,
                           const int32_t* chunk_off_dev, const int32_t* sel_off_dev,
                           int32_t* sel_idx_dev, void* hip_stream) {
  lsa_status st = check_select(shape);
  if (st != LSA_OK) return st;
  if (!scores_dev || !chunk_off_dev || !sel_off_dev || !sel_idx_dev) return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(scores_dev, 4) || !aligned(chunk_off_dev, 4) || !aligned(sel_off_dev, 4) ||
      !aligned(sel_idx_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_select(*shape, scores_dev, chunk_off_dev, sel_off_dev, sel_idx_dev,
                                  static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_gather_chunks(const lsa_shape* shape, const void* k_store_dev,
                             const void* v_store_dev, const int64_t* tok_off_dev,
                             const int32_t* sel_idx_dev, const int32_t* sel_off_dev,
                             void* k_pool_dev, void* v_pool_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  const lsa_shape& s = *shape;
  if (s.head_dim_qk < 1 || (s.v_aliases_k != 0 && s.v_aliases_k != 1)) return LSA_ERR_INVALID_ARGUMENT;
  if (!s.v_aliases_k && s.head_dim_v < 1) return LSA_ERR_INVALID_ARGUMENT;
  if (!k_store_dev || !tok_off_dev || !sel_idx_dev || !sel_off_dev || !k_pool_dev)
    return LSA_ERR_INVALID_ARGUMENT;
  if (s.v_aliases_k ? (v_store_dev || v_pool_dev) : (!v_store_dev || !v_pool_dev))
    return LSA_ERR_INVALID_ARGUMENT;
  const int32_t kb = s.head_dim_qk * elem_bytes(s);
  const int32_t vb = s.v_aliases_k ? 0 : s.head_dim_v * elem_bytes(s);
  if (kb % 16 != 0 || vb % 16 != 0) return LSA_ERR_UNSUPPORTED;
  if (!aligned(k_store_dev, 16) || !aligned(k_pool_dev, 16) ||
      (v_store_dev && (!aligned(v_store_dev, 16) || !aligned(v_pool_dev, 16))) ||
      !aligned(tok_off_dev, 8) || !aligned(sel_idx_dev, 4) || !aligned(sel_off_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_gather(s, k_store_dev, kb, tok_off_dev, sel_idx_dev, sel_off_dev,
                                  k_pool_dev, v_store_dev, vb, v_pool_dev,
                                  static_cast<hipStream_t>(hip_stream)));
}

// Checks of an attention call's arguments other than the workspace.
static lsa_status check_attn_io(const lsa_shape* shape, int32_t kv_mode, const void* q,
                                const void* kb, const void* vb, const int64_t* tok_off,
                                const int32_t* sel_idx, const int32_t* sel_off, const float* out,
                                const float* lse) {
  lsa_status st = check_attn_shape(shape);
  if (st != LSA_OK) return st;
  if (kv_mode != LSA_KV_STORE && kv_mode != LSA_KV_POOL) return LSA_ERR_INVALID_ARGUMENT;
  if (!q || !kb || !tok_off || !sel_idx || !sel_off || !out) return LSA_ERR_INVALID_ARGUMENT;
  if (shape->v_aliases_k ? (vb != nullptr) : (vb == nullptr)) return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kb, 16) || (vb && !aligned(vb, 16)) || !aligned(tok_off, 8) ||
      !aligned(sel_idx, 4) || !aligned(sel_off, 4) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return LSA_ERR_INVALID_ARGUMENT;
  return LSA_OK;
}

// Workspace of a validated attention call: present, 256-byte aligned, large enough.
static lsa_status check_workspace(const AttnSetup& setup, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned(ws, 256)) return LSA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < setup.layout.total) return LSA_ERR_WORKSPACE_TOO_SMALL;
  return LSA_OK;
}

// Checks of an attention call; on success *setup holds its plan and layout.
static lsa_status check_attn_args(const lsa_shape* shape, int32_t kv_mode, const void* q,
                                  const void* kb, const void* vb, const int64_t* tok_off,
                                  const int32_t* sel_idx, const int32_t* sel_off, const float* out,
                                  const float* lse, const void* ws, size_t ws_bytes,
                                  AttnSetup* setup) {
  const lsa_status st = check_attn_io(shape, kv_mode, q, kb, vb, tok_off, sel_idx, sel_off, out, lse);
  if (st != LSA_OK) return st;
  *setup = attn_setup(*shape);
  return check_workspace(*setup, ws, ws_bytes);
}

// Device address of page-locked host memory, or null when `p` is not such memory.
static const void* pinned_device_pointer(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost) return nullptr;
  return attr.devicePointer;
}

lsa_status lsa_pool_delta_update(const lsa_shape* shape, const void* k_host, const void* v_host,
                                 const int64_t* tok_off_dev, const int32_t* chunk_off_dev,
                                 const int32_t* sel_idx_dev, const int32_t* sel_off_dev,
                                 int32_t* table_dev, int32_t* loads_dev, int32_t* load_count_dev,
                                 void* k_pool_dev, void* v_pool_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  const lsa_shape& s = *shape;
  if (s.head_dim_qk < 1 || s.head_dim_v < 1 || (s.v_aliases_k != 0 && s.v_aliases_k != 1))
    return LSA_ERR_INVALID_ARGUMENT;
  if (s.max_chunks > pool_delta_max_stream_chunks()) return LSA_ERR_UNSUPPORTED;
  const int32_t kb = s.head_dim_qk * elem_bytes(s);
  const int32_t vb = s.v_aliases_k ? 0 : s.head_dim_v * elem_bytes(s);
  if (kb % 16 != 0 || vb % 16 != 0) return LSA_ERR_UNSUPPORTED;
  if (!k_host || !tok_off_dev || !chunk_off_dev || !sel_idx_dev || !sel_off_dev || !table_dev ||
      !loads_dev || !load_count_dev || !k_pool_dev)
    return LSA_ERR_INVALID_ARGUMENT;
  if (s.v_aliases_k ? (v_host != nullptr || v_pool_dev != nullptr)
                    : (v_host == nullptr || v_pool_dev == nullptr))
    return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_host, 16) || (v_host && !aligned(v_host, 16)) || !aligned(k_pool_dev, 16) ||
      (v_pool_dev && !aligned(v_pool_dev, 16)) || !aligned(tok_off_dev, 8) ||
      !aligned(chunk_off_dev, 4) || !aligned(sel_idx_dev, 4) || !aligned(sel_off_dev, 4) ||
      !aligned(table_dev, 4) || !aligned(loads_dev, 4) || !aligned(load_count_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  const void* k_dev = pinned_device_pointer(k_host);
  const void* v_dev = v_host ? pinned_device_pointer(v_host) : nullptr;
  if (!k_dev || (v_host && !v_dev)) return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_pool_delta(s, k_dev, kb, v_dev, vb, tok_off_dev, chunk_off_dev,
                                      sel_idx_dev, sel_off_dev, table_dev, loads_dev,
                                      load_count_dev, k_pool_dev, v_pool_dev,
                                      static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_sparse_decode_attn(const lsa_shape* shape, int32_t kv_mode, const void* q_dev,
                                  const void* k_base_dev, const void* v_base_dev,
                                  const int64_t* tok_off_dev, const int32_t* sel_idx_dev,
                                  const int32_t* sel_off_dev, float* out_dev, float* lse_dev,
                                  void* workspace_dev, size_t workspace_bytes, void* hip_stream) {
  AttnSetup setup;
  lsa_status st = check_attn_args(shape, kv_mode, q_dev, k_base_dev, v_base_dev, tok_off_dev,
                                  sel_idx_dev, sel_off_dev, out_dev, lse_dev, workspace_dev,
                                  workspace_bytes, &setup);
  if (st != LSA_OK) return st;
  (void)hipGetLastError();
  return enqueue_attention(*shape, setup, kv_mode, q_dev, k_base_dev, v_base_dev, tok_off_dev,
                           sel_idx_dev, sel_off_dev, out_dev, lse_dev, workspace_dev,
                           static_cast<hipStream_t>(hip_stream));
}

lsa_status lsa_sparse_decode_attn_varlen(const lsa_shape* shape, int32_t kv_mode,
                                         const void* q_dev, const void* k_base_dev,
                                         const void* v_base_dev, const int64_t* base_off_dev,
                                         const int64_t* seq_len_dev, const int32_t* sel_idx_dev,
                                         const int32_t* sel_off_dev, float* out_dev,
                                         float* lse_dev, void* workspace_dev,
                                         size_t workspace_bytes, void* hip_stream) {
  AttnSetup setup;
  lsa_status st = check_attn_args(shape, kv_mode, q_dev, k_base_dev, v_base_dev, base_off_dev,
                                  sel_idx_dev, sel_off_dev, out_dev, lse_dev, workspace_dev,
                                  workspace_bytes, &setup);
  if (st != LSA_OK) return st;
  if (!seq_len_dev || !aligned(seq_len_dev, 8)) return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return enqueue_attention(*shape, setup, kv_mode, q_dev, k_base_dev, v_base_dev, base_off_dev,
                           sel_idx_dev, sel_off_dev, out_dev, lse_dev, workspace_dev,
                           static_cast<hipStream_t>(hip_stream), nullptr, nullptr, seq_len_dev);
}

lsa_status lsa_append_kv(const lsa_shape* shape, const void* k_new_dev, const void* v_new_dev,
                         const int64_t* base_off_dev, int64_t* seq_len_dev, void* k_store_dev,
                         void* v_store_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  const lsa_shape& s = *shape;
  if (s.head_dim_qk < 1 || s.head_dim_v < 1 || (s.v_aliases_k != 0 && s.v_aliases_k != 1))
    return LSA_ERR_INVALID_ARGUMENT;
  const int32_t kb = s.head_dim_qk * elem_bytes(s);
  const int32_t vb = s.v_aliases_k ? 0 : s.head_dim_v * elem_bytes(s);
  if (kb % 16 != 0 || vb % 16 != 0) return LSA_ERR_UNSUPPORTED;
  if (!k_new_dev || !base_off_dev || !seq_len_dev || !k_store_dev) return LSA_ERR_INVALID_ARGUMENT;
  if (s.v_aliases_k ? (v_new_dev != nullptr || v_store_dev != nullptr)
                    : (v_new_dev == nullptr || v_store_dev == nullptr))
    return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new_dev, 16) || (v_new_dev && !aligned(v_new_dev, 16)) ||
      !aligned(k_store_dev, 16) || (v_store_dev && !aligned(v_store_dev, 16)) ||
      !aligned(base_off_dev, 8) || !aligned(seq_len_dev, 8))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_append_kv(s, k_new_dev, v_new_dev, kb, vb, base_off_dev, seq_len_dev,
                                     k_store_dev, v_store_dev,
                                     static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_keep_recent(const lsa_shape* shape, const int64_t* seq_len_dev,
                           const int32_t* chunk_off_dev, const int32_t* sel_idx_dev,
                           const int32_t* sel_off_dev, int32_t max_recent,
                           int32_t* out_sel_idx_dev, int32_t* out_sel_off_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  if (max_recent < 0) return LSA_ERR_INVALID_ARGUMENT;
  if (!seq_len_dev || !chunk_off_dev || !sel_idx_dev || !sel_off_dev || !out_sel_idx_dev ||
      !out_sel_off_dev)
    return LSA_ERR_INVALID_ARGUMENT;
  if (!aligned(seq_len_dev, 8) || !aligned(chunk_off_dev, 4) || !aligned(sel_idx_dev, 4) ||
      !aligned(sel_off_dev, 4) || !aligned(out_sel_idx_dev, 4) || !aligned(out_sel_off_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_keep_recent(*shape, seq_len_dev, chunk_off_dev, sel_idx_dev,
                                       sel_off_dev, max_recent, out_sel_idx_dev, out_sel_off_dev,
                                       static_cast<hipStream_t>(hip_stream)));
}

// Checks of a decode step's arguments other than the workspace (x.reindex
// already set by the schedule).
static lsa_status check_step(const lsa_shape* shape, const lsa_step_args& x) {
  const bool pool = x.materialize_pool != 0;
  const void* kbase = pool ? x.k_pool_dev : x.k_store_dev;
  const void* vbase = pool ? x.v_pool_dev : x.v_store_dev;
  lsa_status st = check_attn_io(shape, pool ? LSA_KV_POOL : LSA_KV_STORE, x.q_dev, kbase, vbase,
                                x.tok_off_dev, x.sel_idx_dev, x.sel_off_dev, x.out_dev, x.lse_dev);
  if (st != LSA_OK) return st;
  if (pool && (!x.k_store_dev || (shape->v_aliases_k ? x.v_store_dev != nullptr : !x.v_store_dev)))
    return LSA_ERR_INVALID_ARGUMENT;
  if (pool && (!aligned(x.k_store_dev, 16) || (x.v_store_dev && !aligned(x.v_store_dev, 16))))
    return LSA_ERR_INVALID_ARGUMENT;
  if (x.reindex) {
    st = check_score(shape);
    if (st != LSA_OK) return st;
    st = check_select(shape);
    if (st != LSA_OK) return st;
    if (!x.q_idx_dev || !x.emb_dev || !x.chunk_off_dev || !x.scores_dev)
      return LSA_ERR_INVALID_ARGUMENT;
    if (!aligned(x.q_idx_dev, 16) || !aligned(x.emb_dev, 16) || !aligned(x.chunk_off_dev, 4) ||
        !aligned(x.scores_dev, 4))
      return LSA_ERR_INVALID_ARGUMENT;
  }
  return LSA_OK;
}

// Enqueues a validated decode step with its split-KV partials in `ws`.
static lsa_status enqueue_step(const lsa_shape* shape, const AttnSetup& setup,
                               const lsa_step_args& x, void* ws, void* hip_stream) {
  const bool pool = x.materialize_pool != 0;
  const hipStream_t hs = static_cast<hipStream_t>(hip_stream);
  (void)hipGetLastError();
  const bool select_in_attention =
      x.reindex && !pool && select_in_attention_kernel(*shape, setup.plan);
  if (x.reindex) {
    if (launch_score(*shape, x.q_idx_dev, x.emb_dev, x.chunk_off_dev, x.scores_dev, hs) !=
        hipSuccess)
      return LSA_ERR_HIP;
    if (!select_in_attention &&
        launch_select(*shape, x.scores_dev, x.chunk_off_dev, x.sel_off_dev, x.sel_idx_dev, hs) !=
            hipSuccess)
      return LSA_ERR_HIP;
    if (pool) {
      const int32_t kb = shape->head_dim_qk * elem_bytes(*shape);
      const int32_t vb = shape->v_aliases_k ? 0 : shape->head_dim_v * elem_bytes(*shape);
      if (launch_gather(*shape, x.k_store_dev, kb, x.tok_off_dev, x.sel_idx_dev, x.sel_off_dev,
                        x.k_pool_dev, x.v_store_dev, vb, x.v_pool_dev, hs) != hipSuccess)
        return LSA_ERR_HIP;
    }
  }
  return enqueue_attention(*shape, setup, pool ? LSA_KV_POOL : LSA_KV_STORE, x.q_dev,
                           pool ? x.k_pool_dev : x.k_store_dev,
                           pool ? x.v_pool_dev : x.v_store_dev, x.tok_off_dev, x.sel_idx_dev,
                           x.sel_off_dev, x.out_dev, x.lse_dev, ws, hs, x.ev_attn_begin,
                           x.ev_attn_end, nullptr, false,
                           select_in_attention ? x.scores_dev : nullptr, x.chunk_off_dev);
}

// The step's arguments with the lookahead schedule applied to x.reindex.
static lsa_status resolve_schedule(const lsa_step_args* args, lsa_step_args* x) {
  if (args == nullptr) return LSA_ERR_INVALID_ARGUMENT;
  *x = *args;
  if (x->reindex_every < 0 || x->reserved != 0) return LSA_ERR_INVALID_ARGUMENT;
  if (x->reindex_every > 0) {
    const int32_t due = lsa_reindex_due(x->step, x->reindex_every);
    if (due < 0) return LSA_ERR_INVALID_ARGUMENT;
    x->reindex = due;
  }
  return LSA_OK;
}

lsa_status lsa_decode_step(const lsa_shape* shape, const lsa_step_args* args, void* workspace_dev,
                           size_t workspace_bytes, void* hip_stream) {
  if (shape == nullptr) return LSA_ERR_INVALID_ARGUMENT;
  lsa_step_args x;
  lsa_status st = resolve_schedule(args, &x);
  if (st != LSA_OK) return st;
  st = check_step(shape, x);
  if (st != LSA_OK) return st;
  const AttnSetup setup = attn_setup(*shape);
  st = check_workspace(setup, workspace_dev, workspace_bytes);
  if (st != LSA_OK) return st;
  return enqueue_step(shape, setup, x, workspace_dev, hip_stream);
}

// ---------------------------------------------------------------------------
// lsa_decode_step_static: lsa_decode_step for callers that cannot allocate.
// Its split-KV partials (the only scratch memory of a step) live in the
// file-scope device array below: each device holds its own copy, from when
// the library's code object is loaded on it until the process ends.  In host
// code `scratch` names a host-side stand-in, never a device address; the
// device address of each device's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address reaches
// the kernels.  Every call on a device shares its copy (overlapping calls on
// one device race).  Of its contents only the per-stream arrival counters
// (the first 64 KiB) must start at zero: the first call on each device
// clears them with a fill kernel on its stream, ahead of its step, and every
// attention launch leaves them at zero; every partial the merge reads is
// written first by the same step.
static __device__ __align__(256) unsigned char scratch[LSA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_dev[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
std::atomic<bool> g_scratch_cleared[kMaxScratchDevices];
}  // namespace

// Device address of the current device's copy of `scratch`, or null; *dev_out
// receives the device.
static void* static_scratch_address(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_dev[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *dev_out = dev;
  return g_scratch_dev[dev];
}

lsa_status lsa_decode_step_static(const lsa_shape* shape, const lsa_step_args* args,
                                  void* hip_stream) {
  if (shape == nullptr) return LSA_ERR_INVALID_ARGUMENT;
  lsa_step_args x;
  lsa_status st = resolve_schedule(args, &x);
  if (st != LSA_OK) return st;
  st = check_step(shape, x);
  if (st != LSA_OK) return st;
  const AttnSetup setup = attn_setup(*shape);
  if (setup.layout.total > LSA_STATIC_SCRATCH_BYTES) return LSA_ERR_WORKSPACE_TOO_SMALL;
  int dev = -1;
  void* ws = static_scratch_address(&dev);
  if (ws == nullptr) {
    (void)hipGetLastError();
    return LSA_ERR_HIP;
  }
  if (!g_scratch_cleared[dev].load(std::memory_order_acquire)) {
    (void)hipGetLastError();
    if (launch_clear_counters(ws, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
      return LSA_ERR_HIP;
    g_scratch_cleared[dev].store(true, std::memory_order_release);
  }
  return enqueue_step(shape, setup, x, ws, hip_stream);
}

lsa_status lsa_check_tables(const lsa_shape* shape, const int64_t* tok_off_dev,
                            const int32_t* chunk_off_dev, const int32_t* sel_off_dev,
                            const int32_t* sel_idx_dev, int32_t kept_ascending,
                            int32_t* error_flags_dev, void* hip_stream) {
  lsa_status st = check_common(shape);
  if (st != LSA_OK) return st;
  if (!chunk_off_dev || !sel_off_dev || !error_flags_dev) return LSA_ERR_INVALID_ARGUMENT;
  if ((tok_off_dev && !aligned(tok_off_dev, 8)) || !aligned(chunk_off_dev, 4) ||
      !aligned(sel_off_dev, 4) || (sel_idx_dev && !aligned(sel_idx_dev, 4)) ||
      !aligned(error_flags_dev, 4))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_check_tables(*shape, tok_off_dev, chunk_off_dev, sel_off_dev,
                                        sel_idx_dev, kept_ascending, error_flags_dev,
                                        static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_bench_attention_partial(const lsa_shape* shape, int32_t kv_mode, const void* q_dev,
                                       const void* k_base_dev, const void* v_base_dev,
                                       const int64_t* tok_off_dev, const int32_t* sel_idx_dev,
                                       const int32_t* sel_off_dev, void* workspace_dev,
                                       size_t workspace_bytes, void* hip_stream) {
  // the checks of lsa_sparse_decode_attn, with the workspace standing in for
  // the outputs it does not write
  AttnSetup setup;
  lsa_status st = check_attn_args(shape, kv_mode, q_dev, k_base_dev, v_base_dev, tok_off_dev,
                                  sel_idx_dev, sel_off_dev, static_cast<const float*>(workspace_dev),
                                  nullptr, workspace_dev, workspace_bytes, &setup);
  if (st != LSA_OK) return st;
  (void)hipGetLastError();
  return enqueue_attention(*shape, setup, kv_mode, q_dev, k_base_dev, v_base_dev, tok_off_dev,
                           sel_idx_dev, sel_off_dev, nullptr, nullptr, workspace_dev,
                           static_cast<hipStream_t>(hip_stream), nullptr, nullptr, nullptr, true);
}

lsa_status lsa_bench_copy(void* dst_dev, const void* src_dev, size_t bytes, void* hip_stream) {
  if (!dst_dev || !src_dev || bytes % 16 != 0 || !aligned(dst_dev, 16) || !aligned(src_dev, 16))
    return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_bench_copy(dst_dev, src_dev, bytes, static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_bench_read(const void* src_dev, size_t bytes, int32_t pattern, void* sink_dev,
                          size_t sink_bytes, void* hip_stream) {
  if (!src_dev || !sink_dev || !aligned(src_dev, 16) || !aligned(sink_dev, 4) ||
      pattern < 0 || pattern > 2 || bytes % (pattern == 2 ? 4096 : 16) != 0)
    return LSA_ERR_INVALID_ARGUMENT;
  if (sink_bytes < static_cast<size_t>(kBenchReadBlocks) * 256 * sizeof(uint32_t))
    return LSA_ERR_WORKSPACE_TOO_SMALL;
  (void)hipGetLastError();
  return hip_status(launch_bench_read(src_dev, bytes, pattern, static_cast<uint32_t*>(sink_dev),
                                      static_cast<hipStream_t>(hip_stream)));
}

lsa_status lsa_bench_flush(void* buf_dev, size_t bytes, void* hip_stream) {
  if (!buf_dev || bytes % 16 != 0 || !aligned(buf_dev, 16)) return LSA_ERR_INVALID_ARGUMENT;
  (void)hipGetLastError();
  return hip_status(launch_bench_flush(buf_dev, bytes, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
