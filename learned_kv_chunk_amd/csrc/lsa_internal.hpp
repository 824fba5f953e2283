// lsa_internal.hpp -- shared definitions of the HIP implementation of lsa.h
// (kernel launch declarations, the split-KV work plan, device helpers).
// Everything here targets gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"
#include "wave.hpp"

namespace lsa {

constexpr int kWave = 64;
constexpr int kTileTokens = 32;        // tokens per attention tile

// ---------------------------------------------------------------------------
// Split-KV work plan.  Stream b owns T_b = k_b * tiles_per_chunk tiles of 32
// tokens (T = sum_b T_b = sel_off[B] * tiles_per_chunk); each attention
// workgroup owns a run of consecutive tiles of one stream, and the W_b
// workgroups of stream b are numbered consecutively in stream order.
//  * fixed split (per > 0): W_b = ceil(T_b / per), runs of `per` tiles;
//  * balanced split (per == 0, at most 64 streams): one run length p for the
//    whole batch, the smallest for which the streams' ceil(T_b / p) runs
//    number at most `target` (the device's CUs); stream b's W_b =
//    ceil(T_b / p) workgroups then hold per_b = ceil(T_b / W_b) <= p tiles
//    each.  The longest run is what the launch waits for, and a stream whose
//    share of the CUs is fractional would otherwise get one workgroup
//    carrying up to 1.5 times the average (32 ragged streams: 102 tiles
//    against 72.6, where this plan's longest run is 79).  A uniform batch
//    (every stream keeps the same count) has the closed form
//    p = ceil(T_b / floor(target / B)); the host computes that split and
//    passes it in (SelCsr::uwgs, uper), so the kernels skip the search;
//  * proportional split (per == 0, more than 64 streams): the `target`
//    workgroups are shared out in proportion to the streams' tiles,
//    w_b = max(1, round(T_b * target / T)), stream b's runs hold
//    per_b = ceil(T_b / w_b) tiles, so every CU gets about T / target tiles,
//    and W_b = ceil(T_b / per_b) <= w_b workgroups carry them.
// Either way a run holds at most run_tile_cap(tiles_per_chunk) tiles (W_b is
// raised where needed), so that the kept-chunk indices of any run fit in
// kMaxRunSlots LDS words.  Workgroup ids at or beyond sum_b W_b do nothing;
// the grid is a bound known on the host from the shape alone.
// ---------------------------------------------------------------------------
constexpr int32_t kMaxRunSlots = 1024;  // kept chunks one run can span

// Longest run of tiles: a run of n tiles starting anywhere spans at most
// n / tpc + 2 chunks.
__host__ __device__ __forceinline__ int32_t run_tile_cap(int32_t tpc) {
  return (kMaxRunSlots - 2) * tpc;
}

struct AttnPlan {
  int32_t tiles_per_chunk;
  int32_t per;      // tiles per workgroup, or 0 for the balanced / proportional split
  int32_t target;   // workgroups the balanced and proportional splits aim at
  int64_t grid;     // workgroups launched (upper bound of sum_b W_b)
  int64_t ws_rows;  // partial results the workspace holds (>= grid)
  int32_t split_heads;  // vector-ALU kernel: the waves share each tile, split its heads
};

// `target` is the number of compute units of the device that will run it.
AttnPlan make_attn_plan(const lsa_shape& s, int32_t target);
// Compute units of the current device (host; queried once per device).
int32_t device_cu_count();

// Workspace layout: first the arrival counters of the kernels that merge a
// stream's partials in its last workgroup, int32 [kCounterStreams] at offset
// 0 for every shape (so that no shape's partials ever overlap another shape's
// counters in a shared workspace; they are zero between calls, every launch
// leaves them as it found them); then the split-KV partials m[rows][H],
// l[rows][H] (fp32, log2 domain max and sum) and o[rows][H][dv]
// (unnormalised; fp32, or bf16 where partial_o_bf16 holds), rows = ws_rows.
// Batches of more than kCounterStreams streams merge in a separate launch.
constexpr int32_t kCounterStreams = 16384;
struct PartialLayout {
  size_t m_off, l_off, o_off, cnt_off, total;
};
PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p);
// Whether the partial output rows o are stored as bf16 (the absorbed-MLA
// kernel: 64 heads x 512 latent columns per partial, so the partials are a
// large fraction of a step's bytes; the maxima and sums stay fp32).
bool partial_o_bf16(const lsa_shape& s);

struct AttnArgs {
  const void* q;          // [B][H][dqk]
  const void* k;          // store or pool
  const void* v;          // store or pool (== k when aliased)
  const int64_t* tok_off;  // rows of stream b start at tok_off[b]
  const int64_t* seq_len;  // L_b, or null: L_b = tok_off[b+1] - tok_off[b]
  const int32_t* sel_idx;
  const int32_t* sel_off;
  float* out;
  float* lse;
  float* ws_m;
  float* ws_l;
  float* ws_o;             // fp32 partial rows, or (o_bf16) the same region as bf16 bits
  int32_t o_bf16;          // 1: partial rows are bf16 (partial_o_bf16)
  int32_t* counters;      // per-stream arrival counters (zero between calls)
  int32_t fuse_merge;     // 1: the partial kernel merges each stream itself
  // In-kernel top-k (sel_scores non-null): every workgroup ranks its
  // stream's scores itself instead of reading sel_idx, and the stream's
  // first workgroup writes the kept set to sel_idx_out.
  const float* sel_scores;   // [total_chunks] fp32 scores, or null
  const int32_t* chunk_off;  // [B+1] (read unless uni_n > 0)
  int32_t* sel_idx_out;      // [total_k]
  int32_t uni_n;             // chunks of every stream when the shape is uniform, else 0
  int32_t B, H, dqk, dv, C;
  int32_t k_row;          // elements between consecutive K rows
  int32_t v_row;          // elements between consecutive V rows
  int32_t pool;           // 1: slot-indexed pool, 0: store indexed by chunk
  int32_t tiles_per_chunk, per, target;
  int32_t uni_k;          // k of every stream when the shape is uniform, else 0
  int32_t uni_wgs, uni_per;  // uniform shape: every stream's workgroups and run length
  int32_t split_heads;    // AttnPlan::split_heads
  float scale_log2;       // softmax_scale * log2(e)
};

// Kernel launchers (each returns hipGetLastError() of its launch).
hipError_t launch_score(const lsa_shape& s, const void* q, const void* emb,
                        const int32_t* chunk_off, float* scores, hipStream_t st);
hipError_t launch_select(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                         const int32_t* sel_off, int32_t* sel_idx, hipStream_t st);
hipError_t launch_gather(const lsa_shape& s, const void* store, int32_t row_bytes,
                         const int64_t* tok_off, const int32_t* sel_idx,
                         const int32_t* sel_off, void* pool, const void* store2,
                         int32_t row_bytes2, void* pool2, hipStream_t st);
bool score_supported(const lsa_shape& s);
bool score_mh_supported(int32_t heads, int32_t head_dim);
hipError_t launch_score_mh(const lsa_shape& s, int32_t layers, int32_t combine, int32_t heads,
                           int32_t head_dim, const void* q, const float* w, const void* rec,
                           const int32_t* chunk_off, float* scores, hipStream_t st);
hipError_t launch_select_threshold(const lsa_shape& s, const float* scores,
                                   const int32_t* chunk_off, float threshold, int32_t max_keep,
                                   int32_t* sel_off, int32_t* sel_idx, int32_t* fallback,
                                   int32_t* counts, hipStream_t st);
int32_t pool_delta_max_stream_chunks();
hipError_t launch_append_kv(const lsa_shape& s, const void* k_new, const void* v_new,
                           int32_t k_row_bytes, int32_t v_row_bytes, const int64_t* base_off,
                           int64_t* seq_len, void* k_store, void* v_store, hipStream_t st);
hipError_t launch_keep_recent(const lsa_shape& s, const int64_t* seq_len,
                              const int32_t* chunk_off, const int32_t* sel_idx,
                              const int32_t* sel_off, int32_t max_recent, int32_t* out_idx,
                              int32_t* out_off, hipStream_t st);
hipError_t launch_pool_delta(const lsa_shape& s, const void* k_host_dev, int32_t k_row_bytes,
                             const void* v_host_dev, int32_t v_row_bytes,
                             const int64_t* tok_off, const int32_t* chunk_off,
                             const int32_t* sel_idx, const int32_t* sel_off, int32_t* table,
                             int32_t* loads, int32_t* load_count, void* k_pool, void* v_pool,
                             hipStream_t st);
// Attention partial kernels (one per kernel family) and the merge.
bool mqa_attn_supported(const lsa_shape& s);
// The MQA kernel can rank each stream's kept chunks itself (in-kernel top-k).
bool mqa_select_in_kernel_supported(const lsa_shape& s);
hipError_t launch_attn_mqa(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st);
bool mla_attn_supported(const lsa_shape& s);
hipError_t launch_attn_mla(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st);
bool portable_attn_supported(const lsa_shape& s);
// Whether the vector-ALU kernel runs its split-heads form for a shape with
// total_tiles tiles on `target` compute units (small inputs, 5-16 heads,
// rows of at most 256 bytes).
bool portable_split_heads(const lsa_shape& s, int64_t total_tiles, int32_t target);
// Whether that form can rank the kept chunks in its prologue (streams of up
// to 4096 chunks keeping up to kMaxRunSlots).
bool portable_select_in_kernel_supported(const lsa_shape& s, const AttnPlan& plan);
hipError_t launch_attn_portable(const lsa_shape& s, const AttnArgs& a, int64_t grid,
                                hipStream_t st);
hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, const AttnPlan& plan,
                             hipStream_t st);
// Zeroes the per-stream arrival counters at the start of a workspace (a
// fill kernel: no memset node if the caller captures the stream in a graph).
hipError_t launch_clear_counters(void* ws, hipStream_t st);
hipError_t launch_check_tables(const lsa_shape& s, const int64_t* tok_off,
                               const int32_t* chunk_off, const int32_t* sel_off,
                               const int32_t* sel_idx, int32_t ascending, int32_t* flag,
                               hipStream_t st);
hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
constexpr int32_t kBenchReadBlocks = 256 * 32;  // workgroups of 256 threads of lsa_bench_read
hipError_t launch_bench_read(const void* src, size_t bytes, int32_t pattern, uint32_t* sink,
                             hipStream_t st);
hipError_t launch_bench_flush(void* buf, size_t bytes, hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ int32_t ceil_div_i(int32_t a, int32_t b) { return (a + b - 1) / b; }

// The kept-chunk offsets sel_off[0..B]: read from memory, or b * uni for a
// uniform shape (every stream keeps uni chunks), which needs no load.
struct SelCsr {
  const int32_t* off;
  int32_t uni;
  int32_t uwgs, uper;  // uniform batch: every stream's W_b and run length (host-computed)
  __device__ __forceinline__ int32_t at(int32_t i) const { return uni > 0 ? i * uni : off[i]; }
};

// Split geometry of a stream of `tiles` tiles (host and device): workgroups
// W_b and tiles per workgroup, given the plan, the total tile count T and the
// balanced run length (0: not the balanced split).
struct StreamSplit {
  int32_t tiles, wgs, per;
};
__host__ __device__ inline int32_t ceil_div_hd(int32_t a, int32_t b) { return (a + b - 1) / b; }
__host__ __device__ inline StreamSplit split_of_tiles(int32_t tiles, int32_t tpc, int32_t per,
                                                      int32_t target, int32_t total_tiles,
                                                      int32_t bal) {
  StreamSplit r;
  r.tiles = tiles;
  if (per > 0) {
    r.per = per;
    r.wgs = ceil_div_hd(r.tiles, per);
  } else if (bal > 0) {
    const int32_t cap = run_tile_cap(tpc);
    const int32_t p = bal < cap ? bal : cap;
    const int32_t w = ceil_div_hd(r.tiles, p);
    r.per = w > 0 ? ceil_div_hd(r.tiles, w) : 1;  // even runs, none longer than p
    r.wgs = w > 0 ? ceil_div_hd(r.tiles, r.per) : 0;
  } else {
    const int64_t num = 2 * static_cast<int64_t>(r.tiles) * target + total_tiles;
    int32_t w = total_tiles > 0 ? static_cast<int32_t>(num / (2 * static_cast<int64_t>(total_tiles))) : 0;
    if (w < 1) w = 1;
    const int32_t w_min = ceil_div_hd(r.tiles, run_tile_cap(tpc));
    if (w < w_min) w = w_min;
    if (w > r.tiles) w = r.tiles;
    r.per = w > 0 ? ceil_div_hd(r.tiles, w) : 1;
    // runs of `per` tiles may need fewer workgroups than w (e.g. 2620 tiles
    // over 256: runs of 11 fill 239), and a workgroup with no tiles would
    // still write a partial that the merge reads
    r.wgs = w > 0 ? ceil_div_hd(r.tiles, r.per) : 0;
  }
  return r;
}

// Balanced run length of a uniform batch (B streams of t tiles each), the
// closed form of balanced_run's search: p = ceil(t / floor(target / B)), or
// t when there are more streams than `target`; 0 when the batch takes another
// split.
__host__ __device__ inline int32_t uniform_balanced_run(int32_t B, int32_t t, int32_t per,
                                                        int32_t target) {
  if (per > 0 || B > kWave || B < 1) return 0;
  const int32_t m = target / B;
  const int32_t p = m >= 1 ? ceil_div_hd(t, m) : t;
  return p > 1 ? p : 1;
}

// Run length p of the balanced split of a ragged batch of B <= 64 streams
// (see the plan above), from lane s's tiles t (stream s; 0 past B) and their
// sum T.  Called by a full wave; every lane returns the same value.
__device__ __forceinline__ int32_t balanced_run(int32_t t, int32_t total_tiles, int32_t B,
                                                int32_t target) {
  // the longest stream (one workgroup each at p = its tiles)
  const uint32_t tmax = wave_max_u32(static_cast<uint32_t>(t));
  if (tmax == 0) return 1;
  // smallest p with sum_b ceil(T_b / p) <= target (the sum does not grow with
  // p; at p = tmax it is the number of streams): at least ceil(T / target),
  // and, since the sum is below T / p + B, at most ceil(T / (target - B))
  int32_t lo = max(1, ceil_div_i(total_tiles, max(target, 1)));
  int32_t hi = static_cast<int32_t>(tmax);
  if (target > B) hi = min(hi, max(lo, ceil_div_i(total_tiles, target - B)));
  if (lo >= hi) return hi;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo) / 2;
    const uint32_t w = t > 0 ? static_cast<uint32_t>(ceil_div_i(t, mid)) : 0u;
    if (wave_sum_u32(w) <= static_cast<uint32_t>(target)) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// A batch of at most 64 streams, one per lane (a full wave): lane s gets
// stream s's split (zero tiles past B) and its first kept index.  The offsets
// are read once, and the balanced run length comes from the same registers.
__device__ __forceinline__ StreamSplit lane_stream_split(SelCsr sel_off, int32_t B, int32_t tpc,
                                                         int32_t per, int32_t target,
                                                         int32_t* so_out) {
  const int lane = threadIdx.x & (kWave - 1);
  int32_t so = 0, t = 0;
  if (lane < B) {
    so = sel_off.at(lane);
    const int32_t k = sel_off.at(lane + 1) - so;
    t = k > 0 ? k * tpc : 0;
  }
  *so_out = so;
  const int32_t bal =
      per > 0 ? 0 : balanced_run(t, static_cast<int32_t>(wave_sum_u32(static_cast<uint32_t>(t))),
                                 B, target);
  return split_of_tiles(t, tpc, per, target, 0, bal);
}

__device__ __forceinline__ StreamSplit stream_split(SelCsr sel_off, int32_t b, int32_t tpc,
                                                    int32_t per, int32_t target,
                                                    int32_t total_tiles, int32_t bal) {
  int32_t k = sel_off.at(b + 1) - sel_off.at(b);
  if (k < 0) k = 0;
  return split_of_tiles(k * tpc, tpc, per, target, total_tiles, bal);
}

// Run by one full wave: the stream owning workgroup `wg`, the workgroup's
// index within that stream, and the stream's split.  b = -1 when wg is past
// the last workgroup.
__device__ __forceinline__ void find_stream_of_wg(SelCsr sel_off, int32_t B, int32_t tpc,
                                                  int32_t per, int32_t target, int32_t wg,
                                                  int32_t* b_out, int32_t* local_out,
                                                  StreamSplit* split_out,
                                                  int32_t* sel0_out = nullptr) {
  const int lane = threadIdx.x & (kWave - 1);
  if (sel_off.uni > 0) {  // every stream has the same split, computed on the host
    const StreamSplit sp = {sel_off.uni * tpc, sel_off.uwgs, sel_off.uper};
    if (sp.wgs > 0 && wg < B * sp.wgs) {
      *b_out = wg / sp.wgs;
      *local_out = wg - *b_out * sp.wgs;
      *split_out = sp;
      if (sel0_out) *sel0_out = *b_out * sel_off.uni;
      return;
    }
    *b_out = -1;
    *local_out = 0;
    *split_out = StreamSplit{0, 0, 1};
    if (sel0_out) *sel0_out = 0;
    return;
  }
  const int32_t total_tiles = B > kWave ? (sel_off.at(B) - sel_off.at(0)) * tpc : 0;
  int32_t base = 0;  // workgroups of streams before the current 64-stream window
  for (int32_t s0 = 0; s0 < B; s0 += kWave) {
    const int32_t s = s0 + lane;
    StreamSplit sp = {0, 0, 1};
    int32_t so = 0;
    if (B <= kWave) {  // one window: the balanced (or fixed) split of lane_stream_split
      sp = lane_stream_split(sel_off, B, tpc, per, target, &so);
    } else if (s < B) {  // more streams: the proportional (or fixed) split
      sp = stream_split(sel_off, s, tpc, per, target, total_tiles, 0);
      so = sel_off.at(s);
    }
    const int32_t incl = static_cast<int32_t>(wave_inclusive_scan(static_cast<uint32_t>(sp.wgs)));
    const int32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (wg < base + total) {
      const uint64_t hit = __ballot(base + incl > wg);
      const int first = __ffsll(static_cast<long long>(hit)) - 1;
      const int32_t excl = __builtin_amdgcn_readlane(incl - sp.wgs, first);
      *b_out = s0 + first;
      *local_out = wg - base - excl;
      split_out->tiles = __builtin_amdgcn_readlane(sp.tiles, first);
      split_out->wgs = __builtin_amdgcn_readlane(sp.wgs, first);
      split_out->per = __builtin_amdgcn_readlane(sp.per, first);
      if (sel0_out) *sel0_out = __builtin_amdgcn_readlane(so, first);
      return;
    }
    base += total;
  }
  *b_out = -1;
  *local_out = 0;
  *split_out = StreamSplit{0, 0, 1};
  if (sel0_out) *sel0_out = 0;
}

// A 64-bit value that is the same in every lane, as scalar registers (the two
// halves are joined unsigned).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(x)));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(x >> 32)));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The run of tiles one attention workgroup owns.
struct AttnRun {
  int32_t b;           // stream, or -1 when the workgroup has no work
  int32_t t_begin;     // tiles [t_begin, t_end) of the stream's kept tokens
  int32_t t_end;
  int32_t sel0;        // sel_off[b]
  int32_t slot_first;  // the run's first kept chunk, counted within the stream
  int32_t local;       // this workgroup's index among the stream's
  int32_t wgs;         // the stream's workgroups (partials)
  int32_t cbase;       // chunk_off[b] (in-kernel top-k only)
  int32_t cn;          // N_b (in-kernel top-k only)
  int32_t kb;          // k_b
  int64_t tb;          // tok_off[b]
  int64_t len;         // L_b
};

// Workgroup prologue of the attention kernels, called by every thread; ends
// with a barrier.  Wave 0 finds the workgroup's stream and run (one round trip
// over sel_off), then loads the stream's token range and the run's kept-chunk
// indices together (a second round trip) into `s_slot` (kMaxRunSlots words)
// and `s_run`, which every thread then reads.
__device__ __forceinline__ AttnRun attn_prologue(const AttnArgs& a, int32_t* s_slot,
                                                 AttnRun* s_run) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int32_t tpc = a.tiles_per_chunk;
    int32_t b, local, sel0;
    StreamSplit sp;
    find_stream_of_wg(SelCsr{a.sel_off, a.uni_k, a.uni_wgs, a.uni_per}, a.B, tpc, a.per,
                      a.target, blockIdx.x, &b, &local, &sp, &sel0);
    AttnRun r = {b, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    if (b >= 0) {
      r.local = local;
      r.wgs = sp.wgs;
      r.kb = sp.tiles / tpc;
      r.t_begin = local * sp.per;
      r.t_end = min(sp.tiles, (local + 1) * sp.per);
      r.sel0 = sel0;
      r.slot_first = r.t_begin / tpc;
      const int32_t nslots = min((r.t_end - 1) / tpc - r.slot_first + 1, kMaxRunSlots);
      const int64_t t0 = a.tok_off[b], t1 = a.tok_off[b + 1];
      const int64_t sl = a.seq_len ? a.seq_len[b] : t1 - t0;
      if (a.sel_scores == nullptr) {
        for (int32_t i = lane; i < nslots; i += kWave)
          s_slot[i] = a.sel_idx[sel0 + r.slot_first + i];
      } else {  // the kept set is ranked in the kernel: the stream's chunk range
        r.cbase = a.uni_n > 0 ? b * a.uni_n : a.chunk_off[b];
        r.cn = a.uni_n > 0 ? a.uni_n : a.chunk_off[b + 1] - r.cbase;
      }
      r.tb = t0;
      r.len = sl < 0 ? 0 : (sl < t1 - t0 ? sl : t1 - t0);
    }
    if (lane == 0) *s_run = r;
  }
  __syncthreads();
  // the run is uniform over the workgroup: scalar registers hold it
  const AttnRun v = *s_run;
  AttnRun u;
  u.b = __builtin_amdgcn_readfirstlane(v.b);
  u.t_begin = __builtin_amdgcn_readfirstlane(v.t_begin);
  u.t_end = __builtin_amdgcn_readfirstlane(v.t_end);
  u.sel0 = __builtin_amdgcn_readfirstlane(v.sel0);
  u.slot_first = __builtin_amdgcn_readfirstlane(v.slot_first);
  u.local = __builtin_amdgcn_readfirstlane(v.local);
  u.wgs = __builtin_amdgcn_readfirstlane(v.wgs);
  u.cbase = __builtin_amdgcn_readfirstlane(v.cbase);
  u.cn = __builtin_amdgcn_readfirstlane(v.cn);
  u.kb = __builtin_amdgcn_readfirstlane(v.kb);
  u.tb = uniform_i64(v.tb);
  u.len = uniform_i64(v.len);
  return u;
}

// Run by one full wave: index of the first workgroup of stream b and its
// workgroup count.
__device__ __forceinline__ void stream_wg_range(SelCsr sel_off, int32_t B, int32_t b,
                                                int32_t tpc, int32_t per, int32_t target,
                                                int32_t* first_out, int32_t* count_out) {
  const int lane = threadIdx.x & (kWave - 1);
  if (sel_off.uni > 0) {  // every stream has the same split, computed on the host
    *first_out = b * sel_off.uwgs;
    *count_out = sel_off.uwgs;
    return;
  }
  if (B <= kWave) {  // one window: the balanced (or fixed) split of lane_stream_split
    int32_t so;
    const StreamSplit sp = lane_stream_split(sel_off, B, tpc, per, target, &so);
    const uint32_t incl = wave_inclusive_scan(static_cast<uint32_t>(sp.wgs));
    *first_out = static_cast<int32_t>(__builtin_amdgcn_readlane(incl - sp.wgs, b));
    *count_out = __builtin_amdgcn_readlane(sp.wgs, b);
    return;
  }
  const int32_t total_tiles = (sel_off.at(B) - sel_off.at(0)) * tpc;
  uint32_t acc = 0;
  for (int32_t s0 = 0; s0 < b; s0 += kWave) {
    const int32_t s = s0 + lane;
    if (s < b)
      acc += static_cast<uint32_t>(stream_split(sel_off, s, tpc, per, target, total_tiles, 0).wgs);
  }
  *first_out = static_cast<int32_t>(wave_sum_u32(acc));
  *count_out = stream_split(sel_off, b, tpc, per, target, total_tiles, 0).wgs;
}

// Device-scope (all XCDs' L2s) coherent stores of the split partials that a
// stream's last workgroup merges: they write through to the device's
// coherence point (global_store with the sc1 bit), so publishing a partial
// needs no write-back of the L2.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes stored at base + byte_off (base the same in every lane, byte_off
// < 2^31; stores past that are dropped) with the sc1 cache policy: written through to the device's coherence point instead of being
// left dirty in the XCD's L2 until the end of the kernel.  For large split
// partials (the MLA kernel's 128 KiB per workgroup, the two-group MQA
// kernel's 16 KiB) that made the partial kernel shorter (1 x 1M: 30.4 -> 28.5
// us; 4 x 512K: 25.4 -> 24.3 us); for 8 KiB partials it was slower (16 x
// 128K: 28.0 -> 28.5 us), interleaved on one box.
typedef uint32_t st_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t st_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_through_16(float* base, uint32_t byte_off, st_u32x4 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 16 /* sc1 */);
}
// The same for 8 bytes.
__device__ __forceinline__ void store_through_8(void* base, uint32_t byte_off, st_u32x2 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 16 /* sc1 */);
}

// Merge of one stream's split-KV partials by the NT threads of the stream's
// last workgroup to finish (after arrive_last): rows first .. first + count -
// 1 of the workspace are combined into out[b] and lse[b].  Thread i owns
// EPT = 8 consecutive output elements of the flattened [H][dv] row (the
// caller guarantees H * dv <= 8 * NT and dv % 8 == 0, so the eight share a
// head), and the loads of a batch of kBlockMergeBatch partials (two 16-byte
// vectors, the maximum and the sum each) are all issued before any is used:
// one memory round trip per batch.  Partials are folded in row order, one
// rescale per batch, so the result is a deterministic function of the plan.
constexpr int kBlockMergeBatch = 16;

template <int NT>
__device__ __forceinline__ void merge_stream_block(const AttnArgs& a, int32_t b, int64_t first,
                                                   int32_t count) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int32_t H = a.H, dv = a.dv, elems = H * dv;
  const int32_t e = static_cast<int32_t>(threadIdx.x) * 8;
  if (e >= elems) return;
  const int32_t h = e / dv;
  float m = -INFINITY, l = 0.f;
  f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int32_t p0 = 0; p0 < count; p0 += kBlockMergeBatch) {
    f4 o0[kBlockMergeBatch], o1[kBlockMergeBatch];
    float mv[kBlockMergeBatch], lv[kBlockMergeBatch];
#pragma unroll
    for (int u = 0; u < kBlockMergeBatch; ++u) {
      const int64_t row = first + min(p0 + u, count - 1);
      const f4* src = reinterpret_cast<const f4*>(a.ws_o + row * elems + e);
      o0[u] = src[0];
      o1[u] = src[1];
      mv[u] = a.ws_m[row * H + h];
      lv[u] = a.ws_l[row * H + h];
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kBlockMergeBatch; ++u)
      if (p0 + u < count) mb = fmaxf(mb, mv[u]);
    const float mu = (mb == -INFINITY) ? 0.f : mb;
    const float f = __builtin_amdgcn_exp2f(m - mu);
    acc0 *= f;
    acc1 *= f;
    l *= f;
#pragma unroll
    for (int u = 0; u < kBlockMergeBatch; ++u) {
      if (p0 + u < count) {
        const float w = __builtin_amdgcn_exp2f(mv[u] - mu);
        acc0 += o0[u] * w;
        acc1 += o1[u] * w;
        l = fmaf(lv[u], w, l);
      }
    }
    m = mb;
  }
  const int64_t orow = static_cast<int64_t>(b) * H + h;
  const int32_t c = e - h * dv;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  f4* dst = reinterpret_cast<f4*>(a.out + orow * dv + c);
  dst[0] = acc0 * inv;
  dst[1] = acc1 * inv;
  if (c == 0 && a.lse != nullptr)
    a.lse[orow] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

// Arrival of a workgroup whose partial for stream b has been written with
// store_coherent or store_through_16: every wave waits until its own stores are acknowledged at
// the device's coherence point, then one thread increments the stream's
// counter (a device-scope atomic).  The workgroup that sees the count reach
// wgs - 1 arrived last: every other partial is already at the coherence
// point, and an acquire at device scope (an invalidation of this XCD's
// caches) makes its plain loads find them.  Returns true in every thread of
// that workgroup, which resets the counter once it has read the partials.
// s_flag: one LDS word.
__device__ __forceinline__ bool arrive_last(const AttnArgs& a, int32_t b, int32_t wgs,
                                            int32_t* s_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t old =
        __hip_atomic_fetch_add(a.counters + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old == wgs - 1) ? 1 : 0;
  }
  __syncthreads();
  if (*s_flag == 0) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

}  // namespace lsa
