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
//  * proportional split (per == 0): the device's `target` workgroups (one per
//    CU) are shared out in proportion to the streams' tiles,
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
  int32_t per;      // tiles per workgroup, or 0 for the proportional split
  int32_t target;   // workgroups the proportional split aims at
  int64_t grid;     // workgroups launched (upper bound of sum_b W_b)
  int64_t ws_rows;  // partial results the workspace holds (>= grid)
};

// `target` is the number of compute units of the device that will run it.
AttnPlan make_attn_plan(const lsa_shape& s, int32_t target);
// Compute units of the current device (host).
int32_t device_cu_count();

// Workspace layout: split-KV partials m[rows][H], l[rows][H] (fp32, log2
// domain max and sum) and o[rows][H][dv] (fp32, unnormalised), rows = ws_rows.
struct PartialLayout {
  size_t m_off, l_off, o_off, total;
};
PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p);

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
  float* ws_o;
  int32_t B, H, dqk, dv, C;
  int32_t k_row;          // elements between consecutive K rows
  int32_t v_row;          // elements between consecutive V rows
  int32_t pool;           // 1: slot-indexed pool, 0: store indexed by chunk
  int32_t tiles_per_chunk, per, target;
  int32_t uni_k;          // k of every stream when the shape is uniform, else 0
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
hipError_t launch_attn_mqa(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st);
bool mla_attn_supported(const lsa_shape& s);
hipError_t launch_attn_mla(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st);
bool portable_attn_supported(const lsa_shape& s);
hipError_t launch_attn_portable(const lsa_shape& s, const AttnArgs& a, int64_t grid,
                                hipStream_t st);
hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, hipStream_t st);
hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t st);
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
  __device__ __forceinline__ int32_t at(int32_t i) const { return uni > 0 ? i * uni : off[i]; }
};

// Split geometry of one stream (device): tiles T_b, workgroups W_b and tiles
// per workgroup, given the plan and the total tile count T.
struct StreamSplit {
  int32_t tiles, wgs, per;
};
__device__ __forceinline__ StreamSplit stream_split(SelCsr sel_off, int32_t b, int32_t tpc,
                                                    int32_t per, int32_t target,
                                                    int32_t total_tiles) {
  StreamSplit r;
  int32_t k = sel_off.at(b + 1) - sel_off.at(b);
  if (k < 0) k = 0;
  r.tiles = k * tpc;
  if (per > 0) {
    r.per = per;
    r.wgs = ceil_div_i(r.tiles, per);
  } else {
    const int64_t num = 2 * static_cast<int64_t>(r.tiles) * target + total_tiles;
    int32_t w = total_tiles > 0 ? static_cast<int32_t>(num / (2 * static_cast<int64_t>(total_tiles))) : 0;
    if (w < 1) w = 1;
    const int32_t w_min = ceil_div_i(r.tiles, run_tile_cap(tpc));
    if (w < w_min) w = w_min;
    if (w > r.tiles) w = r.tiles;
    r.per = w > 0 ? ceil_div_i(r.tiles, w) : 1;
    // runs of `per` tiles may need fewer workgroups than w (e.g. 2620 tiles
    // over 256: runs of 11 fill 239), and a workgroup with no tiles would
    // still write a partial that the merge reads
    r.wgs = w > 0 ? ceil_div_i(r.tiles, r.per) : 0;
  }
  return r;
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
  const int32_t total_tiles = (sel_off.at(B) - sel_off.at(0)) * tpc;
  if (sel_off.uni > 0) {  // every stream has the same split
    const StreamSplit sp = stream_split(sel_off, 0, tpc, per, target, total_tiles);
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
  int32_t base = 0;  // workgroups of streams before the current 64-stream window
  for (int32_t s0 = 0; s0 < B; s0 += kWave) {
    const int32_t s = s0 + lane;
    StreamSplit sp = {0, 0, 1};
    int32_t so = 0;
    if (s < B) {
      sp = stream_split(sel_off, s, tpc, per, target, total_tiles);
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
    find_stream_of_wg(SelCsr{a.sel_off, a.uni_k}, a.B, tpc, a.per, a.target, blockIdx.x, &b,
                      &local, &sp, &sel0);
    AttnRun r = {b, 0, 0, 0, 0, 0, 0};
    if (b >= 0) {
      r.t_begin = local * sp.per;
      r.t_end = min(sp.tiles, (local + 1) * sp.per);
      r.sel0 = sel0;
      r.slot_first = r.t_begin / tpc;
      const int32_t nslots = min((r.t_end - 1) / tpc - r.slot_first + 1, kMaxRunSlots);
      const int64_t t0 = a.tok_off[b], t1 = a.tok_off[b + 1];
      const int64_t sl = a.seq_len ? a.seq_len[b] : t1 - t0;
      for (int32_t i = lane; i < nslots; i += kWave) s_slot[i] = a.sel_idx[sel0 + r.slot_first + i];
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
  const int32_t total_tiles = (sel_off.at(B) - sel_off.at(0)) * tpc;
  if (sel_off.uni > 0) {  // every stream has the same split
    const int32_t w = stream_split(sel_off, 0, tpc, per, target, total_tiles).wgs;
    *first_out = b * w;
    *count_out = w;
    return;
  }
  uint32_t acc = 0;
  for (int32_t s0 = 0; s0 < b; s0 += kWave) {
    const int32_t s = s0 + lane;
    if (s < b) acc += static_cast<uint32_t>(stream_split(sel_off, s, tpc, per, target, total_tiles).wgs);
  }
  *first_out = static_cast<int32_t>(wave_sum_u32(acc));
  *count_out = stream_split(sel_off, b, tpc, per, target, total_tiles).wgs;
}

}  // namespace lsa
