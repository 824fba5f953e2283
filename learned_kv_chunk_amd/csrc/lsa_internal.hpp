// lsa_internal.hpp -- shared definitions of the HIP implementation of lsa.h
// (kernel launch declarations, the split-KV work plan, device helpers).
// Everything here targets gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

constexpr int kWave = 64;
constexpr int kTileTokens = 32;        // tokens per attention tile
constexpr int kAttnWaves = 4;          // waves per attention workgroup
constexpr int kAttnThreads = kAttnWaves * kWave;

// ---------------------------------------------------------------------------
// Split-KV work plan.  Stream b owns T_b = k_b * tiles_per_chunk tiles of 32
// tokens; each attention workgroup owns `per` consecutive tiles of one stream,
// so stream b has W_b = ceil(T_b / per) workgroups, numbered consecutively in
// stream order.  Workgroup ids at or beyond sum_b W_b do nothing.  The grid is
// the bound ceil(sum T_b / per) + B, known on the host from the shape alone.
// ---------------------------------------------------------------------------
struct AttnPlan {
  int32_t tiles_per_chunk;
  int32_t per;      // tiles per workgroup (multiple of kAttnWaves)
  int64_t grid;     // workgroups launched (upper bound of sum_b W_b)
  int64_t ws_rows;  // partial results the workspace holds (>= grid)
};

AttnPlan make_attn_plan(const lsa_shape& s);

// Workspace layout for split-KV partials: m[rows][H], l[rows][H] (fp32, log2
// domain max and sum) then o[rows][H][dv] (fp32, unnormalised), rows = ws_rows.
struct PartialLayout {
  size_t m_off, l_off, o_off, total;
};
PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p);

struct AttnArgs {
  const void* q;          // [B][H][dqk]
  const void* k;          // store or pool
  const void* v;          // store or pool (== k when aliased)
  const int64_t* tok_off;
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
  int32_t tiles_per_chunk, per;
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

// Number of attention workgroups of stream b.
__device__ __forceinline__ int32_t stream_wgs(const int32_t* sel_off, int32_t b, int32_t tpc,
                                              int32_t per) {
  int32_t k = sel_off[b + 1] - sel_off[b];
  if (k < 0) k = 0;
  return ceil_div_i(k * tpc, per);
}

// Run by one full wave: the stream owning workgroup `wg` and the workgroup's
// index within that stream.  Returns b = -1 when wg is past the last one.
__device__ __forceinline__ void find_stream_of_wg(const int32_t* sel_off, int32_t B,
                                                  int32_t tpc, int32_t per, int32_t wg,
                                                  int32_t* b_out, int32_t* local_out) {
  const int lane = threadIdx.x & (kWave - 1);
  int32_t base = 0;  // workgroups of streams before the current 64-stream window
  for (int32_t s0 = 0; s0 < B; s0 += kWave) {
    const int32_t s = s0 + lane;
    int32_t n = (s < B) ? stream_wgs(sel_off, s, tpc, per) : 0;
    // inclusive prefix over the window
    int32_t incl = n;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int32_t y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    const int32_t total = __shfl(incl, kWave - 1, kWave);
    if (wg < base + total) {
      const uint64_t hit = __ballot(base + incl > wg);
      const int first = __ffsll(static_cast<long long>(hit)) - 1;
      const int32_t excl = __shfl(incl - n, first, kWave);
      *b_out = s0 + first;
      *local_out = wg - base - excl;
      return;
    }
    base += total;
  }
  *b_out = -1;
  *local_out = 0;
}

// Run by one full wave: index of the first workgroup of stream b.
__device__ __forceinline__ int32_t first_wg_of_stream(const int32_t* sel_off, int32_t b,
                                                      int32_t tpc, int32_t per) {
  const int lane = threadIdx.x & (kWave - 1);
  int32_t acc = 0;
  for (int32_t s0 = 0; s0 < b; s0 += kWave) {
    const int32_t s = s0 + lane;
    acc += (s < b) ? stream_wgs(sel_off, s, tpc, per) : 0;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  return acc;
}

}  // namespace lsa
