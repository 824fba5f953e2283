// attn_common.hip -- split-KV work plan, partial-result layout and the
// log-sum-exp merge of sparse decode attention.
//
// Dimensionstp review, section 3-2-3 steps 6-7: attention runs over the kept
// chunks only.  The kept tokens of a stream are cut into 32-token tiles;
// workgroups own runs of tiles (the plan in lsa_internal.hpp) and leave one
// partial result each: the running maximum m and sum l of exp2(logit*log2e -
// m) per head, and the unnormalised output row.  The merge combines a
// stream's partials: m* = max m_p, l* = sum l_p 2^(m_p-m*),
// out = sum o_p 2^(m_p-m*) / l*, lse = ln2 * (m* + log2 l*).
#include <math.h>

#include "lsa_internal.hpp"

namespace lsa {

namespace {
constexpr int64_t kTargetWorkgroups = 512;  // two resident workgroups per CU on 256 CUs
constexpr int32_t kMaxTilesPerWorkgroup = 256;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

AttnPlan make_attn_plan(const lsa_shape& s) {
  AttnPlan p;
  p.tiles_per_chunk = (s.chunk_size + kTileTokens - 1) / kTileTokens;
  const int64_t total_tiles = s.total_k * p.tiles_per_chunk;
  int64_t per = s.attn_tiles_per_block;
  if (per <= 0) per = (total_tiles + kTargetWorkgroups - 1) / kTargetWorkgroups;
  per = (per + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
  if (per < kAttnWaves) per = kAttnWaves;
  if (per > kMaxTilesPerWorkgroup) per = kMaxTilesPerWorkgroup;
  p.per = static_cast<int32_t>(per);
  p.grid = (total_tiles + per - 1) / per + s.batch;
  // Partial-result rows reserved in the workspace: a bound on `grid` that is
  // monotone in the shape (the automatic `per` keeps ceil(T/per) below both
  // ceil(T/4) and max(512, ceil(T/256))).
  if (s.attn_tiles_per_block > 0) {
    p.ws_rows = p.grid;
  } else {
    const int64_t a = (total_tiles + kAttnWaves - 1) / kAttnWaves;
    p.ws_rows = (a < kTargetWorkgroups ? a : kTargetWorkgroups) +
                (total_tiles + kMaxTilesPerWorkgroup - 1) / kMaxTilesPerWorkgroup + s.batch;
  }
  return p;
}

PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p) {
  PartialLayout L;
  const size_t rows = static_cast<size_t>(p.ws_rows) * static_cast<size_t>(s.num_q_heads);
  L.m_off = 0;
  L.l_off = align256(rows * sizeof(float));
  L.o_off = L.l_off + align256(rows * sizeof(float));
  L.total = L.o_off + align256(rows * static_cast<size_t>(s.head_dim_v) * sizeof(float));
  return L;
}

namespace {

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnArgs a) {
  __shared__ int32_t s_first, s_count;
  const int b = blockIdx.x;
  if (threadIdx.x < kWave) {
    const int32_t first = first_wg_of_stream(a.sel_off, b, a.tiles_per_chunk, a.per);
    if (threadIdx.x == 0) {
      s_first = first;
      s_count = stream_wgs(a.sel_off, b, a.tiles_per_chunk, a.per);
    }
  }
  __syncthreads();
  const int32_t e = blockIdx.y * kMergeThreads + threadIdx.x;
  if (e >= a.H * a.dv) return;
  const int32_t h = e / a.dv;
  const int32_t c = e - h * a.dv;
  const int32_t first = s_first, count = s_count;
  float m = -INFINITY;
  for (int32_t p = 0; p < count; ++p) m = fmaxf(m, a.ws_m[static_cast<int64_t>(first + p) * a.H + h]);
  float l = 0.f, o = 0.f;
  if (m != -INFINITY) {
    for (int32_t p = 0; p < count; ++p) {
      const int64_t row = static_cast<int64_t>(first + p) * a.H + h;
      const float mp = a.ws_m[row];
      const float f = (mp == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mp - m);
      l = fmaf(a.ws_l[row], f, l);
      o = fmaf(a.ws_o[row * a.dv + c], f, o);
    }
  }
  const int64_t orow = static_cast<int64_t>(b) * a.H + h;
  a.out[orow * a.dv + c] = (l > 0.f) ? o / l : 0.f;
  if (c == 0 && a.lse != nullptr)
    a.lse[orow] = (l > 0.f) ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, hipStream_t st) {
  const int32_t elems = s.num_q_heads * s.head_dim_v;
  dim3 grid(s.batch, (elems + kMergeThreads - 1) / kMergeThreads);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
