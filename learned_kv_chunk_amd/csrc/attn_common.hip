// attn_common.hip -- split-KV work plan and workspace layout of sparse decode
// attention.
//
// Dimensionstp review, section 3-2-3 steps 6-7: attention runs over the kept
// chunks only.  The kept tokens of a stream are cut into 32-token tiles;
// workgroups own runs of tiles (the plan in lsa_internal.hpp) and leave one
// partial result each: per head the running maximum m (log2 domain), the sum
// l of exp2(x - m) and the unnormalised output row o.  The merge combines a
// stream's partials: m* = max_p m_p, weights f_p = 2^(m_p - m*),
// out = sum_p f_p o_p / sum_p f_p l_p, lse = ln2 * (m* + log2 sum_p f_p l_p).
#include <math.h>

#include "lsa_internal.hpp"

namespace lsa {

namespace {
constexpr int32_t kDefaultTarget = 256;  // compute units of an MI355X

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

int32_t device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return kDefaultTarget;
  return cus;
}

AttnPlan make_attn_plan(const lsa_shape& s, int32_t target) {
  AttnPlan p;
  p.tiles_per_chunk = (s.chunk_size + kTileTokens - 1) / kTileTokens;
  const int64_t total_tiles = s.total_k * p.tiles_per_chunk;
  p.target = target > 0 ? target : kDefaultTarget;
  const int64_t cap = run_tile_cap(p.tiles_per_chunk);
  if (s.attn_tiles_per_block > 0) {
    int64_t per = s.attn_tiles_per_block;
    if (per > cap) per = cap;
    p.per = static_cast<int32_t>(per);
    p.grid = (total_tiles + per - 1) / per + s.batch;
    p.ws_rows = p.grid;
  } else {
    // sum_b max(1, round(T_b * target / T), ceil(T_b / cap))
    //   <= sum_b max(1, round(T_b * target / T)) + sum_b ceil(T_b / cap)
    //   <= (target + B) + (T / cap + B)
    p.per = 0;
    const int64_t extra = 2 * static_cast<int64_t>(s.batch) + total_tiles / cap + 1;
    p.grid = p.target + extra;
    p.ws_rows = (p.target > kDefaultTarget ? p.target : kDefaultTarget) + extra;
  }
  return p;
}

PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p) {
  PartialLayout L;
  const size_t rows = static_cast<size_t>(p.ws_rows) * static_cast<size_t>(s.num_q_heads);
  L.m_off = 0;
  L.l_off = L.m_off + align256(rows * sizeof(float));
  L.o_off = L.l_off + align256(rows * sizeof(float));
  L.total = L.o_off + align256(rows * static_cast<size_t>(s.head_dim_v) * sizeof(float));
  return L;
}

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 32;          // partial rows loaded per round trip
constexpr int kMergeMaxPairs = 4096;     // (partial, head) pairs staged in LDS
constexpr int kMergeMaxHeads = 33;       // heads one 256-element block can touch (dv >= 8)

// One workgroup per (stream, 256 output elements): stage the maxima and sums
// of the stream's partials for the block's heads in LDS, turn them into
// weights, then every thread sums its element over all partials with
// kMergeBatch independent loads in flight.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(AttnArgs a) {
  __shared__ float s_m[kMergeMaxPairs];
  __shared__ float s_l[kMergeMaxPairs];
  __shared__ float s_mstar[kMergeMaxHeads];
  __shared__ float s_lstar[kMergeMaxHeads];
  __shared__ int32_t s_info[2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t H = a.H, dv = a.dv;
  const int32_t elems = H * dv;
  const int32_t e0 = static_cast<int32_t>(blockIdx.y) * kMergeThreads;
  if (e0 >= elems) return;
  if (tid < kWave) {
    int32_t first, count;
    stream_wg_range(a.sel_off, a.B, b, a.tiles_per_chunk, a.per, a.target, &first, &count);
    if (tid == 0) {
      s_info[0] = first;
      s_info[1] = count;
    }
  }
  __syncthreads();
  const int64_t first = s_info[0];
  const int32_t count = s_info[1];
  const int32_t h_lo = e0 / dv;
  const int32_t h_hi = (min(elems, e0 + kMergeThreads) - 1) / dv;
  const int32_t nh = h_hi - h_lo + 1;
  const bool staged = count * nh <= kMergeMaxPairs;
  if (staged) {
    for (int32_t i = tid; i < count * nh; i += kMergeThreads) {
      const int32_t p = i / nh, hh = i - p * nh;
      const int64_t row = (first + p) * H + h_lo + hh;
      s_m[i] = a.ws_m[row];
      s_l[i] = a.ws_l[row];
    }
  }
  __syncthreads();
  // per-head maximum and normaliser: wave w reduces heads w, w+4, ... with its
  // lanes spread over the partials
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  for (int32_t hh = wave; hh < nh; hh += kMergeThreads / kWave) {
    float mx = -INFINITY;
    for (int32_t p = lane; p < count; p += kWave)
      mx = fmaxf(mx, staged ? s_m[p * nh + hh] : a.ws_m[(first + p) * H + h_lo + hh]);
    mx = wave_max(mx);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float l = 0.f;
    for (int32_t p = lane; p < count; p += kWave) {
      const float mp = staged ? s_m[p * nh + hh] : a.ws_m[(first + p) * H + h_lo + hh];
      const float lp = staged ? s_l[p * nh + hh] : a.ws_l[(first + p) * H + h_lo + hh];
      l = fmaf(lp, __builtin_amdgcn_exp2f(mp - mu), l);
    }
    l = wave_sum(l);
    if (lane == 0) {
      s_mstar[hh] = mx;
      s_lstar[hh] = l;
    }
  }
  __syncthreads();
  if (staged) {
    for (int32_t i = tid; i < count * nh; i += kMergeThreads) {
      const float mx = s_mstar[i % nh];
      s_m[i] = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[i] - mx);
    }
  }
  __syncthreads();
  const int32_t e = e0 + tid;
  if (e >= elems) return;
  const int32_t h = e / dv;
  const int32_t hh = h - h_lo;
  const int32_t c = e - h * dv;
  const float mx = s_mstar[hh];
  float acc = 0.f;
  for (int32_t p0 = 0; p0 < count; p0 += kMergeBatch) {
    float v[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int32_t p = min(p0 + u, count - 1);
      v[u] = a.ws_o[((first + p) * H + h) * dv + c];
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int32_t p = p0 + u;
      if (p < count) {
        const float w = staged ? s_m[p * nh + hh]
                               : ((mx == -INFINITY) ? 0.f
                                                    : __builtin_amdgcn_exp2f(
                                                          a.ws_m[(first + p) * H + h] - mx));
        acc = fmaf(v[u], w, acc);
      }
    }
  }
  const float l = s_lstar[hh];
  const int64_t orow = static_cast<int64_t>(b) * H + h;
  a.out[orow * dv + c] = (l > 0.f) ? acc / l : 0.f;
  if (c == 0 && a.lse != nullptr)
    a.lse[orow] = (l > 0.f) ? (mx + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, hipStream_t st) {
  const int32_t elems = s.num_q_heads * s.head_dim_v;
  dim3 grid(s.batch, (elems + kMergeThreads - 1) / kMergeThreads);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
