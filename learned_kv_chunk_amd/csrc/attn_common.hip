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

constexpr int kMergeBatch = 16;   // partials whose loads are in flight together
constexpr int kMergeGroups = 64;  // most groups of partials a stream is cut into

// (max, sum, output) state of a set of partials, log2 domain.
struct MergeState {
  float m, l, acc;
};

// Folds partials [p_lo, p_hi) of the stream (rows first + p) into one state,
// kMergeBatch loads in flight and one rescale per batch.  HU: every lane of
// the wave has the same head h, so one load instruction brings a batch's
// sixteen maxima and sixteen sums (lane j < 16: m of partial j, lane 16 + j:
// its l) and lane reads hand them to the whole wave, instead of 32 loads of
// one value per wave (measured: 1 % more steps/s at 1 x 1M, 0.3-0.4 % on
// the MQA workloads).
template <bool HU>
__device__ __forceinline__ MergeState fold_partials(const AttnArgs& a, int64_t first,
                                                    int32_t p_lo, int32_t p_hi, int32_t h,
                                                    int32_t ec) {
  const int32_t H = a.H, elems = a.H * a.dv;
  MergeState st = {-INFINITY, 0.f, 0.f};
  for (int32_t p0 = p_lo; p0 < p_hi; p0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      ov[u] = a.ws_o[(first + min(p0 + u, p_hi - 1)) * elems + ec];
    if (HU) {
      const int lane = threadIdx.x & (kWave - 1);
      const int j = lane & (kMergeBatch - 1);
      const int64_t rj = first + min(p0 + j, p_hi - 1);
      const float* src = (lane & kMergeBatch) ? a.ws_l : a.ws_m;
      const int ml = __float_as_int(src[rj * H + h]);
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        mv[u] = __int_as_float(__builtin_amdgcn_readlane(ml, u));
        lv[u] = __int_as_float(__builtin_amdgcn_readlane(ml, kMergeBatch + u));
      }
    } else {
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int64_t row = first + min(p0 + u, p_hi - 1);
        mv[u] = a.ws_m[row * H + h];
        lv[u] = a.ws_l[row * H + h];
      }
    }
    float mb = st.m;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (p0 + u < p_hi) mb = fmaxf(mb, mv[u]);
    const float mu = (mb == -INFINITY) ? 0.f : mb;
    const float f = __builtin_amdgcn_exp2f(st.m - mu);
    st.acc *= f;
    st.l *= f;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (p0 + u < p_hi) {
        const float w = __builtin_amdgcn_exp2f(mv[u] - mu);
        st.acc = fmaf(ov[u], w, st.acc);
        st.l = fmaf(lv[u], w, st.l);
      }
    }
    st.m = mb;
  }
  return st;
}

// total <- total (+) g
__device__ __forceinline__ void combine_state(MergeState& t, const MergeState& g) {
  const float mx = fmaxf(t.m, g.m);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  const float ft = __builtin_amdgcn_exp2f(t.m - mu);
  const float fg = __builtin_amdgcn_exp2f(g.m - mu);
  t.l = fmaf(g.l, fg, t.l * ft);
  t.acc = fmaf(g.acc, fg, t.acc * ft);
  t.m = mx;
}

// One workgroup of MW waves per (stream, 64 consecutive output elements of the
// flattened [H][dv] row); lane i owns element i of the block.  A stream's
// partials are cut into groups (16, or more per group when a stream has over
// 1024 partials, so that there are at most 64 groups); each group is folded
// into one state, kMergeBatch partials per round trip with one rescale per
// batch, and the group states are combined in group order.  With MW waves,
// wave w folds groups w, w + MW, ... and the states meet in LDS; with one
// wave the combine runs as the groups are folded.  The arithmetic is the same
// for every MW and depends only on the plan, so reruns are bit-identical and
// a stream's result does not depend on the launch shape the batch selects.
template <int MW, bool HU>
__global__ __launch_bounds__(MW * kWave) void merge_kernel(AttnArgs a, int32_t nblk) {
  __shared__ float s_state[MW > 1 ? 3 : 1][MW > 1 ? kMergeGroups : 1][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int32_t b = static_cast<int32_t>(blockIdx.x) / nblk;
  const int32_t blk = static_cast<int32_t>(blockIdx.x) - b * nblk;
  const int32_t H = a.H, dv = a.dv;
  const int32_t elems = H * dv;
  const int32_t e = blk * kWave + lane;
  const int32_t ec = min(e, elems - 1);
  const int32_t h = ec / dv;

  int32_t first, count;
  stream_wg_range(SelCsr{a.sel_off, a.uni_k}, a.B, b, a.tiles_per_chunk, a.per, a.target,
                  &first, &count);
  const int32_t gs = max(kMergeBatch, ceil_div_i(count, kMergeGroups));
  const int32_t ngroups = ceil_div_i(count, gs);

  MergeState total = {-INFINITY, 0.f, 0.f};
  if (MW == 1) {
    for (int32_t g = 0; g < ngroups; ++g)
      combine_state(total, fold_partials<HU>(a, first, g * gs, min(count, (g + 1) * gs), h, ec));
  } else {
    for (int32_t g = wave; g < ngroups; g += MW) {
      const MergeState st = fold_partials<HU>(a, first, g * gs, min(count, (g + 1) * gs), h, ec);
      s_state[0][g][lane] = st.m;
      s_state[1][g][lane] = st.l;
      s_state[2][g][lane] = st.acc;
    }
    __syncthreads();
    if (wave != 0) return;
    for (int32_t g = 0; g < ngroups; ++g)
      combine_state(total, MergeState{s_state[0][g][lane], s_state[1][g][lane],
                                      s_state[2][g][lane]});
  }
  if (e >= elems) return;
  const int64_t orow = static_cast<int64_t>(b) * H + h;
  const int32_t c = e - h * dv;
  a.out[orow * dv + c] = (total.l > 0.f) ? total.acc / total.l : 0.f;
  if (c == 0 && a.lse != nullptr)
    a.lse[orow] = (total.l > 0.f) ? (total.m + log2f(total.l)) * 0.69314718055994530942f
                                  : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, hipStream_t st) {
  const int32_t nblk = (s.num_q_heads * s.head_dim_v + kWave - 1) / kWave;
  const int64_t grid = static_cast<int64_t>(nblk) * s.batch;
  // one wave per workgroup while a stream has a couple of groups of partials
  // on average, eight when streams have many (a long single stream)
  const AttnPlan plan = make_attn_plan(s, a.target);
  const bool one = plan.grid <= static_cast<int64_t>(2 * kMergeBatch) * s.batch;
  // a block of 64 output elements lies inside one head when dv is a multiple of 64
  const bool hu = s.head_dim_v % kWave == 0;
  const dim3 g(static_cast<uint32_t>(grid));
  if (one && hu)
    hipLaunchKernelGGL((merge_kernel<1, true>), g, dim3(kWave), 0, st, a, nblk);
  else if (one)
    hipLaunchKernelGGL((merge_kernel<1, false>), g, dim3(kWave), 0, st, a, nblk);
  else if (hu)
    hipLaunchKernelGGL((merge_kernel<8, true>), g, dim3(8 * kWave), 0, st, a, nblk);
  else
    hipLaunchKernelGGL((merge_kernel<8, false>), g, dim3(8 * kWave), 0, st, a, nblk);
  return hipGetLastError();
}

}  // namespace lsa
