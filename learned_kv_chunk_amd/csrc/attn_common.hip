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

#include <atomic>

#include "lsa_internal.hpp"

namespace lsa {

namespace {
constexpr int32_t kDefaultTarget = 256;  // compute units of an MI355X
constexpr int64_t kPortTilesPerWg = 4;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
}  // namespace

// The compute-unit count of each device is queried once and kept: a device
// attribute that never changes, so every later call (one per attention
// enqueue) costs only hipGetDevice.
int32_t device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int32_t> cached[kMaxDevices];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return kDefaultTarget;
  }
  const bool keep = dev >= 0 && dev < kMaxDevices;
  if (keep) {
    const int32_t c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    return kDefaultTarget;
  }
  if (keep) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

AttnPlan make_attn_plan(const lsa_shape& s, int32_t target) {
  AttnPlan p;
  p.tiles_per_chunk = (s.chunk_size + kTileTokens - 1) / kTileTokens;
  const int64_t total_tiles = s.total_k * p.tiles_per_chunk;
  p.target = target > 0 ? target : kDefaultTarget;
  // The vector-ALU kernel on small inputs: a workgroup of four waves gets
  // four tiles (one per wave) rather than one tile per CU, so that few
  // workgroups cover a short stream and it merges in its last one.  More
  // tiles per wave cost more than they save there (measured on the 4K-token
  // fp32 workload, 16 tiles: partial kernel 14.5 us with one tile per wave,
  // 22.4 with two, 37.9 with four).
  // With few tiles and at least five heads the waves of a workgroup share
  // each tile and split its heads instead (portable_split_heads): then one
  // tile per workgroup.
  p.split_heads = 0;
  if (!mqa_attn_supported(s) && !mla_attn_supported(s)) {
    p.split_heads = portable_split_heads(s, total_tiles, p.target) ? 1 : 0;
    const int64_t per_wg = p.split_heads ? 1 : kPortTilesPerWg;
    const int64_t want = (total_tiles + per_wg - 1) / per_wg;
    if (want < p.target) p.target = want > 0 ? static_cast<int32_t>(want) : 1;
  }
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

// The absorbed-MLA partials hold 64 heads x 512 columns each (128 KiB in
// fp32, a third of the KV bytes of a 1M-token step over 239 workgroups);
// rounding the unnormalised rows to bf16 halves what the partial kernel
// writes and the merge reads.  The rounding (at most 2^-9 relative per
// element, round to nearest even) is of the order of the one the kernel
// already applies to the attention weights before the P.V product; the
// maxima, the sums and every accumulation stay fp32.
bool partial_o_bf16(const lsa_shape& s) { return mla_attn_supported(s); }

PartialLayout partial_layout(const lsa_shape& s, const AttnPlan& p) {
  PartialLayout L;
  const size_t oes = partial_o_bf16(s) ? 2 : sizeof(float);
  const size_t rows = static_cast<size_t>(p.ws_rows) * static_cast<size_t>(s.num_q_heads);
  L.cnt_off = 0;  // same place for every shape (see kCounterStreams)
  L.m_off = static_cast<size_t>(kCounterStreams) * sizeof(int32_t);
  L.l_off = L.m_off + align256(rows * sizeof(float));
  L.o_off = L.l_off + align256(rows * sizeof(float));
  L.total = L.o_off + align256(rows * static_cast<size_t>(s.head_dim_v) * oes);
  return L;
}

namespace {

constexpr int kMergeBatch = 16;   // partials whose loads are in flight together
// most groups of partials a stream is cut into (fewer for the bf16 partials,
// whose group states take EPL words per lane in LDS)
template <int EPL>
constexpr int merge_groups() { return EPL == 1 ? 64 : 16; }

// (max, sum, output) state of a set of partials, log2 domain; EPL output
// elements per lane.
template <int EPL>
struct MergeState {
  float m, l, acc[EPL];
};

// Output elements ec .. ec + EPL - 1 of partial row `row`: one fp32 element,
// or (EPL = 2, bf16 partials) an aligned pair of bf16 in one 4-byte load.
template <int EPL>
__device__ __forceinline__ void load_partial(const AttnArgs& a, int64_t row, int32_t elems,
                                             int32_t ec, float (&v)[EPL]) {
  static_assert(EPL == 1 || EPL == 2, "one fp32 element or two bf16 elements per lane");
  if constexpr (EPL == 1) {
    v[0] = a.ws_o[row * elems + ec];
  } else {  // ec is even: the pair is one aligned 32-bit word
    const uint32_t w = *reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const uint16_t*>(a.ws_o) + (row * elems + ec));
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xffff0000u);
  }
}

// Folds partials [p_lo, p_hi) of the stream (rows first + p) into one state,
// kMergeBatch loads in flight and one rescale per batch.  HU: every lane of
// the wave has the same head h, so one load instruction brings a batch's
// sixteen maxima and sixteen sums (lane j < 16: m of partial j, lane 16 + j:
// its l) and lane reads hand them to the whole wave, instead of 32 loads of
// one value per wave (measured: 1 % more steps/s at 1 x 1M, 0.3-0.4 % on
// the MQA workloads).
template <bool HU, int EPL>
__device__ __forceinline__ MergeState<EPL> fold_partials(const AttnArgs& a, int64_t first,
                                                         int32_t p_lo, int32_t p_hi, int32_t h,
                                                         int32_t ec) {
  const int32_t H = a.H, elems = a.H * a.dv;
  MergeState<EPL> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) st.acc[i] = 0.f;
  for (int32_t p0 = p_lo; p0 < p_hi; p0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch][EPL];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      load_partial<EPL>(a, first + min(p0 + u, p_hi - 1), elems, ec, ov[u]);
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
#pragma unroll
    for (int i = 0; i < EPL; ++i) st.acc[i] *= f;
    st.l *= f;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (p0 + u < p_hi) {
        const float w = __builtin_amdgcn_exp2f(mv[u] - mu);
#pragma unroll
        for (int i = 0; i < EPL; ++i) st.acc[i] = fmaf(ov[u][i], w, st.acc[i]);
        st.l = fmaf(lv[u], w, st.l);
      }
    }
    st.m = mb;
  }
  return st;
}

// total <- total (+) g
template <int EPL>
__device__ __forceinline__ void combine_state(MergeState<EPL>& t, const MergeState<EPL>& g) {
  const float mx = fmaxf(t.m, g.m);
  const float mu = (mx == -INFINITY) ? 0.f : mx;
  const float ft = __builtin_amdgcn_exp2f(t.m - mu);
  const float fg = __builtin_amdgcn_exp2f(g.m - mu);
  t.l = fmaf(g.l, fg, t.l * ft);
#pragma unroll
  for (int i = 0; i < EPL; ++i) t.acc[i] = fmaf(g.acc[i], fg, t.acc[i] * ft);
  t.m = mx;
}

// One workgroup of MW waves per (stream, 64 * EPL consecutive output elements
// of the flattened [H][dv] row); lane i owns elements EPL i .. EPL i + EPL - 1
// of the block (EPL = 2 for bf16 partials, one 4-byte load per partial).  A
// stream's partials are cut into groups (16, or more per group when a stream
// has over 1024 partials, so that there are at most 64 groups); each group is
// folded into one state, kMergeBatch partials per round trip with one rescale
// per batch, and the group states are combined in group order.  With MW
// waves, wave w folds groups w, w + MW, ... and the states meet in LDS; with
// one wave the combine runs as the groups are folded.  The arithmetic is the
// same for every MW and depends only on the plan, so reruns are bit-identical
// and a stream's result does not depend on the launch shape the batch selects.
template <int MW, bool HU, int EPL>
__global__ __launch_bounds__(MW * kWave) void merge_kernel(AttnArgs a, int32_t nblk) {
  constexpr int kGroups = merge_groups<EPL>();
  __shared__ float s_state[MW > 1 ? 2 + EPL : 1][MW > 1 ? kGroups : 1][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int32_t b = static_cast<int32_t>(blockIdx.x) / nblk;
  const int32_t blk = static_cast<int32_t>(blockIdx.x) - b * nblk;
  const int32_t H = a.H, dv = a.dv;
  const int32_t elems = H * dv;
  const int32_t e = (blk * kWave + lane) * EPL;
  const int32_t ec = min(e, elems - EPL);
  const int32_t h = ec / dv;

  int32_t first, count;
  stream_wg_range(SelCsr{a.sel_off, a.uni_k, a.uni_wgs, a.uni_per}, a.B, b, a.tiles_per_chunk,
                  a.per, a.target, &first, &count);
  const int32_t gs = max(kMergeBatch, ceil_div_i(count, kGroups));
  const int32_t ngroups = ceil_div_i(count, gs);

  MergeState<EPL> total;
  total.m = -INFINITY;
  total.l = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) total.acc[i] = 0.f;
  if (MW == 1) {
    for (int32_t g = 0; g < ngroups; ++g)
      combine_state(total,
                    fold_partials<HU, EPL>(a, first, g * gs, min(count, (g + 1) * gs), h, ec));
  } else {
    for (int32_t g = wave; g < ngroups; g += MW) {
      const MergeState<EPL> st =
          fold_partials<HU, EPL>(a, first, g * gs, min(count, (g + 1) * gs), h, ec);
      s_state[0][g][lane] = st.m;
      s_state[1][g][lane] = st.l;
#pragma unroll
      for (int i = 0; i < EPL; ++i) s_state[2 + i][g][lane] = st.acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int32_t g = 0; g < ngroups; ++g) {
      MergeState<EPL> st;
      st.m = s_state[0][g][lane];
      st.l = s_state[1][g][lane];
#pragma unroll
      for (int i = 0; i < EPL; ++i) st.acc[i] = s_state[2 + i][g][lane];
      combine_state(total, st);
    }
  }
  if (e >= elems) return;
  const int64_t orow = static_cast<int64_t>(b) * H + h;
  const int32_t c = e - h * dv;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    a.out[orow * dv + c + i] = (total.l > 0.f) ? total.acc[i] / total.l : 0.f;
  if (c == 0 && a.lse != nullptr)
    a.lse[orow] = (total.l > 0.f) ? (total.m + log2f(total.l)) * 0.69314718055994530942f
                                  : -INFINITY;
}

__global__ __launch_bounds__(256) void clear_counters_kernel(int32_t* counters) {
  const int32_t i = static_cast<int32_t>(blockIdx.x) * 256 + static_cast<int32_t>(threadIdx.x);
  if (i < kCounterStreams) counters[i] = 0;
}

}  // namespace

hipError_t launch_clear_counters(void* ws, hipStream_t st) {
  hipLaunchKernelGGL(clear_counters_kernel, dim3((kCounterStreams + 255) / 256), dim3(256), 0, st,
                     static_cast<int32_t*>(ws));
  return hipGetLastError();
}

hipError_t launch_attn_merge(const lsa_shape& s, const AttnArgs& a, const AttnPlan& plan,
                             hipStream_t st) {
  // one wave per workgroup while a stream has a couple of groups of partials
  // on average, eight when streams have many (a long single stream)
  const bool one = plan.grid <= static_cast<int64_t>(2 * kMergeBatch) * s.batch;
  // a block of 64 output elements lies inside one head when dv is a multiple of 64
  const bool hu = s.head_dim_v % kWave == 0;
  if (a.o_bf16) {
    // bf16 partials: two elements per lane (one 4-byte load per partial), a
    // block of 128 inside one head; sixteen waves, so that each folds one
    // group of a long stream.  Measured at 1 x 1M (239 partials, attention
    // phase, interleaved on one box): 34.0 us with eight waves, 33.5 with
    // sixteen, the same with four elements per lane, 35.5 with eight.
    constexpr int EPL = 2;
    if (s.head_dim_v % (EPL * kWave) != 0) return hipErrorNotSupported;
    const int32_t nblk = s.num_q_heads * s.head_dim_v / (EPL * kWave);
    const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(nblk) * s.batch));
    if (one)
      hipLaunchKernelGGL((merge_kernel<1, true, EPL>), g, dim3(kWave), 0, st, a, nblk);
    else
      hipLaunchKernelGGL((merge_kernel<16, true, EPL>), g, dim3(16 * kWave), 0, st, a, nblk);
    return hipGetLastError();
  }
  const int32_t nblk = (s.num_q_heads * s.head_dim_v + kWave - 1) / kWave;
  const dim3 g(static_cast<uint32_t>(static_cast<int64_t>(nblk) * s.batch));
  if (one && hu)
    hipLaunchKernelGGL((merge_kernel<1, true, 1>), g, dim3(kWave), 0, st, a, nblk);
  else if (one)
    hipLaunchKernelGGL((merge_kernel<1, false, 1>), g, dim3(kWave), 0, st, a, nblk);
  else if (hu)
    hipLaunchKernelGGL((merge_kernel<8, true, 1>), g, dim3(8 * kWave), 0, st, a, nblk);
  else
    hipLaunchKernelGGL((merge_kernel<8, false, 1>), g, dim3(8 * kWave), 0, st, a, nblk);
  return hipGetLastError();
}

}  // namespace lsa
