// select.hip -- per-stream keep sets: top-k (lsa_select_topk) and threshold
// with a dense fallback (lsa_select_threshold).
//
// Dimensionstp review, section 3-2-3 step 5: the keep mask comes from a top-k
// or a threshold; sections 4-3 and 5-1: exact-retrieval tasks need a
// threshold fallback.  One workgroup (a single wave for short streams) per
// stream runs the radix select of select_core.hpp over the stream's fp32
// scores.  The threshold set takes two launches: the first counts each
// stream's kept chunks (the chunks at or above the threshold, capped, or all
// of them when none passes), the second turns the counts into the CSR offsets
// -- every workgroup sums the counts of the streams before its own -- and
// writes the indices: all of them (fallback), the passing ones compacted in
// order (one block-wide scan), or, when the cap binds, the radix top-k.
#include "lsa_internal.hpp"
#include "select_core.hpp"
#include "table_check.hpp"

namespace lsa {
namespace {

// uni_n, uni_k > 0: every stream has uni_n chunks and keeps uni_k (the
// offsets are b * uni_n and b * uni_k, not read).
template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void select_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ chunk_off,
                                                        const int32_t* __restrict__ sel_off,
                                                        int32_t* __restrict__ sel_idx,
                                                        int32_t uni_n, int32_t uni_k) {
  __shared__ SelectLds<THREADS> lds;
  const int b = blockIdx.x;
  const int32_t base = uni_n > 0 ? b * uni_n : chunk_off[b];
  int32_t n = uni_n > 0 ? uni_n : chunk_off[b + 1] - base;
  const int32_t s0 = uni_k > 0 ? b * uni_k : sel_off[b];
  int32_t k = uni_k > 0 ? uni_k : sel_off[b + 1] - s0;
  if (n <= 0 || k <= 0) return;
  // violated preconditions (a stream longer than max_chunks, or k_b > N_b):
  // rank only the keys a block holds and never write past them, so the
  // result is still a deterministic function of the scores
  n = select_clamp_keys(n, THREADS * KPT);
  k = select_clamp_keys(k, n);
  int32_t* out = sel_idx + s0;
  if (k == n) {
    for (int32_t i = threadIdx.x; i < n; i += THREADS) out[i] = i;
    return;
  }
  select_topk_block<THREADS, KPT>(scores + base, n, k, out, lds);
}

// Sum of one value per thread over the THREADS threads (all must call it);
// s_part holds THREADS / 64 words used by this call only.
template <int THREADS>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* s_part) {
  const uint32_t w = wave_sum_u32(v);
  if (THREADS == kWave) return w;
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) s_part[wave] = w;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < THREADS / kWave; ++i) t += s_part[i];
  return t;
}

// Kept chunks of stream b under the threshold rule: c of the n chunks pass.
__device__ __forceinline__ int32_t threshold_keep(uint32_t c, int32_t n, int32_t max_keep) {
  if (c == 0) return n;
  const int32_t k = static_cast<int32_t>(c);
  return (max_keep > 0 && k > max_keep) ? max_keep : k;
}

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void threshold_count_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ chunk_off, float threshold,
    int32_t max_keep, int32_t* __restrict__ counts, int32_t* __restrict__ fallback) {
  __shared__ uint32_t s_part[THREADS / kWave];
  const int b = blockIdx.x;
  const int32_t base = chunk_off[b];
  // a stream longer than THREADS * KPT violates the shape: only its first
  // chunks are seen, so that nothing is read or written out of range
  const int32_t n = min(chunk_off[b + 1] - base, THREADS * KPT);
  uint32_t c = 0;
  if (n > 0) {
    uint32_t key[KPT];
    select_load_keys<THREADS, KPT>(scores + base, n, key);
    const uint32_t tkey = order_key(threshold);
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      c += (static_cast<int32_t>(threadIdx.x) * KPT + i < n && key[i] >= tkey) ? 1u : 0u;
  }
  c = block_sum<THREADS>(c, s_part);
  if (threadIdx.x == 0) {
    counts[b] = n > 0 ? threshold_keep(c, n, max_keep) : 0;
    if (fallback) fallback[b] = (n > 0 && c == 0) ? 1 : 0;
  }
}

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void threshold_write_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ chunk_off, float threshold,
    const int32_t* __restrict__ counts, int32_t B, int32_t* __restrict__ sel_off,
    int32_t* __restrict__ sel_idx) {
  __shared__ SelectLds<THREADS> lds;
  __shared__ uint32_t s_part[2][THREADS / kWave];
  const int b = blockIdx.x;
  uint32_t before = 0;
  for (int32_t j = threadIdx.x; j < b; j += THREADS) before += static_cast<uint32_t>(counts[j]);
  const int32_t off = static_cast<int32_t>(block_sum<THREADS>(before, s_part[0]));
  const int32_t k = counts[b];
  if (threadIdx.x == 0) {
    sel_off[b] = off;
    if (b == B - 1) sel_off[B] = off + k;
  }
  const int32_t base = chunk_off[b];
  const int32_t n = min(chunk_off[b + 1] - base, THREADS * KPT);
  if (n <= 0 || k <= 0) return;  // uniform over the workgroup
  int32_t* out = sel_idx + off;
  if (k >= n) {
    for (int32_t i = threadIdx.x; i < n; i += THREADS) out[i] = i;
    return;
  }
  uint32_t key[KPT];
  select_load_keys<THREADS, KPT>(scores + base, n, key);
  const uint32_t tkey = order_key(threshold);
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    c += (static_cast<int32_t>(threadIdx.x) * KPT + i < n && key[i] >= tkey) ? 1u : 0u;
  const uint32_t passing = block_sum<THREADS>(c, s_part[1]);
  if (passing == static_cast<uint32_t>(k)) {
    // the passing chunks in index order: thread t holds chunks [t*KPT, t*KPT+KPT)
    uint32_t pos, unused;
    select_exclusive_scan2<THREADS>(c, 0u, &pos, &unused, lds.tot);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int32_t idx = threadIdx.x * KPT + i;
      if (idx < n && key[i] >= tkey) out[pos++] = idx;
    }
    return;
  }
  select_topk_keys<THREADS, KPT>(key, n, k, out, lds);  // the cap binds: k < passing
}

template <int THREADS, int KPT>
hipError_t launch_threshold_t(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                              float threshold, int32_t max_keep, int32_t* sel_off,
                              int32_t* sel_idx, int32_t* fallback, int32_t* counts,
                              hipStream_t st) {
  hipLaunchKernelGGL((threshold_count_kernel<THREADS, KPT>), dim3(s.batch), dim3(THREADS), 0, st,
                     scores, chunk_off, threshold, max_keep, counts, fallback);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((threshold_write_kernel<THREADS, KPT>), dim3(s.batch), dim3(THREADS), 0, st,
                     scores, chunk_off, threshold, counts, s.batch, sel_off, sel_idx);
  return hipGetLastError();
}

template <int THREADS, int KPT>
hipError_t launch_select_t(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                           const int32_t* sel_off, int32_t* sel_idx, hipStream_t st) {
  const bool uni = (s.flags & LSA_SHAPE_UNIFORM) != 0;
  hipLaunchKernelGGL((select_kernel<THREADS, KPT>), dim3(s.batch), dim3(THREADS), 0, st, scores,
                     chunk_off, sel_off, sel_idx, uni ? s.max_chunks : 0, uni ? s.max_k : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_threshold(const lsa_shape& s, const float* scores,
                                   const int32_t* chunk_off, float threshold, int32_t max_keep,
                                   int32_t* sel_off, int32_t* sel_idx, int32_t* fallback,
                                   int32_t* counts, hipStream_t st) {
  const int32_t n = s.max_chunks;
#define LSA_THR(T_, K_)                                                                      \
  if (n <= (T_) * (K_))                                                                      \
    return launch_threshold_t<T_, K_>(s, scores, chunk_off, threshold, max_keep, sel_off,     \
                                      sel_idx, fallback, counts, st);
  LSA_THR(256, 1) LSA_THR(256, 4) LSA_THR(512, 4) LSA_THR(1024, 4) LSA_THR(1024, 8)
  LSA_THR(1024, 16) LSA_THR(1024, 32) LSA_THR(1024, 64)
#undef LSA_THR
  return hipErrorNotSupported;
}

// Four keys per thread (one 16-byte load) and as few waves as that allows up
// to 4096 chunks, then 1024 threads with more keys each (measured fastest for
// 2048 and 8192 chunks).
hipError_t launch_select(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                         const int32_t* sel_off, int32_t* sel_idx, hipStream_t st) {
  const int32_t n = s.max_chunks;
#define LSA_SEL(T_, K_) \
  if (n <= (T_) * (K_)) return launch_select_t<T_, K_>(s, scores, chunk_off, sel_off, sel_idx, st);
  LSA_SEL(256, 1) LSA_SEL(256, 4) LSA_SEL(512, 4) LSA_SEL(1024, 4) LSA_SEL(1024, 8)
  LSA_SEL(1024, 16) LSA_SEL(1024, 32) LSA_SEL(1024, 64)
#undef LSA_SEL
  return hipErrorNotSupported;
}

}  // namespace lsa
