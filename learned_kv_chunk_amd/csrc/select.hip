// select.hip -- per-stream top-k keep set.
//
// Dimensionstp review, section 3-2-3 step 5: the retriever's scores give a
// top-k keep mask over the chunks.  Ties go to the lower chunk index, NaN
// ranks below every number and -0.0 equals +0.0; kept indices are written in
// ascending order.
//
// One workgroup of 1024 threads per stream; thread t holds the KPT
// consecutive scores [t*KPT, t*KPT+KPT) in registers as order-preserving
// 32-bit keys.  An MSB-first radix select (four 8-bit digit passes over LDS
// histograms) finds the exact k-th largest key T and how many keys equal to T
// are needed.  The first pass sees few distinct digits (the sign and top
// exponent bits), so waves aggregate equal digits with ballots before one
// lane adds the count; later passes spread over many bins and add directly.
// A block-wide exclusive scan of (#keys > T, #keys == T) then gives each kept
// chunk its output position, which yields ascending indices and the
// lower-index tie rule without any sort.
#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;                 // NaN: below every number
  if ((u << 1) == 0u) u = 0u;            // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of two counters over the block.  Returns the exclusive
// prefixes; every thread must call it.
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* ea,
                                                      uint32_t* eb, uint32_t* s_tot) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t ya = __shfl_up(ia, off, kWave);
    uint32_t yb = __shfl_up(ib, off, kWave);
    if (lane >= off) {
      ia += ya;
      ib += yb;
    }
  }
  if (lane == kWave - 1) {
    s_tot[2 * wave] = ia;
    s_tot[2 * wave + 1] = ib;
  }
  __syncthreads();
  uint32_t ba = 0, bb = 0;
  for (int w = 0; w < wave; ++w) {
    ba += s_tot[2 * w];
    bb += s_tot[2 * w + 1];
  }
  *ea = ba + ia - a;
  *eb = bb + ib - b;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ chunk_off,
                                                            const int32_t* __restrict__ sel_off,
                                                            int32_t* __restrict__ sel_idx) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_tot[2 * kSelWaves];
  __shared__ uint32_t s_pick[2];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int32_t base = chunk_off[b];
  const int32_t n = chunk_off[b + 1] - base;
  int32_t k = sel_off[b + 1] - sel_off[b];
  if (n <= 0 || k <= 0) return;
  if (k > n) k = n;  // precondition violated: never write past the stream's range
  int32_t* out = sel_idx + sel_off[b];
  if (k == n) {  // every chunk kept
    for (int32_t i = tid; i < n; i += kSelThreads) out[i] = i;
    return;
  }

  uint32_t key[KPT];
  bool valid[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int32_t idx = tid * KPT + i;
    valid[i] = idx < n;
    key[i] = valid[i] ? order_key(scores[base + idx]) : 0u;
  }

  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = static_cast<uint32_t>(k);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool part = valid[i] && ((key[i] & mask) == prefix);
      const uint32_t d = (key[i] >> shift) & 0xffu;
      if (pass == 0) {
        uint64_t active = __ballot(part);
        while (active) {
          const int leader = __ffsll(static_cast<long long>(active)) - 1;
          const uint32_t ld = __shfl(d, leader, kWave);
          const uint64_t same = __ballot(part && d == ld) & active;
          if (lane == leader) atomicAdd(&hist[ld], static_cast<uint32_t>(__popcll(same)));
          active &= ~same;
        }
      } else if (part) {
        atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 4l..4l+3; count keys at or above each digit
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[4 * lane + j];
      const uint32_t tot = c[0] + c[1] + c[2] + c[3];
      uint32_t suffix = tot;  // inclusive sum over lanes >= this lane
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_down(suffix, off, kWave);
        if (lane + off < kWave) suffix += y;
      }
      uint32_t ge = suffix - tot;  // keys with a digit above this lane's four
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const uint32_t gt = ge;
        ge += c[j];
        if (gt < remaining && remaining <= ge) {
          s_pick[0] = 4u * lane + j;
          s_pick[1] = remaining - gt;
        }
      }
    }
    __syncthreads();
    prefix |= s_pick[0] << shift;
    mask |= 0xffu << shift;
    remaining = s_pick[1];
    __syncthreads();  // s_pick and hist are rewritten by the next pass
  }

  // prefix is the k-th largest key; `remaining` keys equal to it are kept.
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    n_gt += (valid[i] && key[i] > prefix) ? 1u : 0u;
    n_eq += (valid[i] && key[i] == prefix) ? 1u : 0u;
  }
  uint32_t gt_before, eq_before;
  block_exclusive_scan2(n_gt, n_eq, &gt_before, &eq_before, s_tot);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (!valid[i]) continue;
    const int32_t idx = tid * KPT + i;
    if (key[i] > prefix) {
      out[gt_before + min(eq_before, remaining)] = idx;
      ++gt_before;
    } else if (key[i] == prefix) {
      if (eq_before < remaining) out[gt_before + eq_before] = idx;
      ++eq_before;
    }
  }
}

}  // namespace

hipError_t launch_select(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                         const int32_t* sel_off, int32_t* sel_idx, hipStream_t st) {
  const int32_t per_thread = (s.max_chunks + kSelThreads - 1) / kSelThreads;
  dim3 grid(s.batch), block(kSelThreads);
#define LSA_SEL_CASE(K_)                                                                     \
  if (per_thread <= K_) {                                                                    \
    hipLaunchKernelGGL(select_kernel<K_>, grid, block, 0, st, scores, chunk_off, sel_off,    \
                       sel_idx);                                                             \
    return hipGetLastError();                                                                \
  }
  LSA_SEL_CASE(1) LSA_SEL_CASE(2) LSA_SEL_CASE(4) LSA_SEL_CASE(8) LSA_SEL_CASE(16)
  LSA_SEL_CASE(32) LSA_SEL_CASE(64)
#undef LSA_SEL_CASE
  return hipErrorNotSupported;
}

}  // namespace lsa
