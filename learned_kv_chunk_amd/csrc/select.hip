// select.hip -- standalone per-stream top-k keep set (lsa_select_topk).
//
// Dimensionstp review, section 3-2-3 step 5: keep the top-k chunks of each
// stream.  One workgroup (a single wave for short streams) per stream runs
// the radix select of select_core.hpp over the stream's fp32 scores.
#include "lsa_internal.hpp"
#include "select_core.hpp"

namespace lsa {
namespace {

template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void select_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ chunk_off,
                                                        const int32_t* __restrict__ sel_off,
                                                        int32_t* __restrict__ sel_idx) {
  __shared__ SelectLds<THREADS> lds;
  const int b = blockIdx.x;
  const int32_t base = chunk_off[b];
  const int32_t n = chunk_off[b + 1] - base;
  int32_t k = sel_off[b + 1] - sel_off[b];
  if (n <= 0 || k <= 0) return;
  if (k > n) k = n;  // violated precondition: never write past the stream's range
  int32_t* out = sel_idx + sel_off[b];
  if (k == n) {
    for (int32_t i = threadIdx.x; i < n; i += THREADS) out[i] = i;
    return;
  }
  select_topk_block<THREADS, KPT>(scores + base, n, k, out, lds);
}

template <int THREADS, int KPT>
hipError_t launch_select_t(const lsa_shape& s, const float* scores, const int32_t* chunk_off,
                           const int32_t* sel_off, int32_t* sel_idx, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<THREADS, KPT>), dim3(s.batch), dim3(THREADS), 0, st, scores,
                     chunk_off, sel_off, sel_idx);
  return hipGetLastError();
}

}  // namespace

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
