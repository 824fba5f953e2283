// score.hip -- chunk scoring: one dual-encoder inner product per chunk.
//
// Dimensionstp review, sections 2-1 and 3-2-4, and the wiki note's "Key
// points": the memory indexer is a dual encoder, so a chunk's relevance is
// the inner product of the stream's query embedding and the chunk embedding.
//
// A batched GEMV streamed from HBM (1 flop per byte: no MFMA).  A group of G
// lanes owns one embedding row; lane i of the group reads the row's 16-byte
// vectors i, i+G, ..., so each wave load instruction covers 64/G whole rows
// with consecutive addresses.  The query's matching vectors stay in
// registers for the whole workgroup, partial dots are reduced across the
// group with lane shuffles, and the group's first lane writes the fp32 score.
// Grid: (row blocks, B); workgroups past the end of a stream exit at once.
#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScorePasses = 4;  // rows per group per workgroup (loads in flight)

template <typename T>
struct Vec16 {
  static constexpr int kElems = 16 / sizeof(T);
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen(const u32x4& v, float* f, float) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ void widen(const u32x4& v, float* f, uint16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// T: float or uint16_t (bf16 bits).  G lanes per row, NV vectors per lane.
template <typename T, int G, int NV>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const T* __restrict__ q, const T* __restrict__ emb, const int32_t* __restrict__ chunk_off,
    float* __restrict__ scores, int32_t D) {
  constexpr int E = Vec16<T>::kElems;
  constexpr int kGroups = kScoreThreads / G;
  constexpr int kRowsPerBlock = kGroups * kScorePasses;
  const int b = blockIdx.y;
  const int32_t r_end = chunk_off[b + 1];
  const int32_t r_begin = chunk_off[b] + static_cast<int32_t>(blockIdx.x) * kRowsPerBlock;
  if (r_begin >= r_end) return;

  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;

  float qf[NV][E];
  const u32x4* qrow = reinterpret_cast<const u32x4*>(q + static_cast<int64_t>(b) * D);
#pragma unroll
  for (int i = 0; i < NV; ++i) widen(qrow[gl + i * G], qf[i], T());

  u32x4 ev[kScorePasses][NV];
#pragma unroll
  for (int p = 0; p < kScorePasses; ++p) {
    const int32_t row = r_begin + p * kGroups + grp;
    const u32x4* erow = reinterpret_cast<const u32x4*>(emb + static_cast<int64_t>(row) * D);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      ev[p][i] = (row < r_end) ? __builtin_nontemporal_load(erow + gl + i * G) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int p = 0; p < kScorePasses; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float ef[E];
      widen(ev[p][i], ef, T());
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(qf[i][e], ef[e], acc);
    }
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, G);
    const int32_t row = r_begin + p * kGroups + grp;
    if (gl == 0 && row < r_end) scores[row] = acc;
  }
}

template <typename T, int G, int NV>
hipError_t launch_score_t(const lsa_shape& s, const void* q, const void* emb,
                          const int32_t* chunk_off, float* scores, hipStream_t st) {
  constexpr int kRowsPerBlock = (kScoreThreads / G) * kScorePasses;
  const int32_t blocks = (s.max_chunks + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks == 0) return hipSuccess;
  dim3 grid(blocks, s.batch);
  hipLaunchKernelGGL((score_kernel<T, G, NV>), grid, dim3(kScoreThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(emb), chunk_off, scores,
                     s.index_dim);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_score(const lsa_shape& s, const void* q, const void* emb,
                          const int32_t* chunk_off, float* scores, hipStream_t st) {
  const int rv = s.index_dim / Vec16<T>::kElems;  // 16-byte vectors per row
  // G = largest power of two <= 32 dividing rv; NV = rv / G in {1, 2, 4}
  int g = 1;
  while (g < 32 && rv % (2 * g) == 0) g *= 2;
  const int nv = rv / g;
#define LSA_SCORE_CASE(G_, NV_) \
  if (g == G_ && nv == NV_) return launch_score_t<T, G_, NV_>(s, q, emb, chunk_off, scores, st);
  LSA_SCORE_CASE(1, 1) LSA_SCORE_CASE(2, 1) LSA_SCORE_CASE(4, 1) LSA_SCORE_CASE(8, 1)
  LSA_SCORE_CASE(16, 1) LSA_SCORE_CASE(32, 1) LSA_SCORE_CASE(32, 2) LSA_SCORE_CASE(32, 3) LSA_SCORE_CASE(32, 4)
  LSA_SCORE_CASE(1, 3) LSA_SCORE_CASE(2, 3) LSA_SCORE_CASE(4, 3) LSA_SCORE_CASE(8, 3)
  LSA_SCORE_CASE(16, 3) LSA_SCORE_CASE(1, 5) LSA_SCORE_CASE(2, 5) LSA_SCORE_CASE(4, 5)
  LSA_SCORE_CASE(8, 5) LSA_SCORE_CASE(16, 5) LSA_SCORE_CASE(1, 7) LSA_SCORE_CASE(2, 7)
  LSA_SCORE_CASE(4, 7) LSA_SCORE_CASE(8, 7) LSA_SCORE_CASE(16, 7)
#undef LSA_SCORE_CASE
  return hipErrorNotSupported;
}

}  // namespace

bool score_supported(const lsa_shape& s) {
  const int esz = s.dtype == LSA_DTYPE_BF16 ? 2 : 4;
  if (s.index_dim <= 0 || s.index_dim > 1024 || (s.index_dim * esz) % 16 != 0) return false;
  const int rv = s.index_dim * esz / 16;
  int g = 1;
  while (g < 32 && rv % (2 * g) == 0) g *= 2;
  const int nv = rv / g;
  if (g == 32) return nv >= 1 && nv <= 4;
  return nv == 1 || nv == 3 || nv == 5 || nv == 7;
}

hipError_t launch_score(const lsa_shape& s, const void* q, const void* emb,
                        const int32_t* chunk_off, float* scores, hipStream_t st) {
  if (s.dtype == LSA_DTYPE_BF16)
    return dispatch_score<uint16_t>(s, q, emb, chunk_off, scores, st);
  return dispatch_score<float>(s, q, emb, chunk_off, scores, st);
}

}  // namespace lsa
