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
// registers, partial dots are reduced across the group with DPP row
// operations and a lane swap (group_sum: no trip through the LDS crossbar),
// and the group's first lane writes the fp32 score.  Grid: (row blocks, B);
// workgroups past the end of a stream exit at once.

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kScoreThreads = 256;
// Rows per group per workgroup.  One: more, smaller workgroups spread the
// short cold read over every CU sooner (measured decode steps/s, interleaved
// A/B: from 4 rows to 2 +0.4 % at 16 x 128K and +0.6 % at 1 x 1M, from 2 to
// 1 another +0.5 % and +0.3 %; 8 rows 1 % slower than 4).
constexpr int kScorePasses = 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec16 {
  static constexpr int kElems = 16 / sizeof(T);
};

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

// Scores of rows [r_begin, min(r_begin + rows per block, r_end)) of stream b.
template <typename T, int G, int NV>
__device__ __forceinline__ void score_rows(const T* __restrict__ q, const T* __restrict__ emb,
                                           float* __restrict__ scores, int32_t D, int b,
                                           int32_t r_begin, int32_t r_end) {
  constexpr int E = Vec16<T>::kElems;
  constexpr int kGroups = kScoreThreads / G;
  const int tid = threadIdx.x;
  const int grp = tid / G;
  const int gl = tid % G;

  // embedding loads first, then the (cache-resident) query vectors
  u32x4 ev[kScorePasses][NV];
#pragma unroll
  for (int p = 0; p < kScorePasses; ++p) {
    const int32_t row = min(r_begin + p * kGroups + grp, r_end - 1);
    const u32x4* erow = reinterpret_cast<const u32x4*>(emb + static_cast<int64_t>(row) * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) ev[p][i] = __builtin_nontemporal_load(erow + gl + i * G);
  }
  float qf[NV][E];
  const u32x4* qrow = reinterpret_cast<const u32x4*>(q + static_cast<int64_t>(b) * D);
#pragma unroll
  for (int i = 0; i < NV; ++i) widen(qrow[gl + i * G], qf[i], T());
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
    acc = group_sum<G>(acc);
    const int32_t row = r_begin + p * kGroups + grp;
    if (gl == 0 && row < r_end) scores[row] = acc;
  }
}

// uni_n > 0: every stream has uni_n chunks (chunk_off[b] = b * uni_n, not read).
template <typename T, int G, int NV>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const T* __restrict__ q, const T* __restrict__ emb, const int32_t* __restrict__ chunk_off,
    float* __restrict__ scores, int32_t D, int32_t uni_n) {
  constexpr int kRowsPerBlock = (kScoreThreads / G) * kScorePasses;
  const int b = blockIdx.y;
  const int32_t r0 = uni_n > 0 ? b * uni_n : chunk_off[b];
  const int32_t r_end = uni_n > 0 ? r0 + uni_n : chunk_off[b + 1];
  const int32_t r_begin = r0 + static_cast<int32_t>(blockIdx.x) * kRowsPerBlock;
  if (r_begin >= r_end) return;
  score_rows<T, G, NV>(q, emb, scores, D, b, r_begin, r_end);
}

bool score_geometry(const lsa_shape& s, int* g, int* nv) {
  const int esz = s.dtype == LSA_DTYPE_BF16 ? 2 : 4;
  if (s.index_dim <= 0 || (s.index_dim * esz) % 16 != 0) return false;
  const int rv = s.index_dim * esz / 16;  // 16-byte vectors per row
  if (rv & (rv - 1)) return false;        // power of two
  if (rv < 4 || rv > 128) return false;
  *g = rv < 32 ? rv : 32;
  *nv = rv / *g;
  return true;
}

template <typename T, int G, int NV>
hipError_t launch_score_t(const lsa_shape& s, const void* q, const void* emb,
                          const int32_t* chunk_off, float* scores, hipStream_t st) {
  constexpr int kRowsPerBlock = (kScoreThreads / G) * kScorePasses;
  dim3 grid((s.max_chunks + kRowsPerBlock - 1) / kRowsPerBlock, s.batch);
  hipLaunchKernelGGL((score_kernel<T, G, NV>), grid, dim3(kScoreThreads), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(emb), chunk_off, scores,
                     s.index_dim, (s.flags & LSA_SHAPE_UNIFORM) ? s.max_chunks : 0);
  return hipGetLastError();
}

#define LSA_SCORE_GEOMETRIES(X) X(4, 1) X(8, 1) X(16, 1) X(32, 1) X(32, 2) X(32, 4)

template <typename T>
hipError_t dispatch_score(const lsa_shape& s, const void* q, const void* emb,
                          const int32_t* chunk_off, float* scores, hipStream_t st) {
  int g = 0, nv = 0;
  if (!score_geometry(s, &g, &nv)) return hipErrorNotSupported;
#define LSA_SCORE_CASE(G_, NV_) \
  if (g == G_ && nv == NV_) return launch_score_t<T, G_, NV_>(s, q, emb, chunk_off, scores, st);
  LSA_SCORE_GEOMETRIES(LSA_SCORE_CASE)
#undef LSA_SCORE_CASE
  return hipErrorNotSupported;
}

}  // namespace

bool score_supported(const lsa_shape& s) {
  int g, nv;
  return score_geometry(s, &g, &nv);
}

hipError_t launch_score(const lsa_shape& s, const void* q, const void* emb,
                        const int32_t* chunk_off, float* scores, hipStream_t st) {
  if (s.dtype == LSA_DTYPE_BF16) return dispatch_score<uint16_t>(s, q, emb, chunk_off, scores, st);
  return dispatch_score<float>(s, q, emb, chunk_off, scores, st);
}

}  // namespace lsa
