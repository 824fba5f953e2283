// residency.hip -- delta residency of the chunk pool over a host-memory
// backing store (lsa_pool_delta_update).
//
// Wiki note flowchart: only the selected chunks stay resident on the GPU; the
// rest of the cache lives in host memory and chunks move between the two as
// the selection changes.  Dimensionstp review section 3-2-5: that swap engine
// is not released, so the slot rule here is this library's own: a slot whose
// chunk is still kept keeps it, and the newly kept chunks (ascending) go to
// the freed slots (ascending).  Only those chunks cross the host link.
//
// Two launches.  The first (one workgroup per stream) marks the new kept set
// and the chunks the slots already hold in LDS bitmaps, numbers the freed
// slots and the chunks to load with block-wide scans, and rewrites the slot
// table.  The second (one workgroup per (load, stream)) copies each loaded
// chunk's rows straight from page-locked host memory into its pool slot with
// 16-byte loads, zero-filling rows past the end of the stream.
#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDeltaThreads = 1024;
constexpr int kDeltaWaves = kDeltaThreads / kWave;
constexpr int kMaxStreamChunks = 65536;             // per stream
constexpr int kBitmapWords = kMaxStreamChunks / 32;
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__device__ __forceinline__ bool test_bit(const uint32_t* bm, int32_t c) {
  return (bm[c >> 5] >> (c & 31)) & 1u;
}

// Exclusive scan of one count per thread over the workgroup, plus the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_part,
                                                         uint32_t* total) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_part[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kDeltaWaves; ++w) {
    const uint32_t t = s_part[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();  // s_part is reused by the next call
  *total = all;
  return before + incl - v;
}

__global__ __launch_bounds__(kDeltaThreads) void pool_delta_kernel(
    const int32_t* __restrict__ chunk_off, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_off, int32_t* __restrict__ table, int32_t* __restrict__ loads,
    int32_t* __restrict__ load_count) {
  __shared__ uint32_t s_wanted[kBitmapWords];
  __shared__ uint32_t s_held[kBitmapWords];
  __shared__ uint32_t s_part[kDeltaWaves];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t n = min(chunk_off[b + 1] - chunk_off[b], kMaxStreamChunks);
  const int32_t s0 = sel_off[b];
  const int32_t k = max(sel_off[b + 1] - s0, 0);
  const int32_t words = (max(n, 0) + 31) / 32;
  for (int32_t i = tid; i < words; i += kDeltaThreads) {
    s_wanted[i] = 0u;
    s_held[i] = 0u;
  }
  __syncthreads();
  for (int32_t j = tid; j < k; j += kDeltaThreads) {
    const int32_t c = sel_idx[s0 + j];
    if (c >= 0 && c < n) atomicOr(&s_wanted[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  // a slot keeps its chunk when the chunk is still wanted (the first slot
  // holding it, should the old table repeat a chunk); rounds of kDeltaThreads
  // consecutive slots number the freed ones in slot order
  uint32_t n_free = 0;
  for (int32_t p0 = 0; p0 < k; p0 += kDeltaThreads) {
    const int32_t p = p0 + tid;
    bool freed = false;
    if (p < k) {
      const int32_t c = table[s0 + p];
      bool keep = c >= 0 && c < n && test_bit(s_wanted, c);
      if (keep) {
        const uint32_t bit = 1u << (c & 31);
        keep = (atomicOr(&s_held[c >> 5], bit) & bit) == 0u;
      }
      freed = !keep;
    }
    uint32_t round_total;
    const uint32_t rank = n_free + block_exclusive_scan(freed ? 1u : 0u, s_part, &round_total);
    if (freed) loads[s0 + rank] = s0 + p;  // the rank-th freed slot
    n_free += round_total;
  }
  __syncthreads();  // freed-slot list and held bitmap complete
  // the chunks to load, in chunk order, take the freed slots in slot order
  uint32_t n_load = 0;
  for (int32_t j0 = 0; j0 < k; j0 += kDeltaThreads) {
    const int32_t j = j0 + tid;
    int32_t c = -1;
    bool need = false;
    if (j < k) {
      c = sel_idx[s0 + j];
      need = c >= 0 && c < n && !test_bit(s_held, c);
    }
    uint32_t round_total;
    const uint32_t rank = n_load + block_exclusive_scan(need ? 1u : 0u, s_part, &round_total);
    if (need && rank < n_free) table[loads[s0 + rank]] = c;
    n_load += round_total;
  }
  const uint32_t used = min(n_load, n_free);
  for (uint32_t r = used + tid; r < n_free; r += kDeltaThreads) table[loads[s0 + r]] = -1;
  if (tid == 0) load_count[b] = static_cast<int32_t>(used);
}

__device__ __forceinline__ void copy_rows(const char* __restrict__ src, char* __restrict__ dst,
                                          int64_t valid_bytes, int64_t total_bytes) {
  constexpr int64_t kStep = static_cast<int64_t>(kCopyThreads) * 16;
  for (int64_t off0 = static_cast<int64_t>(threadIdx.x) * 16; off0 < total_bytes;
       off0 += kStep * kCopyUnroll) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t off = off0 + u * kStep;
      v[u] = (off < valid_bytes) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off))
                                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t off = off0 + u * kStep;
      if (off < total_bytes) *reinterpret_cast<u32x4*>(dst + off) = v[u];
    }
  }
}

__global__ __launch_bounds__(kCopyThreads) void pool_load_kernel(
    const char* __restrict__ k_host, int32_t k_row_bytes, const char* __restrict__ v_host,
    int32_t v_row_bytes, const int64_t* __restrict__ tok_off, const int32_t* __restrict__ sel_off,
    const int32_t* __restrict__ table, const int32_t* __restrict__ loads,
    const int32_t* __restrict__ load_count, char* __restrict__ k_pool, char* __restrict__ v_pool,
    int32_t C) {
  const int b = blockIdx.y;
  const int32_t j = blockIdx.x;
  if (j >= load_count[b]) return;
  const int64_t slot = loads[sel_off[b] + j];
  const int64_t n = table[slot];
  const int64_t len = tok_off[b + 1] - tok_off[b];
  int64_t valid = len - n * C;
  if (n < 0 || valid < 0) valid = 0;
  if (valid > C) valid = C;
  const int64_t row0 = tok_off[b] + n * C;
  copy_rows(k_host + row0 * k_row_bytes, k_pool + slot * C * k_row_bytes, valid * k_row_bytes,
            static_cast<int64_t>(C) * k_row_bytes);
  if (v_pool != nullptr)
    copy_rows(v_host + row0 * v_row_bytes, v_pool + slot * C * v_row_bytes, valid * v_row_bytes,
              static_cast<int64_t>(C) * v_row_bytes);
}

}  // namespace

int32_t pool_delta_max_stream_chunks() { return kMaxStreamChunks; }

hipError_t launch_pool_delta(const lsa_shape& s, const void* k_host_dev, int32_t k_row_bytes,
                             const void* v_host_dev, int32_t v_row_bytes,
                             const int64_t* tok_off, const int32_t* chunk_off,
                             const int32_t* sel_idx, const int32_t* sel_off, int32_t* table,
                             int32_t* loads, int32_t* load_count, void* k_pool, void* v_pool,
                             hipStream_t st) {
  hipLaunchKernelGGL(pool_delta_kernel, dim3(s.batch), dim3(kDeltaThreads), 0, st, chunk_off,
                     sel_idx, sel_off, table, loads, load_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pool_load_kernel, dim3(s.max_k, s.batch), dim3(kCopyThreads), 0, st,
                     static_cast<const char*>(k_host_dev), k_row_bytes,
                     static_cast<const char*>(v_host_dev), v_row_bytes, tok_off, sel_off, table,
                     loads, load_count, static_cast<char*>(k_pool), static_cast<char*>(v_pool),
                     s.chunk_size);
  return hipGetLastError();
}

}  // namespace lsa
