// gather.hip -- resident chunk pool and measurement helpers.
//
// Wiki note flowchart (its resident-chunk node) and the molayo explainer's
// paragraph on gathering only the selected chunks: only the kept chunks stay
// resident.
// The gather copies each kept chunk of the K (and V) history into its pool
// slot; rows past the end of the stream are zero-filled.  One workgroup per
// (kept slot, stream); each thread moves 16-byte vectors with several loads
// in flight, so a chunk is read and written as whole cache lines.  Loads and
// stores carry the non-temporal hint: at 4 x 512K (215 MB moved) that took
// the gather from 45.5 to 38.0 us, against 41.2 with the hint on the loads
// only and 40.0 on the stores only.
#include "lsa_internal.hpp"

namespace lsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

__device__ __forceinline__ void copy_chunk(const char* __restrict__ src, char* __restrict__ dst,
                                           int64_t valid_bytes, int64_t total_bytes) {
  const int tid = threadIdx.x;
  constexpr int64_t kStep = static_cast<int64_t>(kGatherThreads) * 16;
  for (int64_t off0 = static_cast<int64_t>(tid) * 16; off0 < total_bytes;
       off0 += kStep * kGatherUnroll) {
    u32x4 v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t off = off0 + u * kStep;
      v[u] = (off < valid_bytes)
                 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off))
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int64_t off = off0 + u * kStep;
      if (off < total_bytes) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(dst + off));
    }
  }
}

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(
    const char* __restrict__ store, int32_t row_bytes, const int64_t* __restrict__ tok_off,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_off,
    char* __restrict__ pool, const char* __restrict__ store2, int32_t row_bytes2,
    char* __restrict__ pool2, int32_t C, int32_t uni_k) {
  const int b = blockIdx.y;
  const int32_t j = blockIdx.x;
  const int32_t s0 = uni_k > 0 ? b * uni_k : sel_off[b];  // uniform: not read
  const int32_t k = uni_k > 0 ? uni_k : sel_off[b + 1] - s0;
  if (j >= k) return;
  const int64_t slot = static_cast<int64_t>(s0) + j;
  const int64_t len = tok_off[b + 1] - tok_off[b];
  const int64_t n = sel_idx[slot];
  int64_t valid = len - n * C;
  if (n < 0 || valid < 0) valid = 0;
  if (valid > C) valid = C;
  const int64_t row0 = tok_off[b] + n * C;
  copy_chunk(store + row0 * row_bytes, pool + slot * C * row_bytes, valid * row_bytes,
             static_cast<int64_t>(C) * row_bytes);
  if (pool2 != nullptr)
    copy_chunk(store2 + row0 * row_bytes2, pool2 + slot * C * row_bytes2, valid * row_bytes2,
               static_cast<int64_t>(C) * row_bytes2);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(256) void flush_kernel(u32x4* __restrict__ buf, int64_t n,
                                                    uint32_t salt) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride)
    buf[i] = u32x4{salt, static_cast<uint32_t>(i), salt ^ 0x5bd1e995u, 1u};
}

// Read-only streaming of n 16-byte vectors in one of three access patterns
// (the calibration references of the HBM read counters):
//   0  plain loads, each wave instruction covering 1 KiB of consecutive bytes;
//   1  the same with the non-temporal hint;
//   2  the multi-query attention kernel's K operand pattern: the buffer seen
//      as 256-byte rows in blocks of 16 rows, a wave instruction covering 64
//      bytes of each of the 16 rows and the next instruction the next 64,
//      with the non-temporal hint.
// Every loaded word is folded into one value per thread, written to
// sink[thread] so that no load can be removed.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                   int32_t pattern, uint32_t* __restrict__ sink) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  if (pattern == 2) {
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x / 64);
    const int64_t wave = tid / 64;
    const int64_t blocks = n / 256;  // 16 rows x 16 vectors
    for (int64_t blk = wave; blk < blocks; blk += waves) {
      const u32x4* rowp = src + blk * 256 + r16 * 16 + g;
      u32x4 v[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) v[s2] = __builtin_nontemporal_load(rowp + 4 * s2);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc ^= v[s2].x ^ v[s2].y ^ v[s2].z ^ v[s2].w;
    }
  } else {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = tid; i < n; i += stride) {
      const u32x4 v = pattern == 1 ? __builtin_nontemporal_load(src + i) : src[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  sink[tid] = acc;
}

}  // namespace

hipError_t launch_bench_read(const void* src, size_t bytes, int32_t pattern, uint32_t* sink,
                             hipStream_t st) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  hipLaunchKernelGGL(read_kernel, dim3(kBenchReadBlocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(src), n, pattern, sink);
  return hipGetLastError();
}

hipError_t launch_gather(const lsa_shape& s, const void* store, int32_t row_bytes,
                         const int64_t* tok_off, const int32_t* sel_idx,
                         const int32_t* sel_off, void* pool, const void* store2,
                         int32_t row_bytes2, void* pool2, hipStream_t st) {
  if (s.max_k <= 0) return hipSuccess;
  dim3 grid(s.max_k, s.batch);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kGatherThreads), 0, st,
                     static_cast<const char*>(store), row_bytes, tok_off, sel_idx, sel_off,
                     static_cast<char*>(pool), static_cast<const char*>(store2), row_bytes2,
                     static_cast<char*>(pool2), s.chunk_size,
                     (s.flags & LSA_SHAPE_UNIFORM) ? s.max_k : 0);
  return hipGetLastError();
}

hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_bench_flush(void* buf, size_t bytes, hipStream_t st) {
  const uint32_t salt = 0x9e3779b9u;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(flush_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, st,
                     static_cast<u32x4*>(buf), n, salt);
  return hipGetLastError();
}

}  // namespace lsa
