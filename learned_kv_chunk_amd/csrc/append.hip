// append.hip -- decode-time growth of the context: appending each stream's
// new K/V row (lsa_append_kv) and the attention keep set of a context that
// grew since the last re-index (lsa_keep_recent).
//
// Dimensionstp review section 3-2-3, steps 2 and 7: the history goes to the
// cache and decode attends to the kept chunks.  The pages say nothing of the
// tokens written after the last re-index; this library attends to them
// through the last scored chunk (it was the partial tail when the indexer saw
// it) and every chunk the indexer has not scored yet, next to the kept ones.
//
// The stores use a capacity layout: stream b owns rows base_off[b] ..
// base_off[b+1]-1 and holds seq_len[b] of them.  Both kernels run one
// workgroup per stream; the keep-set kernel finds its output offset by
// summing the added-chunk counts of the streams before its own (each a few
// loads), so the ragged result needs a single launch.
#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 64;
constexpr int kRecentThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kv_kernel(
    const char* __restrict__ k_new, const char* __restrict__ v_new, int32_t kb, int32_t vb,
    const int64_t* __restrict__ base_off, int64_t* __restrict__ seq_len,
    char* __restrict__ k_store, char* __restrict__ v_store) {
  const int b = blockIdx.x;
  const int64_t len = seq_len[b];
  const int64_t cap = base_off[b + 1] - base_off[b];
  __syncthreads();  // every thread has read seq_len[b] before it is advanced
  if (len < 0 || len >= cap) return;  // a full stream is left unchanged
  const int64_t row = base_off[b] + len;
  for (int32_t i = threadIdx.x * 16; i < kb; i += kAppendThreads * 16)
    *reinterpret_cast<u32x4*>(k_store + row * kb + i) =
        *reinterpret_cast<const u32x4*>(k_new + static_cast<int64_t>(b) * kb + i);
  if (v_store != nullptr)
    for (int32_t i = threadIdx.x * 16; i < vb; i += kAppendThreads * 16)
      *reinterpret_cast<u32x4*>(v_store + row * vb + i) =
          *reinterpret_cast<const u32x4*>(v_new + static_cast<int64_t>(b) * vb + i);
  if (threadIdx.x == 0) seq_len[b] = len + 1;
}

// Chunks stream j attends to beyond its kept ones: the last scored chunk
// M-1 unless kept (kept chunks ascend and lie below M, so only the last can
// be M-1), then M .. ceil(L/C)-1; when more than max_recent qualify, the
// newest max_recent (the chunk of the token being decoded is always one).
// They are the consecutive chunks first .. first + count - 1.
struct Recent {
  int32_t first;
  int32_t count;
};

__device__ __forceinline__ Recent recent_of(const int64_t* seq_len, const int32_t* chunk_off,
                                            const int32_t* sel_idx, const int32_t* sel_off,
                                            int32_t C, int32_t max_recent, int32_t j) {
  const int32_t m = chunk_off[j + 1] - chunk_off[j];
  const int32_t k = sel_off[j + 1] - sel_off[j];
  const int64_t len = seq_len[j] < 0 ? 0 : seq_len[j];
  const int64_t total = (len + C - 1) / C;
  const bool last_kept = k > 0 && sel_idx[sel_off[j + 1] - 1] == m - 1;
  int64_t first = (m > 0 && !last_kept) ? m - 1 : m;
  if (total - first > max_recent) first = total - max_recent;
  Recent r;
  r.first = static_cast<int32_t>(first);
  r.count = static_cast<int32_t>(total > first ? total - first : 0);
  return r;
}

__global__ __launch_bounds__(kRecentThreads) void keep_recent_kernel(
    const int64_t* __restrict__ seq_len, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_off, int32_t C,
    int32_t max_recent, int32_t B, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_off) {
  __shared__ uint32_t s_part[kRecentThreads / kWave];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  uint32_t before = 0;
  for (int32_t j = tid; j < b; j += kRecentThreads)
    before += static_cast<uint32_t>(
        recent_of(seq_len, chunk_off, sel_idx, sel_off, C, max_recent, j).count);
  before = wave_sum_u32(before);
  if ((tid & (kWave - 1)) == 0) s_part[tid / kWave] = before;
  __syncthreads();
  uint32_t added = 0;
#pragma unroll
  for (int w = 0; w < kRecentThreads / kWave; ++w) added += s_part[w];
  const int32_t s0 = sel_off[b];
  const int32_t k = sel_off[b + 1] - s0;
  const int32_t off = s0 + static_cast<int32_t>(added);
  const Recent r = recent_of(seq_len, chunk_off, sel_idx, sel_off, C, max_recent, b);
  if (tid == 0) {
    out_off[b] = off;
    if (b == B - 1) out_off[B] = off + k + r.count;
  }
  for (int32_t i = tid; i < k; i += kRecentThreads) out_idx[off + i] = sel_idx[s0 + i];
  for (int32_t i = tid; i < r.count; i += kRecentThreads)
    out_idx[off + k + i] = r.first + i;
}

}  // namespace

hipError_t launch_append_kv(const lsa_shape& s, const void* k_new, const void* v_new,
                           int32_t k_row_bytes, int32_t v_row_bytes, const int64_t* base_off,
                           int64_t* seq_len, void* k_store, void* v_store, hipStream_t st) {
  hipLaunchKernelGGL(append_kv_kernel, dim3(s.batch), dim3(kAppendThreads), 0, st,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     k_row_bytes, v_row_bytes, base_off, seq_len, static_cast<char*>(k_store),
                     static_cast<char*>(v_store));
  return hipGetLastError();
}

hipError_t launch_keep_recent(const lsa_shape& s, const int64_t* seq_len,
                              const int32_t* chunk_off, const int32_t* sel_idx,
                              const int32_t* sel_off, int32_t max_recent, int32_t* out_idx,
                              int32_t* out_off, hipStream_t st) {
  hipLaunchKernelGGL(keep_recent_kernel, dim3(s.batch), dim3(kRecentThreads), 0, st, seq_len,
                     chunk_off, sel_idx, sel_off, s.chunk_size, max_recent, s.batch, out_idx,
                     out_off);
  return hipGetLastError();
}

}  // namespace lsa
