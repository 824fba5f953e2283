// check.hip -- lsa_check_tables: the offset-table and kept-index
// preconditions of lsa.h checked on the device (a debug aid; the hot-path
// kernels never run it).  One wave per stream evaluates table_check.hpp's
// checks and ORs the error bits of the batch into one device word.
#include "lsa_internal.hpp"
#include "table_check.hpp"

namespace lsa {
namespace {

__global__ __launch_bounds__(kWave) void clear_flag_kernel(int32_t* flag) {
  if (threadIdx.x == 0) *flag = 0;
}

__global__ __launch_bounds__(kWave) void check_tables_kernel(TableShape s, const int64_t* tok_off,
                                                            const int32_t* chunk_off,
                                                            const int32_t* sel_off,
                                                            const int32_t* sel_idx,
                                                            int32_t ascending, int32_t* flag) {
  const int32_t b = blockIdx.x;
  const int lane = threadIdx.x;
  StreamRange r;
  uint32_t e = table_check_offsets(s, b, tok_off, chunk_off, sel_off, &r);
  if (sel_idx != nullptr)
    for (int32_t i = lane; i < r.k; i += kWave) e |= table_check_index(sel_idx, r, i, ascending != 0);
  // OR over the wave, one bit at a time
  uint32_t all = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit)
    if (__ballot((e >> bit) & 1u) != 0) all |= 1u << bit;
  if (lane == 0 && all != 0) atomicOr(flag, static_cast<int32_t>(all));
}

}  // namespace

hipError_t launch_check_tables(const lsa_shape& s, const int64_t* tok_off,
                               const int32_t* chunk_off, const int32_t* sel_off,
                               const int32_t* sel_idx, int32_t ascending, int32_t* flag,
                               hipStream_t st) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(kWave), 0, st, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const TableShape ts = {s.batch, s.chunk_size, s.max_chunks, s.max_k, s.total_chunks, s.total_k,
                         (s.flags & LSA_SHAPE_UNIFORM) ? 1 : 0};
  hipLaunchKernelGGL(check_tables_kernel, dim3(s.batch), dim3(kWave), 0, st, ts, tok_off,
                     chunk_off, sel_off, sel_idx, ascending, flag);
  return hipGetLastError();
}

}  // namespace lsa
