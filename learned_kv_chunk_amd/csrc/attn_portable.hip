// attn_portable.hip -- portable split-KV sparse decode attention on the
// vector ALUs, for fp32 inputs and for head shapes the matrix-core kernels do
// not cover (up to 16 query heads, head dims up to 256).
//
// Dimensionstp review, section 3-2-3 steps 6-7: softmax attention over the
// tokens of the kept chunks.  One wave per workgroup owns a run of 32-token
// tiles of one stream: lane t computes the logits of token t for every head
// (queries staged in LDS as fp32), the wave keeps an fp32 online softmax per
// head (wave-wide max / sum reductions), the tile's weights go through LDS,
// and lanes accumulate output columns c, c+64, ... reading value rows with
// coalesced loads.  Key and value reads are issued kPortBatch at a time so
// that their memory latency overlaps.  The wave's (m, l, o) is its workgroup's partial result.
#include <math.h>

#include "wave.hpp"
#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kPortHeads = 16;
constexpr int kPortMaxDim = 256;
constexpr int kPortBatch = 16;  // independent loads in flight per lane

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i]);
}

// HM: heads held in registers (>= H); CV: output columns per lane / 64.
template <typename T, int HM, int CV>
__global__ __launch_bounds__(kWave) void attn_portable_kernel(AttnArgs a) {
  __shared__ float s_q[HM * kPortMaxDim];
  __shared__ float s_p[HM][kTileTokens];
  __shared__ int32_t s_plan[3];

  const int lane = threadIdx.x;
  {
    int32_t b, local;
    StreamSplit sp;
    find_stream_of_wg(SelCsr{a.sel_off, a.uni_k}, a.B, a.tiles_per_chunk, a.per, a.target,
                      blockIdx.x, &b, &local, &sp);
    if (lane == 0) {
      s_plan[0] = b;
      s_plan[1] = local * sp.per;
      s_plan[2] = min(sp.tiles, (local + 1) * sp.per);
    }
  }
  __syncthreads();
  const int32_t b = s_plan[0];
  if (b < 0) return;
  const T* __restrict__ q = static_cast<const T*>(a.q);
  const T* __restrict__ kb = static_cast<const T*>(a.k);
  const T* __restrict__ vb = static_cast<const T*>(a.v);
  const int32_t H = a.H, dqk = a.dqk, dv = a.dv, C = a.C, tpc = a.tiles_per_chunk;
  for (int32_t i = lane; i < H * dqk; i += kWave)
    s_q[i] = load_elem(q, static_cast<int64_t>(b) * H * dqk + i);
  __syncthreads();

  const int32_t sel0 = SelCsr{a.sel_off, a.uni_k}.at(b);
  const int64_t cap = a.tok_off[b + 1] - a.tok_off[b];
  const int64_t sl = a.seq_len ? a.seq_len[b] : cap;
  const int64_t len = sl < 0 ? 0 : (sl < cap ? sl : cap);
  const int32_t t_begin = s_plan[1];
  const int32_t t_end = s_plan[2];

  float m[HM], l[HM], o[HM][CV];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < CV; ++i) o[h][i] = 0.f;
  }

  for (int32_t t = t_begin; t < t_end; ++t) {
    const int32_t slot = sel0 + t / tpc;
    const int32_t sub = t - (t / tpc) * tpc;
    const int64_t n = a.sel_idx[slot];
    int64_t valid = len - n * C;
    if (n < 0 || valid < 0) valid = 0;
    if (valid > C) valid = C;
    valid -= static_cast<int64_t>(sub) * kTileTokens;
    if (valid <= 0) continue;
    const int32_t nv = valid > kTileTokens ? kTileTokens : static_cast<int32_t>(valid);
    const int64_t row0 = a.pool ? static_cast<int64_t>(slot) * C + sub * kTileTokens
                                : a.tok_off[b] + n * C + sub * kTileTokens;

    float x[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) x[h] = 0.f;
    if (lane < nv) {
      // the token's key row, kPortBatch elements per round trip
      const int64_t kr = (row0 + lane) * a.k_row;
      for (int32_t j0 = 0; j0 < dqk; j0 += kPortBatch) {
        float kv[kPortBatch];
#pragma unroll
        for (int u = 0; u < kPortBatch; ++u) kv[u] = load_elem(kb, kr + min(j0 + u, dqk - 1));
#pragma unroll
        for (int u = 0; u < kPortBatch; ++u) {
          if (j0 + u < dqk) {
#pragma unroll
            for (int h = 0; h < HM; ++h)
              if (h < H) x[h] = fmaf(s_q[h * dqk + j0 + u], kv[u], x[h]);
          }
        }
      }
    }
    float alpha[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h >= H) {
        alpha[h] = 1.f;
        continue;
      }
      const float xs = (lane < nv) ? x[h] * a.scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[h], wave_max(xs));
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      alpha[h] = __builtin_amdgcn_exp2f(m[h] - m_use);
      const float p = (lane < nv) ? __builtin_amdgcn_exp2f(xs - m_use) : 0.f;
      l[h] = l[h] * alpha[h] + wave_sum(p);
      m[h] = m_new;
      if (lane < kTileTokens) s_p[h][lane] = p;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int32_t c = lane + i * kWave;
      if (c >= dv) continue;
      float acc[HM];
#pragma unroll
      for (int h = 0; h < HM; ++h) acc[h] = o[h][i] * alpha[h];
      for (int32_t t0 = 0; t0 < nv; t0 += kPortBatch) {
        float vv[kPortBatch];
#pragma unroll
        for (int u = 0; u < kPortBatch; ++u)
          vv[u] = load_elem(vb, (row0 + min(t0 + u, nv - 1)) * a.v_row + c);
#pragma unroll
        for (int u = 0; u < kPortBatch; ++u) {
          if (t0 + u < nv) {
#pragma unroll
            for (int h = 0; h < HM; ++h)
              if (h < H) acc[h] = fmaf(s_p[h][t0 + u], vv[u], acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < HM; ++h) o[h][i] = acc[h];
    }
    __syncthreads();
  }

  const int64_t wg = blockIdx.x;
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    if (h >= H) continue;
    if (lane == 0) {
      a.ws_m[wg * H + h] = m[h];
      a.ws_l[wg * H + h] = l[h];
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int32_t c = lane + i * kWave;
      if (c < dv) a.ws_o[(wg * H + h) * dv + c] = o[h][i];
    }
  }
}

template <typename T, int HM>
hipError_t launch_portable_h(const AttnArgs& a, int64_t grid, hipStream_t st) {
  const int cv = (a.dv + kWave - 1) / kWave;
#define LSA_PORT_CASE(CV_)                                                                  \
  if (cv == CV_) {                                                                          \
    hipLaunchKernelGGL((attn_portable_kernel<T, HM, CV_>), dim3(static_cast<uint32_t>(grid)), \
                       dim3(kWave), 0, st, a);                                              \
    return hipGetLastError();                                                               \
  }
  LSA_PORT_CASE(1) LSA_PORT_CASE(2) LSA_PORT_CASE(3) LSA_PORT_CASE(4)
#undef LSA_PORT_CASE
  return hipErrorNotSupported;
}

template <typename T>
hipError_t launch_portable_t(const AttnArgs& a, int64_t grid, hipStream_t st) {
  if (a.H <= 4) return launch_portable_h<T, 4>(a, grid, st);
  if (a.H <= 8) return launch_portable_h<T, 8>(a, grid, st);
  return launch_portable_h<T, 16>(a, grid, st);
}

}  // namespace

bool portable_attn_supported(const lsa_shape& s) {
  return s.num_q_heads >= 1 && s.num_q_heads <= kPortHeads && s.head_dim_qk >= 1 &&
         s.head_dim_qk <= kPortMaxDim && s.head_dim_v >= 1 && s.head_dim_v <= kPortMaxDim;
}

hipError_t launch_attn_portable(const lsa_shape& s, const AttnArgs& a, int64_t grid,
                                hipStream_t st) {
  if (s.dtype == LSA_DTYPE_BF16) return launch_portable_t<uint16_t>(a, grid, st);
  return launch_portable_t<float>(a, grid, st);
}

}  // namespace lsa
