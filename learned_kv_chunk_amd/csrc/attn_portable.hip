// attn_portable.hip -- split-KV sparse decode attention on the vector ALUs,
// for fp32 inputs and for head shapes the matrix-core kernels do not cover
// (up to 16 query heads, head dims up to 256).
//
// Dimensionstp review, section 3-2-3 steps 6-7: softmax attention over the
// tokens of the kept chunks.  A workgroup owns a run of 32-token tiles of one
// stream.  Two forms: on short inputs with 5-16 heads the split-heads form
// further below (the waves share each tile and split its heads); otherwise
// the tile-parallel form here, whose waves take the run's tiles in turn
// (wave w: tiles w, w + NW, ...).  Per tile a wave
//   * loads the tile's K and V rows as 16-byte vectors of consecutive
//     addresses (a tile of a chunk is contiguous in memory: one round trip
//     for the whole tile), the next tile's loads already in flight in a
//     second register set while the current tile is computed from LDS,
//   * computes the logits with lane = token (lanes 0-31 and 32-63 take
//     alternate heads) from its LDS copy of K and the stream's queries,
//   * updates the per-head online softmax (half-wave max and sum
//     reductions), writing the weights to LDS,
//   * accumulates O with lane = output column, reading V rows from LDS
//     (consecutive lanes, consecutive words).
// The waves' (max, sum, output) states are tree-merged through LDS into the
// workgroup's partial result; a stream served by one workgroup writes its
// output directly, otherwise the stream's last workgroup to finish merges
// the partials (when the library chose that, see capi.hip) or a merge launch
// does.
#include <math.h>

#include "lsa_internal.hpp"
#include "select_core.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

constexpr int kPortHeads = 16;
constexpr int kPortMaxDim = 256;
constexpr int kPortMaxRowBytes = kPortMaxDim * 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ f32x4 widen4(const unsigned char* p);
template <>
__device__ __forceinline__ f32x4 widen4<float>(const unsigned char* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 widen4<uint16_t>(const unsigned char* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}

template <typename T>
__device__ __forceinline__ float widen1(const unsigned char* p);
template <>
__device__ __forceinline__ float widen1<float>(const unsigned char* p) {
  return *reinterpret_cast<const float*>(p);
}
template <>
__device__ __forceinline__ float widen1<uint16_t>(const unsigned char* p) {
  return __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16);
}

// Max / sum over each half-wave (lanes 0-31, 32-63), in every lane: DPP
// steps within each 16-lane row, then one row swap (no LDS round trips; the
// shuffle form cost five dependent LDS accesses per reduction).
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  return xor16_max(v);
}
__device__ __forceinline__ float half_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return xor16_sum(v);
}

// Geometry of one wave's tile loads: row bytes of K and V (multiples of 16),
// their 16-byte vectors per row, and the vectors per lane of a 32-row tile.
struct PortGeom {
  int32_t kb, vb;      // row bytes read per token (K: dqk elements, V: dv elements)
  int32_t kvec, vvec;  // 16-byte vectors per row
  int64_t kstride, vstride;  // bytes between consecutive rows in memory
};

// 16-byte vectors of a 32-row tile per lane, at most: 32 * 1024 / 16 / 64.
constexpr int kPortLoads = kTileTokens * kPortMaxRowBytes / 16 / kWave;

// LP: loads per lane of K and of V (compile-time bound of vec * 32 / 64).
template <int LP>
struct PortRegs {
  u32x4 k[LP];
  u32x4 v[LP];
};

// Issues the loads of one tile (rows row0 .. row0 + 31, rows past nvalid
// re-read the last valid row; nvalid == 0 reads row0): lane l takes vectors
// l, l + 64, ... of the tile.
template <int LP>
__device__ __forceinline__ void port_issue(const unsigned char* __restrict__ kbase,
                                           const unsigned char* __restrict__ vbase,
                                           const PortGeom& g, int64_t row0, int32_t nvalid,
                                           PortRegs<LP>& r, int lane) {
  const int32_t last = nvalid > 0 ? nvalid - 1 : 0;
#pragma unroll
  for (int i = 0; i < LP; ++i) {
    const int32_t v = i * kWave + lane;
    const int32_t rk = min(v / g.kvec, last), sk = v % g.kvec;
    const int32_t rv = min(v / g.vvec, last), sv = v % g.vvec;
    if (v < kTileTokens * g.kvec)
      r.k[i] = *reinterpret_cast<const u32x4*>(kbase + (row0 + rk) * g.kstride + sk * 16);
    if (v < kTileTokens * g.vvec)
      r.v[i] = *reinterpret_cast<const u32x4*>(vbase + (row0 + rv) * g.vstride + sv * 16);
  }
}

// The registers of a tile into this wave's LDS tiles (rows padded by 16
// bytes so that the 32 lanes reading one column of different rows spread
// over the banks).
template <int LP>
__device__ __forceinline__ void port_stage(const PortRegs<LP>& r, const PortGeom& g,
                                           unsigned char* sk_tile, unsigned char* sv_tile,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < LP; ++i) {
    const int32_t v = i * kWave + lane;
    if (v < kTileTokens * g.kvec)
      *reinterpret_cast<u32x4*>(sk_tile + (v / g.kvec) * (g.kb + 16) + (v % g.kvec) * 16) = r.k[i];
    if (v < kTileTokens * g.vvec)
      *reinterpret_cast<u32x4*>(sv_tile + (v / g.vvec) * (g.vb + 16) + (v % g.vvec) * 16) = r.v[i];
  }
}

template <int HM, int CV>
struct PortState {
  float acc[HM][CV];  // lane's output columns lane + 64 i, unnormalised
};

// Waves per workgroup: four while four waves' K and V tiles fit the LDS
// beside the queries (rows up to 256 bytes), else two.
template <int LP>
constexpr int port_waves() { return LP <= 8 ? 4 : 2; }

// HM heads (>= H, even); CV output columns per lane / 64; LP tile loads per
// lane (rows of up to LP * 32 bytes).
template <typename T, int HM, int CV, int LP>
__global__ __launch_bounds__(port_waves<LP>() * kWave) void attn_portable_kernel(AttnArgs a) {
  constexpr int NW = port_waves<LP>();
  constexpr int kWaveTileBytes = 2 * kTileTokens * (LP * 32 + 16);  // K and V tiles
  constexpr bool kDoubleBuffer = LP <= 8;  // two register sets fit beside the accumulators
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * kWaveTileBytes];
  __shared__ int32_t s_slot[kMaxRunSlots];
  __shared__ AttnRun s_run;
  __shared__ float s_q[HM * kPortMaxDim];
  __shared__ float s_p[NW][HM][kTileTokens];
  __shared__ float s_stat[NW][3][HM];  // per wave: running max, sum, this tile's rescale
  __shared__ int32_t s_last;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const AttnRun run = attn_prologue(a, s_slot, &s_run);
  if (run.b < 0) return;
  const int32_t b = run.b;
  const int32_t H = a.H, dqk = a.dqk, dv = a.dv, C = a.C, tpc = a.tiles_per_chunk;
  constexpr int ES = sizeof(T);
  PortGeom g;
  g.kb = dqk * ES;
  g.vb = dv * ES;
  g.kvec = g.kb / 16;
  g.vvec = g.vb / 16;
  g.kstride = static_cast<int64_t>(a.k_row) * ES;
  g.vstride = static_cast<int64_t>(a.v_row) * ES;
  unsigned char* sk_tile = smem + wave * kWaveTileBytes;
  unsigned char* sv_tile = sk_tile + kTileTokens * (g.kb + 16);

  const unsigned char* __restrict__ kbase = static_cast<const unsigned char*>(a.k);
  const unsigned char* __restrict__ vbase = static_cast<const unsigned char*>(a.v);
  const int64_t last_chunk = run.len > 0 ? (run.len - 1) / C : 0;
  // tile i of this wave: (first row, valid tokens)
  auto tile_of = [&](int32_t i, int64_t* row0, int32_t* nvalid) {
    const int32_t t = run.t_begin + wave + NW * i;
    const int32_t j = t / tpc;
    const int32_t sub = t - j * tpc;
    int64_t n = s_slot[min(j - run.slot_first, kMaxRunSlots - 1)];
    n = n < 0 ? 0 : (n > last_chunk ? last_chunk : n);
    int64_t valid = run.len - n * C;
    if (valid > C) valid = C;
    valid -= static_cast<int64_t>(sub) * kTileTokens;
    const int64_t chunk_row = a.pool ? static_cast<int64_t>(run.sel0 + j) * C : run.tb + n * C;
    if (valid <= 0) {
      *nvalid = 0;
      *row0 = chunk_row;
    } else {
      *nvalid = valid > kTileTokens ? kTileTokens : static_cast<int32_t>(valid);
      *row0 = chunk_row + sub * kTileTokens;
    }
  };
  const int32_t n_mine = (run.t_end - run.t_begin - wave + NW - 1) / NW;

  // the first tile's loads go out before the queries are staged
  PortRegs<LP> ra;
  int64_t row_a = 0, row_b = 0;
  int32_t nv_a = 0, nv_b = 0;
  if (n_mine > 0) {
    tile_of(0, &row_a, &nv_a);
    port_issue<LP>(kbase, vbase, g, row_a, nv_a, ra, lane);
  }
  {
    const unsigned char* qb = static_cast<const unsigned char*>(a.q) +
                              static_cast<int64_t>(b) * H * dqk * ES;
    for (int32_t i = tid; i < H * dqk; i += NW * kWave) s_q[i] = widen1<T>(qb + i * ES);
    for (int32_t i = H * dqk + tid; i < HM * dqk; i += NW * kWave) s_q[i] = 0.f;
  }
  if (lane < HM) {
    s_stat[wave][0][lane] = -INFINITY;
    s_stat[wave][1][lane] = 0.f;
  }
  __syncthreads();

  PortState<HM, CV> st;
#pragma unroll
  for (int h = 0; h < HM; ++h)
#pragma unroll
    for (int i = 0; i < CV; ++i) st.acc[h][i] = 0.f;

  const int tok = lane & (kTileTokens - 1), half = lane >> 5;
  auto compute = [&](const PortRegs<LP>& r, int32_t nv) {
    port_stage<LP>(r, g, sk_tile, sv_tile, lane);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
    // logits: lane = token, heads half, half + 2, ...
    float x[HM / 2];
#pragma unroll
    for (int j = 0; j < HM / 2; ++j) x[j] = 0.f;
    const unsigned char* krow = sk_tile + tok * (g.kb + 16);
#pragma unroll 4
    for (int32_t d0 = 0; d0 < dqk; d0 += 4) {
      const f32x4 kv = widen4<T>(krow + d0 * ES);
#pragma unroll
      for (int j = 0; j < HM / 2; ++j) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(s_q + (2 * j + half) * dqk + d0);
        x[j] = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, x[j]))));
      }
    }
    // online softmax per head (the lanes of a half share the head)
#pragma unroll
    for (int j = 0; j < HM / 2; ++j) {
      const int h = 2 * j + half;
      const float xs = tok < nv ? x[j] * a.scale_log2 : -INFINITY;
      const float m_old = s_stat[wave][0][h];
      const float m_new = fmaxf(m_old, half_max(xs));
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float p = tok < nv ? __builtin_amdgcn_exp2f(xs - m_use) : 0.f;
      const float ps = half_sum(p);
      s_p[wave][h][tok] = p;
      if (tok == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
        s_stat[wave][0][h] = m_new;
        s_stat[wave][1][h] = s_stat[wave][1][h] * alpha + ps;
        s_stat[wave][2][h] = alpha;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // O += P V: lane = column; four tokens per step (weights past nv are 0
    // and their V rows hold finite values)
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      const float alpha = s_stat[wave][2][h];
#pragma unroll
      for (int i = 0; i < CV; ++i) st.acc[h][i] *= alpha;
    }
#pragma unroll 4
    for (int32_t t0 = 0; t0 < nv; t0 += 4) {
      float vv[4][CV];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned char* vrow = sv_tile + (t0 + u) * (g.vb + 16);
#pragma unroll
        for (int i = 0; i < CV; ++i) {
          const int32_t c = min(lane + i * kWave, dv - 1);
          vv[u][i] = widen1<T>(vrow + c * ES);
        }
      }
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const f32x4 p = *reinterpret_cast<const f32x4*>(&s_p[wave][h][t0]);
#pragma unroll
        for (int i = 0; i < CV; ++i)
          st.acc[h][i] = fmaf(p.x, vv[0][i], fmaf(p.y, vv[1][i],
                              fmaf(p.z, vv[2][i], fmaf(p.w, vv[3][i], st.acc[h][i]))));
      }
    }
    __builtin_amdgcn_wave_barrier();  // LDS tiles are rewritten by the next stage
  };

  if constexpr (kDoubleBuffer) {
    PortRegs<LP> rb;
    for (int32_t i = 0; i < n_mine; i += 2) {
      if (i + 1 < n_mine) {
        tile_of(i + 1, &row_b, &nv_b);
        port_issue<LP>(kbase, vbase, g, row_b, nv_b, rb, lane);
      }
      compute(ra, nv_a);
      if (i + 1 >= n_mine) break;
      if (i + 2 < n_mine) {
        tile_of(i + 2, &row_a, &nv_a);
        port_issue<LP>(kbase, vbase, g, row_a, nv_a, ra, lane);
      }
      compute(rb, nv_b);
    }
  } else {  // rows over 256 bytes: one register set, tiles loaded one at a time
    for (int32_t i = 0; i < n_mine; ++i) {
      if (i > 0) {
        tile_of(i, &row_a, &nv_a);
        port_issue<LP>(kbase, vbase, g, row_a, nv_a, ra, lane);
      }
      compute(ra, nv_a);
    }
  }

  // tree-merge the waves' states into wave 0 (output columns through LDS,
  // reusing the tile buffers)
  float* so = reinterpret_cast<float*>(smem);  // [NW/2][HM][CV][64]
#pragma unroll
  for (int stride = NW / 2; stride >= 1; stride /= 2) {
    __syncthreads();
    if (wave >= stride && wave < 2 * stride) {
      float* dst = so + (wave - stride) * HM * CV * kWave;
#pragma unroll
      for (int h = 0; h < HM; ++h)
#pragma unroll
        for (int i = 0; i < CV; ++i) dst[(h * CV + i) * kWave + lane] = st.acc[h][i];
    }
    __syncthreads();
    if (wave < stride) {
      const float* src = so + wave * HM * CV * kWave;
      const int other = wave + stride;
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const float m0 = s_stat[wave][0][h], m1 = s_stat[other][0][h];
        const float mx = fmaxf(m0, m1);
        const float mu = (mx == -INFINITY) ? 0.f : mx;
        const float f0 = __builtin_amdgcn_exp2f(m0 - mu), f1 = __builtin_amdgcn_exp2f(m1 - mu);
#pragma unroll
        for (int i = 0; i < CV; ++i)
          st.acc[h][i] = st.acc[h][i] * f0 + src[(h * CV + i) * kWave + lane] * f1;
      }
    }
    __syncthreads();
    if (wave < stride && lane < HM) {
      const int h = lane, other = wave + stride;
      const float m0 = s_stat[wave][0][h], m1 = s_stat[other][0][h];
      const float mx = fmaxf(m0, m1);
      const float mu = (mx == -INFINITY) ? 0.f : mx;
      s_stat[wave][1][h] = s_stat[wave][1][h] * __builtin_amdgcn_exp2f(m0 - mu) +
                           s_stat[other][1][h] * __builtin_amdgcn_exp2f(m1 - mu);
      s_stat[wave][0][h] = mx;
    }
  }
  __syncthreads();

  const int64_t wg = blockIdx.x;
  if (a.fuse_merge && run.wgs == 1) {  // the stream's whole state: output directly
    if (wave == 0) {
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        if (h >= H) continue;
        const float lt = s_stat[0][1][h];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int64_t orow = static_cast<int64_t>(b) * H + h;
#pragma unroll
        for (int i = 0; i < CV; ++i) {
          const int32_t c = lane + i * kWave;
          if (c < dv) a.out[orow * dv + c] = st.acc[h][i] * inv;
        }
        if (lane == 0 && a.lse != nullptr)
          a.lse[orow] = lt > 0.f ? (s_stat[0][0][h] + log2f(lt)) * 0.69314718055994530942f
                                 : -INFINITY;
      }
    }
    return;
  }
  if (wave == 0) {
#pragma unroll
    for (int h = 0; h < HM; ++h) {
      if (h >= H) continue;
      float* om = a.ws_m + wg * H + h;
      float* ol = a.ws_l + wg * H + h;
      float* oo = a.ws_o + (wg * H + h) * dv;
      if (lane == 0) {
        if (a.fuse_merge) {
          store_coherent(om, s_stat[0][0][h]);
          store_coherent(ol, s_stat[0][1][h]);
        } else {
          *om = s_stat[0][0][h];
          *ol = s_stat[0][1][h];
        }
      }
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int32_t c = lane + i * kWave;
        if (c >= dv) continue;
        if (a.fuse_merge) store_coherent(oo + c, st.acc[h][i]);
        else oo[c] = st.acc[h][i];
      }
    }
  }
  if (!a.fuse_merge) return;
  if (!arrive_last(a, b, run.wgs, &s_last)) return;
  merge_stream_block<NW * kWave>(a, b, wg - run.local, run.wgs);
  if (tid == 0)
    __hip_atomic_store(a.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Split-heads form, for inputs of few tiles (the plan then gives a workgroup
// one tile) with 5-16 heads and rows of at most 256 bytes: the four waves of
// the workgroup share each tile -- its 256 threads load it and stage it once
// in LDS -- and wave w takes heads w * HPW .. w * HPW + HPW - 1 (its two
// half-waves alternate between them).  A tile then costs each wave a quarter
// of the logits and of P.V, and the waves' states need no merging: each wave
// owns the whole state of its heads.  KSEL > 0: the workgroup ranks its
// stream's kept chunks itself before its first tile (KSEL keys per thread,
// attn_select_stream) instead of reading them.
constexpr int kShWaves = 4;
constexpr int kShThreads = kShWaves * kWave;
constexpr int kShMaxRowBytes = 256;
constexpr int kShLoads = kTileTokens * (kShMaxRowBytes / 16) / kShThreads;  // per thread per array

template <typename T, int HM, int CV, int KSEL>
__global__ __launch_bounds__(kShThreads) void attn_portable_sh_kernel(AttnArgs a) {
  constexpr int HPW = HM / kShWaves;  // heads per wave
  constexpr int JH = HPW / 2;         // heads per half-wave
  constexpr int kPitchMax = kShMaxRowBytes + 16;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kTileTokens * kPitchMax];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[kTileTokens * kPitchMax];
  __shared__ int32_t s_slot[kMaxRunSlots];
  __shared__ AttnRun s_run;
  __shared__ __attribute__((aligned(16))) float s_q[HM * (kShMaxRowBytes / 2)];
  __shared__ __attribute__((aligned(16))) float s_p[HM][kTileTokens];
  __shared__ float s_stat[3][HM];  // per head: running max, sum, this tile's rescale
  __shared__ int32_t s_last;
  static_assert(sizeof(SelectLds<kShThreads>) <= sizeof(s_k), "the top-k scratch aliases s_k");

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid & (kWave - 1);
  const AttnRun run = attn_prologue(a, s_slot, &s_run);
  if (run.b < 0) return;
  const int32_t b = run.b;
  const int32_t H = a.H, dqk = a.dqk, dv = a.dv, C = a.C, tpc = a.tiles_per_chunk;
  constexpr int ES = sizeof(T);

  // the stream's queries, HM x dqk (rows past H zero), kQPer values per thread
  constexpr int kQPer = HM * (kShMaxRowBytes / 2) / kShThreads;
  float qreg[kQPer];
  auto load_q = [&]() {
    const unsigned char* qb = static_cast<const unsigned char*>(a.q) +
                              static_cast<int64_t>(b) * H * dqk * ES;
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int32_t i = u * kShThreads + tid;
      qreg[u] = i < H * dqk ? widen1<T>(qb + i * ES) : 0.f;
    }
  };
  if constexpr (KSEL > 0) {  // the query loads are in flight while the top-k runs
    load_q();
    attn_select_stream<kShThreads, KSEL>(a, run, s_slot,
                                         *reinterpret_cast<SelectLds<kShThreads>*>(s_k));
  }
  // s_slot holds the run's kept chunks, or the whole stream's when ranked here
  const int32_t slot_first = KSEL > 0 ? 0 : run.slot_first;
  PortGeom g;
  g.kb = dqk * ES;
  g.vb = dv * ES;
  g.kvec = g.kb / 16;
  g.vvec = g.vb / 16;
  g.kstride = static_cast<int64_t>(a.k_row) * ES;
  g.vstride = static_cast<int64_t>(a.v_row) * ES;
  const int32_t kpitch = g.kb + 16, vpitch = g.vb + 16;

  const unsigned char* __restrict__ kbase = static_cast<const unsigned char*>(a.k);
  const unsigned char* __restrict__ vbase = static_cast<const unsigned char*>(a.v);
  const int64_t last_chunk = run.len > 0 ? (run.len - 1) / C : 0;
  // tile i of the run: (first row, valid tokens), as in the kernel above
  auto tile_of = [&](int32_t i, int64_t* row0, int32_t* nvalid) {
    const int32_t t = run.t_begin + i;
    const int32_t j = t / tpc;
    const int32_t sub = t - j * tpc;
    int64_t n = s_slot[min(j - slot_first, kMaxRunSlots - 1)];
    n = n < 0 ? 0 : (n > last_chunk ? last_chunk : n);
    int64_t valid = run.len - n * C;
    if (valid > C) valid = C;
    valid -= static_cast<int64_t>(sub) * kTileTokens;
    const int64_t chunk_row = a.pool ? static_cast<int64_t>(run.sel0 + j) * C : run.tb + n * C;
    if (valid <= 0) {
      *nvalid = 0;
      *row0 = chunk_row;
    } else {
      *nvalid = valid > kTileTokens ? kTileTokens : static_cast<int32_t>(valid);
      *row0 = chunk_row + sub * kTileTokens;
    }
  };
  const int32_t n_tiles = run.t_end - run.t_begin;

  // thread tid loads vectors tid, tid + 256, ... of the tile's K and V rows
  // (rows past nvalid re-read the last valid row)
  struct ShRegs {
    u32x4 k[kShLoads];
    u32x4 v[kShLoads];
  };
  auto issue = [&](int64_t row0, int32_t nvalid, ShRegs& r) {
    const int32_t last = nvalid > 0 ? nvalid - 1 : 0;
#pragma unroll
    for (int i = 0; i < kShLoads; ++i) {
      const int32_t v = i * kShThreads + tid;
      if (v < kTileTokens * g.kvec)
        r.k[i] = *reinterpret_cast<const u32x4*>(
            kbase + (row0 + min(v / g.kvec, last)) * g.kstride + (v % g.kvec) * 16);
      if (v < kTileTokens * g.vvec)
        r.v[i] = *reinterpret_cast<const u32x4*>(
            vbase + (row0 + min(v / g.vvec, last)) * g.vstride + (v % g.vvec) * 16);
    }
  };
  auto stage = [&](const ShRegs& r) {
#pragma unroll
    for (int i = 0; i < kShLoads; ++i) {
      const int32_t v = i * kShThreads + tid;
      if (v < kTileTokens * g.kvec)
        *reinterpret_cast<u32x4*>(s_k + (v / g.kvec) * kpitch + (v % g.kvec) * 16) = r.k[i];
      if (v < kTileTokens * g.vvec)
        *reinterpret_cast<u32x4*>(s_v + (v / g.vvec) * vpitch + (v % g.vvec) * 16) = r.v[i];
    }
  };

  // the first tile's loads go out before the queries are staged
  ShRegs ra, rb;
  int64_t row_a = 0, row_b = 0;
  int32_t nv_a = 0, nv_b = 0;
  if (n_tiles > 0) {
    tile_of(0, &row_a, &nv_a);
    issue(row_a, nv_a, ra);
  }
  if constexpr (KSEL == 0) load_q();
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int32_t i = u * kShThreads + tid;
    if (i < HM * dqk) s_q[i] = qreg[u];
  }
  if (tid < HM) {
    s_stat[0][tid] = -INFINITY;
    s_stat[1][tid] = 0.f;
  }

  float acc[HPW][CV];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int i = 0; i < CV; ++i) acc[hh][i] = 0.f;

  const int tok = lane & (kTileTokens - 1), half = lane >> 5;
  const int h0 = wave * HPW;  // this wave's first head
  auto compute = [&](int32_t nv) {
    // logits: lane = token, heads h0 + half, h0 + 2 + half, ...
    float x[JH];
#pragma unroll
    for (int j = 0; j < JH; ++j) x[j] = 0.f;
    const unsigned char* krow = s_k + tok * kpitch;
#pragma unroll 4
    for (int32_t d0 = 0; d0 < dqk; d0 += 4) {
      const f32x4 kv = widen4<T>(krow + d0 * ES);
#pragma unroll
      for (int j = 0; j < JH; ++j) {
        const f32x4 qv = *reinterpret_cast<const f32x4*>(s_q + (h0 + 2 * j + half) * dqk + d0);
        x[j] = fmaf(qv.x, kv.x, fmaf(qv.y, kv.y, fmaf(qv.z, kv.z, fmaf(qv.w, kv.w, x[j]))));
      }
    }
    // online softmax per head (the lanes of a half share the head)
#pragma unroll
    for (int j = 0; j < JH; ++j) {
      const int h = h0 + 2 * j + half;
      const float xs = tok < nv ? x[j] * a.scale_log2 : -INFINITY;
      const float m_old = s_stat[0][h];
      const float m_new = fmaxf(m_old, half_max(xs));
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float p = tok < nv ? __builtin_amdgcn_exp2f(xs - m_use) : 0.f;
      const float ps = half_sum(p);
      s_p[h][tok] = p;
      if (tok == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_use);
        s_stat[0][h] = m_new;
        s_stat[1][h] = s_stat[1][h] * alpha + ps;
        s_stat[2][h] = alpha;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the weights are in LDS
    __builtin_amdgcn_wave_barrier();
    // O += P V for this wave's heads: lane = column, four tokens per step
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float alpha = s_stat[2][h0 + hh];
#pragma unroll
      for (int i = 0; i < CV; ++i) acc[hh][i] *= alpha;
    }
#pragma unroll 4
    for (int32_t t0 = 0; t0 < nv; t0 += 4) {
      float vv[4][CV];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const unsigned char* vrow = s_v + (t0 + u) * vpitch;
#pragma unroll
        for (int i = 0; i < CV; ++i) vv[u][i] = widen1<T>(vrow + min(lane + i * kWave, dv - 1) * ES);
      }
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const f32x4 p = *reinterpret_cast<const f32x4*>(&s_p[h0 + hh][t0]);
#pragma unroll
        for (int i = 0; i < CV; ++i)
          acc[hh][i] = fmaf(p.x, vv[0][i], fmaf(p.y, vv[1][i],
                            fmaf(p.z, vv[2][i], fmaf(p.w, vv[3][i], acc[hh][i]))));
      }
    }
  };

  // every wave stages its share of a tile, then every wave computes on it;
  // the barrier after the products frees the tile buffers for the next one
  __syncthreads();
  for (int32_t i = 0; i < n_tiles; i += 2) {
    if (i + 1 < n_tiles) {
      tile_of(i + 1, &row_b, &nv_b);
      issue(row_b, nv_b, rb);
    }
    stage(ra);
    __syncthreads();
    compute(nv_a);
    __syncthreads();
    if (i + 1 >= n_tiles) break;
    if (i + 2 < n_tiles) {
      tile_of(i + 2, &row_a, &nv_a);
      issue(row_a, nv_a, ra);
    }
    stage(rb);
    __syncthreads();
    compute(nv_b);
    __syncthreads();
  }

  const int64_t wg = blockIdx.x;
  if (a.fuse_merge && run.wgs == 1) {  // the stream's whole state: output directly
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = h0 + hh;
      if (h >= H) continue;
      const float lt = s_stat[1][h];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t orow = static_cast<int64_t>(b) * H + h;
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int32_t c = lane + i * kWave;
        if (c < dv) a.out[orow * dv + c] = acc[hh][i] * inv;
      }
      if (lane == 0 && a.lse != nullptr)
        a.lse[orow] = lt > 0.f ? (s_stat[0][h] + log2f(lt)) * 0.69314718055994530942f
                               : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = h0 + hh;
    if (h >= H) continue;
    float* om = a.ws_m + wg * H + h;
    float* ol = a.ws_l + wg * H + h;
    float* oo = a.ws_o + (wg * H + h) * dv;
    if (lane == 0) {
      if (a.fuse_merge) {
        store_coherent(om, s_stat[0][h]);
        store_coherent(ol, s_stat[1][h]);
      } else {
        *om = s_stat[0][h];
        *ol = s_stat[1][h];
      }
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int32_t c = lane + i * kWave;
      if (c >= dv) continue;
      if (a.fuse_merge) store_coherent(oo + c, acc[hh][i]);
      else oo[c] = acc[hh][i];
    }
  }
  if (!a.fuse_merge) return;
  if (!arrive_last(a, b, run.wgs, &s_last)) return;
  merge_stream_block<kShThreads>(a, b, wg - run.local, run.wgs);
  if (tid == 0)
    __hip_atomic_store(a.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int HM, int KSEL>
hipError_t launch_portable_sh_k(const AttnArgs& a, int64_t grid, hipStream_t st) {
  const dim3 g(static_cast<uint32_t>(grid));
  if (a.dv <= kWave)
    hipLaunchKernelGGL((attn_portable_sh_kernel<T, HM, 1, KSEL>), g, dim3(kShThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_portable_sh_kernel<T, HM, 2, KSEL>), g, dim3(kShThreads), 0, st, a);
  return hipGetLastError();
}

// KSEL from the longest stream when the kernel ranks the kept chunks itself
template <typename T, int HM>
hipError_t launch_portable_sh(const AttnArgs& a, int32_t max_chunks, int64_t grid,
                              hipStream_t st) {
  if (a.sel_scores == nullptr) return launch_portable_sh_k<T, HM, 0>(a, grid, st);
  if (max_chunks <= kShThreads) return launch_portable_sh_k<T, HM, 1>(a, grid, st);
  if (max_chunks <= kShThreads * 8) return launch_portable_sh_k<T, HM, 8>(a, grid, st);
  if (max_chunks <= kShThreads * 16) return launch_portable_sh_k<T, HM, 16>(a, grid, st);
  return hipErrorNotSupported;
}

template <typename T, int HM, int CV>
hipError_t launch_portable_l(const AttnArgs& a, int64_t grid, hipStream_t st) {
  const int kb = a.dqk * static_cast<int>(sizeof(T)), vb = a.dv * static_cast<int>(sizeof(T));
  const int vec = (kb > vb ? kb : vb) / 16;
  const int lp = (kTileTokens * vec + kWave - 1) / kWave;
  const dim3 g(static_cast<uint32_t>(grid));
#define LSA_PORT_LP(LP_)                                                                   \
  if (lp <= LP_) {                                                                         \
    hipLaunchKernelGGL((attn_portable_kernel<T, HM, CV, LP_>), g,                          \
                       dim3(port_waves<LP_>() * kWave), 0, st, a);                         \
    return hipGetLastError();                                                              \
  }
  LSA_PORT_LP(4) LSA_PORT_LP(8) LSA_PORT_LP(16) LSA_PORT_LP(kPortLoads)
#undef LSA_PORT_LP
  return hipErrorNotSupported;
}

template <typename T, int HM>
hipError_t launch_portable_h(const AttnArgs& a, int64_t grid, hipStream_t st) {
  const int cv = (a.dv + kWave - 1) / kWave;
  if (cv == 1) return launch_portable_l<T, HM, 1>(a, grid, st);
  if (cv == 2) return launch_portable_l<T, HM, 2>(a, grid, st);
  return launch_portable_l<T, HM, 4>(a, grid, st);
}

template <typename T>
hipError_t launch_portable_t(const AttnArgs& a, int32_t max_chunks, int64_t grid,
                             hipStream_t st) {
  if (a.split_heads) {
    if (a.H <= 4 || a.H > kPortHeads || a.dqk * static_cast<int>(sizeof(T)) > kShMaxRowBytes ||
        a.dv * static_cast<int>(sizeof(T)) > kShMaxRowBytes)
      return hipErrorNotSupported;
    if (a.H <= 8) return launch_portable_sh<T, 8>(a, max_chunks, grid, st);
    return launch_portable_sh<T, 16>(a, max_chunks, grid, st);
  }
  if (a.sel_scores != nullptr) return hipErrorNotSupported;
  if (a.H <= 4) return launch_portable_h<T, 4>(a, grid, st);
  if (a.H <= 8) return launch_portable_h<T, 8>(a, grid, st);
  return launch_portable_h<T, 16>(a, grid, st);
}

}  // namespace

bool portable_attn_supported(const lsa_shape& s) {
  return s.num_q_heads >= 1 && s.num_q_heads <= kPortHeads && s.head_dim_qk >= 1 &&
         s.head_dim_qk <= kPortMaxDim && s.head_dim_v >= 1 && s.head_dim_v <= kPortMaxDim;
}

bool portable_select_in_kernel_supported(const lsa_shape& s, const AttnPlan& plan) {
  return plan.split_heads != 0 && s.max_chunks <= kShThreads * 16 && s.max_k <= kMaxRunSlots;
}

bool portable_split_heads(const lsa_shape& s, int64_t total_tiles, int32_t target) {
  const int es = s.dtype == LSA_DTYPE_BF16 ? 2 : 4;
  return portable_attn_supported(s) && s.num_q_heads > 4 &&
         s.head_dim_qk * es <= kShMaxRowBytes && s.head_dim_v * es <= kShMaxRowBytes &&
         total_tiles <= target;
}

hipError_t launch_attn_portable(const lsa_shape& s, const AttnArgs& a, int64_t grid,
                                hipStream_t st) {
  if (s.dtype == LSA_DTYPE_BF16) return launch_portable_t<uint16_t>(a, s.max_chunks, grid, st);
  return launch_portable_t<float>(a, s.max_chunks, grid, st);
}

}  // namespace lsa
