// score_mh.hip -- multi-head relevance of float8 compressed-key chunk records
// (lsa_score_fp8_multihead).
//
// Dimensionstp review, section 3-2-1 (a chunk's record: D float8 e4m3 key
// values and a float32 dequantisation scale), section 3-2-2 (the released
// retriever's scorer: the sum over heads of a head weight times the ReLU of
// the head query's dot product with the dequantised key) and section 4-3 (128
// heads of dimension 128).  The sigmoid of that formula is monotone and is not
// applied: the kernel writes the ranking score
//   score = sum_h w_h * max(0, c * <q_h, k8>)      (c the record's scale)
//
// Per stream this is a GEMM, S[chunk][head] = K8[chunk][:] . Q[head][:], on
// the matrix cores (v_mfma_f32_16x16x32_bf16): float8 e4m3 values convert to
// bf16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1), so the products are
// those of the decoded keys.  In the accumulator a lane holds four chunks of
// one head; the scale, ReLU and head weight apply per element and a reduction
// over the 16 lanes of a row gives each chunk's score.  A workgroup stages its
// stream's head queries (the B operand of every product, 32 KB for 128 x 128)
// in LDS once, in rows padded by 16 bytes so that the 16 rows one operand read
// touches start in distinct banks; its four waves then walk 16-chunk blocks,
// whose records are 16 x (D + 4) contiguous bytes.
#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMhThreads = 256;
constexpr int kMhRounds = 2;  // 16-chunk blocks per wave
constexpr int kMhChunksPerBlock = (kMhThreads / kWave) * 16 * kMhRounds;

// Four float8 e4m3 values (one dword, byte 0 first) as four bf16.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Records of one layer for the two rounds of a wave: A operand of round r,
// step s -- the key bytes s*32 + 8*(lane/16) .. +7 of chunk c0 + lane%16
// (rows past the stream repeat its last chunk) -- and the scales of the
// chunks c0 + 4*(lane/16) + 0..3 whose results the lane will hold.
template <int D>
struct MhRecords {
  uint32_t kw[kMhRounds][D / 32][2];
  float sc[kMhRounds][4];
};

template <int D>
__device__ __forceinline__ void mh_load_records(MhRecords<D>& R, const unsigned char* rec,
                                                int32_t base, int32_t n, int32_t blk0, int r16,
                                                int g) {
  constexpr int RB = D + 4;
#pragma unroll
  for (int r = 0; r < kMhRounds; ++r) {
    const int32_t c0 = min((blk0 + r) * 16, n - 1);
    const unsigned char* rp = rec + static_cast<int64_t>(base + min(c0 + r16, n - 1)) * RB;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rp + s * 32 + 8 * g);
      R.kw[r][s][0] = p[0];
      R.kw[r][s][1] = p[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      R.sc[r][i] = *reinterpret_cast<const float*>(
          rec + static_cast<int64_t>(base + min(c0 + 4 * g + i, n - 1)) * RB + D);
  }
}

// Layer l of the ensemble reads q + l*B*Hs*D, hw + l*B*Hs and
// rec + l*rec_layer_bytes; the per-chunk results of the layers are combined
// by max or by the mean (the sum in layer order, divided by the layer count).
template <int D, int NHB>
__global__ __launch_bounds__(kMhThreads) void score_mh_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ hw,
    const unsigned char* __restrict__ rec, const int32_t* __restrict__ chunk_off,
    float* __restrict__ scores, int32_t layers, int32_t combine, int64_t rec_layer_bytes) {
  constexpr int Hs = 16 * NHB;
  constexpr int QP = 2 * D + 16;     // LDS pitch of a head query row
  __shared__ __attribute__((aligned(16))) unsigned char s_q[Hs * QP];
  const int b = blockIdx.y;
  const int32_t B = gridDim.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int32_t base = chunk_off[b];
  const int32_t n = chunk_off[b + 1] - base;
  const int32_t blk_wg = static_cast<int32_t>(blockIdx.x) * (kMhThreads / kWave) * kMhRounds;
  if (blk_wg * 16 >= n) return;  // uniform over the workgroup
  const int32_t blk0 = blk_wg + wave * kMhRounds;

  // the first layer's records before its queries, so that the two latencies
  // overlap; each later layer's records are in flight during the layer before
  MhRecords<D> cur;
  mh_load_records<D>(cur, rec, base, n, blk0, r16, g);
  float res[kMhRounds][4];
  // B operand of lane (r16, g) for head block hb, step s: Q[hb*16 + r16][s*32 + 8g .. +7]
  const unsigned char* qrow = s_q + r16 * QP + g * 16;

  for (int32_t l = 0; l < layers; ++l) {
    if (l > 0) __syncthreads();  // every wave is done with the previous layer's queries
    // stage layer l's head queries of the stream: Hs rows of D bf16
    constexpr int kVecs = Hs * D / 8, kPerRow = D / 8;
    constexpr int kIters = (kVecs + kMhThreads - 1) / kMhThreads;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        q + (static_cast<int64_t>(l) * B + b) * Hs * D);
    u32x4 v[kIters];
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const int i = threadIdx.x + j * kMhThreads;
      if (kVecs % kMhThreads == 0 || i < kVecs) v[j] = src[i];
    }
    float wv[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
      wv[hb] = hw[(static_cast<int64_t>(l) * B + b) * Hs + hb * 16 + r16];
    MhRecords<D> nxt;
    if (l + 1 < layers)
      mh_load_records<D>(nxt, rec + (l + 1) * rec_layer_bytes, base, n, blk0, r16, g);
#pragma unroll
    for (int j = 0; j < kIters; ++j) {
      const int i = threadIdx.x + j * kMhThreads;
      if (kVecs % kMhThreads == 0 || i < kVecs)
        *reinterpret_cast<u32x4*>(s_q + (i / kPerRow) * QP + (i % kPerRow) * 16) = v[j];
    }
    __syncthreads();

    // every round is computed (rounds past the stream's end on repeated
    // chunks, their results not stored), so that no branch moves the record
    // loads after the staging
#pragma unroll
    for (int r = 0; r < kMhRounds; ++r) {
      bf16x8 kf[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const uint2 a = fp8x4_to_bf16x4(cur.kw[r][s][0]);
        const uint2 c = fp8x4_to_bf16x4(cur.kw[r][s][1]);
        kf[s] = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, c.x, c.y});
      }
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const bf16x8 qv = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(qrow + hb * 16 * QP + s * 64));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], qv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          part[i] = fmaf(wv[hb], fmaxf(acc[i] * cur.sc[r][i], 0.f), part[i]);
      }
      // sum over the 16 heads a row of lanes holds (every lane gets its row's sum)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = part[i];
        x += dpp_f32<kDppQuadXor1>(x);
        x += dpp_f32<kDppQuadXor2>(x);
        x += dpp_f32<kDppRowRor4>(x);
        x += dpp_f32<kDppRowRor8>(x);
        if (l == 0) res[r][i] = x;
        else res[r][i] = combine == LSA_COMBINE_MAX ? fmaxf(res[r][i], x) : res[r][i] + x;
      }
    }
    if (l + 1 < layers) cur = nxt;
  }

#pragma unroll
  for (int r = 0; r < kMhRounds; ++r) {
    const int32_t c0 = (blk0 + r) * 16;
    if (r16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t c = c0 + 4 * g + i;
        float x = res[r][i];
        if (combine == LSA_COMBINE_MEAN && layers > 1) x = x / static_cast<float>(layers);
        if (c < n) scores[base + c] = x;
      }
    }
  }
}

template <int D>
hipError_t launch_mh_d(const lsa_shape& s, int32_t layers, int32_t combine, int32_t heads,
                       const void* q, const float* w, const void* rec, const int32_t* chunk_off,
                       float* scores, hipStream_t st) {
  dim3 grid((s.max_chunks + kMhChunksPerBlock - 1) / kMhChunksPerBlock, s.batch);
  const int64_t rec_layer_bytes = s.total_chunks * static_cast<int64_t>(D + 4);
#define LSA_MH_CASE(NHB_)                                                                      \
  if (heads == 16 * (NHB_)) {                                                                  \
    hipLaunchKernelGGL((score_mh_kernel<D, NHB_>), grid, dim3(kMhThreads), 0, st,              \
                       static_cast<const uint16_t*>(q), w,                                     \
                       static_cast<const unsigned char*>(rec), chunk_off, scores, layers,      \
                       combine, rec_layer_bytes);                                              \
    return hipGetLastError();                                                                  \
  }
  LSA_MH_CASE(1) LSA_MH_CASE(2) LSA_MH_CASE(4) LSA_MH_CASE(8)
#undef LSA_MH_CASE
  return hipErrorNotSupported;
}

}  // namespace

bool score_mh_supported(int32_t heads, int32_t head_dim) {
  return (head_dim == 64 || head_dim == 128) &&
         (heads == 16 || heads == 32 || heads == 64 || heads == 128);
}

hipError_t launch_score_mh(const lsa_shape& s, int32_t layers, int32_t combine, int32_t heads,
                           int32_t head_dim, const void* q, const float* w, const void* rec,
                           const int32_t* chunk_off, float* scores, hipStream_t st) {
  if (head_dim == 128)
    return launch_mh_d<128>(s, layers, combine, heads, q, w, rec, chunk_off, scores, st);
  if (head_dim == 64)
    return launch_mh_d<64>(s, layers, combine, heads, q, w, rec, chunk_off, scores, st);
  return hipErrorNotSupported;
}

}  // namespace lsa
