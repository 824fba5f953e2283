// attn_mla.hip -- split-KV sparse decode attention on the matrix cores for
// absorbed multi-head latent attention: every query head attends to one
// shared latent row per token, K = [latent (512) | rope key (64)] (576 bf16)
// and V = the latent itself (the first 512 columns of the same row), so the
// cache holds each token once.
//
// Dimensionstp review, section 3-2-3 steps 6-7: softmax attention restricted
// to the kept chunks; the cache seen as chunk memory is the compressed
// attention cache of section 3-2-1.
//
// A workgroup owns a run of 32-token tiles of one stream and all (up to 64)
// query heads.  Each tile is read from HBM once per workgroup, straight into
// LDS with global_load_lds (no register staging), into one of three buffers,
// so two tiles are in flight while a third is computed.  Eight waves (two per
// SIMD) work in pairs: the pair (2h, 2h+1) serves heads 16h..16h+15, each
// wave of the pair computes S^T for one 16-token half of the tile
//   S^T[token][head] = K_tile . Q^T     (v_mfma_f32_16x16x32_bf16, K = 576)
// the halves are swapped through LDS, both waves run the same fp32 online
// softmax (exp2 domain, weights rounded to bf16), and each accumulates one
// half of the latent columns
//   O^T[col][head]  += V_tile^T . P^T    (v_mfma_f32_16x16x32_bf16, K = tokens)
// so the matrix work is split evenly with nothing computed twice, and a wave
// holds 64 accumulator registers.  The transposed products keep the softmax
// state of a head in one lane (no cross-lane traffic to rescale), as in the
// MQA kernel.  Each pair writes the partial result of its own heads.
#include <math.h>

#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaWaves = 8;  // two per SIMD: (head group, half) pairs
constexpr int kMlaThreads = kMlaWaves * kWave;
constexpr int kRowVecs = kMlaDqk / 8;                        // 16-byte vectors per row (72)
constexpr int kPitchVecs = kRowVecs + 1;                     // padded LDS row (73 vectors)
constexpr int kPitch = kPitchVecs * 16;                      // 1168 bytes
constexpr int kTileSlots = kTileTokens * kPitchVecs;         // 2336 16-byte slots
constexpr int kDmaPerWave = (kTileSlots + kMlaThreads - 1) / kMlaThreads;  // 5
constexpr int kBufBytes = kMlaWaves * kDmaPerWave * kWave * 16;            // 40960
constexpr int kBufs = 3;

// s_waitcnt immediate (gfx9 encoding) waiting for every vector-memory
// operation, leaving the export and LDS/scalar counters unconstrained.
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);

static_assert(kTileSlots <= kMlaWaves * kDmaPerWave * kWave, "tile does not fit the DMA slots");
static_assert(kDmaPerWave == 5, "the pipeline waits below count 5 loads per tile");

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct TileInfo {
  int64_t row0;    // element row of the tile's first token in the K base
  int32_t nvalid;  // tokens of the tile inside the stream (0..32)
};

// One 16-byte-per-lane global -> LDS load: lane i's 16 bytes at sbase + voff
// land at LDS address lds_addr + 16 i.  Written as inline assembly so that the
// compiler, which does not see the LDS write, adds no wait of its own for it
// before LDS reads: the pipeline below does its own counting.
__device__ __forceinline__ void dma16(const unsigned char* sbase, uint32_t voff,
                                      uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(sbase)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const unsigned char* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p));
}

// Copy one tile (rows row0 .. row0+31, rows past nvalid repeat the last valid
// row) into an LDS buffer with padded rows.  Each DMA instruction fills 64
// consecutive 16-byte slots, lane i writing slot i; slot s of the buffer is
// row s / 73, vector s % 73 (vector 72 is the pad, and slots past the tile
// load the tile's first vector).
__device__ __forceinline__ void dma_tile(const unsigned char* __restrict__ kbytes,
                                         int64_t row_bytes, const TileInfo& ti,
                                         const unsigned char* buf, int wave, int lane) {
  const int last = ti.nvalid > 0 ? ti.nvalid - 1 : 0;
  const uint64_t addr = reinterpret_cast<uint64_t>(kbytes) + static_cast<uint64_t>(ti.row0 * row_bytes);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  const unsigned char* sbase =
      reinterpret_cast<const unsigned char*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t lds0 = lds_address(buf);
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int inst = wave * kDmaPerWave + j;
    const int slot = inst * kWave + lane;
    const int row = slot / kPitchVecs;
    const int vec = slot - row * kPitchVecs;
    const bool real = row < kTileTokens && vec < kRowVecs;
    const uint32_t voff =
        real ? static_cast<uint32_t>(min(row, last) * row_bytes) + vec * 16 : 0u;
    dma16(sbase, voff, __builtin_amdgcn_readfirstlane(lds0 + inst * kWave * 16));
  }
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then meet the other waves at a barrier.
#define LSA_MLA_WAIT_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory")
// Barrier after this wave's LDS writes have completed.
#define LSA_MLA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// S^T for one 16-token half of a tile and the 16 heads of this wave:
// S^T[token][head] = K . Q^T over the 576 key dims.  The K operand of a lane is
// token (half*16 + lane%16), dims s*32 + 8g .. +7; all 18 operands are read
// before the products so the LDS latency is paid once.
__device__ __forceinline__ f32x4 qk_half(const unsigned char* __restrict__ kt, int half,
                                         const bf16x8 (&qf)[kMlaDqk / 32], int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  const unsigned char* ka = kt + (half * 16 + r16) * kPitch + g * 16;
  u32x4 av[kMlaDqk / 32];
#pragma unroll
  for (int s = 0; s < kMlaDqk / 32; ++s) av[s] = *reinterpret_cast<const u32x4*>(ka + s * 64);
  __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMlaDqk / 32; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[s]), qf[s], acc, 0, 0, 0);
  return acc;
}

// Online softmax of one tile for this wave's 16 heads, given S^T of both
// halves, then O^T += V^T P^T over this wave's 256 latent columns.
// Lane (r16, g) holds tokens 4g..4g+3 (first half) and 16+4g..16+4g+3 (second
// half) of head r16, which is exactly its slice of the P^T operand.
__device__ __forceinline__ void softmax_pv(const unsigned char* __restrict__ kt, int col_half,
                                           f32x4 s0, f32x4 s1, int32_t nvalid, float& m,
                                           float& l, f32x4 (&o)[kMlaDv / 32], float scale_log2,
                                           int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = 16 * (j >> 2) + 4 * g + (j & 3);
    const float sv = (j < 4) ? s0[j & 3] : s1[j & 3];
    x[j] = (tok < nvalid) ? sv * scale_log2 : -INFINITY;
  }
  float mt = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
  mt = xor32_max(xor16_max(mt));
  const float m_new = fmaxf(m, mt);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m - m_use);
  bf16x8 pf;
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - m_use);
    ps += p;
    pf[j] = static_cast<__bf16>(p);
  }
  l = fmaf(l, alpha, ps);
  m = m_new;

  // ds_read_b64_tr_b16 gives lane i of a 16-lane group element (i & 3) of the
  // 8-byte chunk addressed by lane 4j + (i >> 2) of the group, as its element
  // j: lane s of group g addresses row 4g + (s >> 2) (and +16), columns
  // c0 + 4*(s & 3) .. +3 of the 16-column group starting at c0.
  const unsigned char* vrow =
      kt + (4 * g + (r16 >> 2)) * kPitch + 8 * (r16 & 3) + col_half * (kMlaDv / 2) * 2;
  constexpr int kBatch = 8;  // column groups whose operands are read together
#pragma unroll
  for (int c0 = 0; c0 < kMlaDv / 32; c0 += kBatch) {
    u32x4 vt[kBatch];
#pragma unroll
    for (int c = 0; c < kBatch; ++c) {
      const unsigned char* p0 = vrow + (c0 + c) * 32;
      const u32x2 lo =
          __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * kPitch)));
      vt[c] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int c = 0; c < kBatch; ++c)
      o[c0 + c] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt[c]), pf, o[c0 + c] * alpha, 0, 0, 0);
  }
}

__global__ __launch_bounds__(kMlaThreads, 1) void attn_mla_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBufs * kBufBytes];
  __shared__ __attribute__((aligned(16))) f32x4 s_xch[kMlaWaves][kWave];  // S^T halves
  __shared__ int32_t s_plan[3];
  __shared__ int32_t s_slot[kMaxRunSlots];  // the run's kept-chunk indices

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int hg = wave >> 1;    // head group: heads 16 hg .. 16 hg + 15
  const int half = wave & 1;   // token half of S^T and column half of O^T

  if (wave == 0) {
    int32_t b, local;
    StreamSplit sp;
    find_stream_of_wg(a.sel_off, a.B, a.tiles_per_chunk, a.per, a.target, blockIdx.x, &b,
                      &local, &sp);
    if (lane == 0) {
      s_plan[0] = b;
      s_plan[1] = local * sp.per;                       // first tile
      s_plan[2] = min(sp.tiles, (local + 1) * sp.per);  // end tile
    }
  }
  __syncthreads();
  const int32_t b = s_plan[0];
  if (b < 0) return;
  const int32_t tpc = a.tiles_per_chunk, C = a.C, H = a.H;
  const int32_t sel0 = a.sel_off[b];
  const int32_t t_begin = s_plan[1];
  const int32_t t_end = s_plan[2];
  const int32_t slot_first = t_begin / tpc;
  const int32_t nslots = (t_end - 1) / tpc - slot_first + 1;
  for (int32_t i = tid; i < min(nslots, kMaxRunSlots); i += kMlaThreads)
    s_slot[i] = a.sel_idx[sel0 + slot_first + i];
  const int64_t tb = a.tok_off[b];
  const int64_t len = a.tok_off[b + 1] - tb;
  const int64_t last_chunk = len > 0 ? (len - 1) / C : 0;
  const int head = hg * 16 + r16;
  const bool active = hg * 16 < H;  // wave-uniform
  __syncthreads();

  // tile t of the run: an empty tile (past the end of a partial chunk) points
  // at its chunk's first row with nvalid = 0; a kept index outside [0, N_b)
  // (a violated precondition) is clamped so that no read leaves the stream
  auto tile_info = [&](int32_t t) {
    TileInfo ti;
    const int32_t j = t / tpc;
    const int32_t sub = t - j * tpc;
    int64_t n = s_slot[min(j - slot_first, kMaxRunSlots - 1)];
    n = n < 0 ? 0 : (n > last_chunk ? last_chunk : n);
    int64_t valid = len - n * C;
    if (valid > C) valid = C;
    valid -= static_cast<int64_t>(sub) * kTileTokens;
    const int64_t chunk_row = a.pool ? static_cast<int64_t>(sel0 + j) * C : tb + n * C;
    if (valid <= 0) {
      ti.nvalid = 0;
      ti.row0 = chunk_row;
    } else {
      ti.nvalid = valid > kTileTokens ? kTileTokens : static_cast<int32_t>(valid);
      ti.row0 = chunk_row + sub * kTileTokens;
    }
    return ti;
  };

  const unsigned char* __restrict__ kbytes = static_cast<const unsigned char*>(a.k);
  const int64_t row_bytes = static_cast<int64_t>(a.k_row) * 2;

  float m = -INFINITY, l = 0.f;
  f32x4 o[kMlaDv / 32];
#pragma unroll
  for (int c = 0; c < kMlaDv / 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Three-buffer pipeline: tiles i+1 and i+2 are in flight while tile i is
  // computed.  Each wave issues exactly kDmaPerWave loads per tile and no
  // other vector-memory operation inside the loop, so "tile i has landed" is
  // "at most kDmaPerWave of this wave's loads outstanding" (the loads of tile
  // i+1), and the first barrier makes every wave's part of tile i visible.
  // The buffer refilled with tile i+2 held tile i-1, which every wave finished
  // before that barrier.  The second barrier publishes the S^T halves; a half
  // is rewritten only after the next first barrier, which its reader reaches
  // after reading it.
  const int32_t n = t_end - t_begin;
  int32_t nv0 = 0, nv1 = 0, nv2 = 0;  // valid tokens of tiles i, i+1, i+2
  if (n > 0) {
    const TileInfo t0 = tile_info(t_begin);
    nv0 = t0.nvalid;
    dma_tile(kbytes, row_bytes, t0, smem, wave, lane);
  }
  if (n > 1) {
    const TileInfo t1 = tile_info(t_begin + 1);
    nv1 = t1.nvalid;
    dma_tile(kbytes, row_bytes, t1, smem + kBufBytes, wave, lane);
  }

  // Q^T operand of this wave's heads: lane holds Q[head][s*32 + 8g .. +7].
  // Loaded after the first two tiles' copies are under way and waited for
  // together with them, so the loop holds no compiler-tracked load.
  bf16x8 qf[kMlaDqk / 32];
  {
    const uint16_t* __restrict__ qb = static_cast<const uint16_t*>(a.q);
    const u32x4* src = reinterpret_cast<const u32x4*>(
                           qb + (static_cast<int64_t>(b) * H + min(head, H - 1)) * kMlaDqk) + g;
#pragma unroll
    for (int s = 0; s < kMlaDqk / 32; ++s)
      qf[s] = as_bf16x8(head < H ? src[s * 4] : u32x4{0u, 0u, 0u, 0u});
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  int buf = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (i + 1 < n) LSA_MLA_WAIT_BARRIER(5);
    else LSA_MLA_WAIT_BARRIER(0);
    if (i + 2 < n) {
      const int nb = buf >= 1 ? buf - 1 : kBufs - 1;  // (i + 2) % 3
      const TileInfo t2 = tile_info(t_begin + i + 2);
      nv2 = t2.nvalid;
      dma_tile(kbytes, row_bytes, t2, smem + nb * kBufBytes, wave, lane);
    }
    const unsigned char* kt = smem + buf * kBufBytes;
    f32x4 s_mine = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      s_mine = qk_half(kt, half, qf, lane);
      s_xch[wave][lane] = s_mine;
    }
    LSA_MLA_BARRIER();
    if (active) {
      const f32x4 s_other = s_xch[wave ^ 1][lane];
      softmax_pv(kt, half, half ? s_other : s_mine, half ? s_mine : s_other, nv0, m, l, o,
                 a.scale_log2, lane);
    }
    nv0 = nv1;
    nv1 = nv2;
    buf = buf + 1 == kBufs ? 0 : buf + 1;
  }

  if (!active || head >= H) return;
  const int64_t wg = blockIdx.x;
  if (half == 0) {
    const float lt = xor32_sum(xor16_sum(l));
    if (g == 0) {
      a.ws_m[wg * H + head] = m;
      a.ws_l[wg * H + head] = lt;
    }
  }
  float* orow = a.ws_o + (wg * H + head) * kMlaDv + half * (kMlaDv / 2) + 4 * g;
#pragma unroll
  for (int c = 0; c < kMlaDv / 32; ++c) *reinterpret_cast<f32x4*>(orow + c * 16) = o[c];
}

}  // namespace

// bf16, K = [latent | rope] of 576, V aliasing the first 512 columns, 1..64
// query heads.
bool mla_attn_supported(const lsa_shape& s) {
  return s.dtype == LSA_DTYPE_BF16 && s.v_aliases_k && s.head_dim_qk == kMlaDqk &&
         s.head_dim_v == kMlaDv && s.num_q_heads >= 1 && s.num_q_heads <= 8 * kMlaWaves;
}

hipError_t launch_attn_mla(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st) {
  if (!mla_attn_supported(s)) return hipErrorNotSupported;
  hipLaunchKernelGGL(attn_mla_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kMlaThreads), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace lsa
