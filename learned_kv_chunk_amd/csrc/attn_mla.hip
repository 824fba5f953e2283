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
// LDS with global_load_lds (no register staging), into one of four buffers,
// so three tiles are in flight while a fourth is computed.  Eight waves (two per
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
// MQA kernel.  Each pair writes the partial result of its own heads: the
// maximum and sum in fp32, the unnormalised output row rounded to bf16.
#include <math.h>

#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
constexpr int kRowVecs = kMlaDqk / 8;                 // 16-byte vectors per row (72)
constexpr int kPitch = kRowVecs * 16;                 // 1152-byte LDS rows, no padding
constexpr int kTileSlots = kTileTokens * kRowVecs;    // 2304 16-byte slots
constexpr int kTileInsts = kTileSlots / kWave;        // 36 DMA instructions per tile
constexpr int kDmaMax = (kTileInsts + kMlaWaves - 1) / kMlaWaves;  // 5 (waves 0-3), else 4
constexpr int kBufBytes = kTileSlots * 16;            // 36864
constexpr int kBufs = 4;                              // three tiles in flight
constexpr float kLazyLog2 = 8.f;  // reference-maximum slack of the online softmax (log2)

static_assert(kTileInsts * kWave == kTileSlots, "DMA instructions must tile the buffer");
static_assert(kTileInsts == 4 * 5 + 4 * 4, "waves 0-3 issue 5 loads per tile, waves 4-7 issue 4");
static_assert(kRowVecs % 8 == 0, "the swizzle permutes vectors inside aligned groups of 8");

// LDS layout of a tile: row r (token) at r * kPitch, its 16-byte vector v at
// slot v ^ swz(r) with swz(r) = r & 7 (so a vector stays in its aligned group
// of 8).  Both read patterns -- the K operand reads (16 consecutive rows, one
// vector each, per 16-lane group) and the transposed V reads (8 consecutive
// rows, one aligned vector pair each, per 32-lane group) -- then run without
// bank conflicts; this was measured with the SQ_LDS_BANK_CONFLICT counter on
// gfx950 for each pattern and several candidate swizzles (unpadded rows
// conflict on both; other XOR patterns that a 64-bank, 16-lanes-per-cycle
// model predicts conflict-free were not).
__device__ __forceinline__ int swz(int r) { return r & 7; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

struct TileInfo {
  int64_t row0;    // element row of the tile's first token in the K base
  int32_t nvalid;  // tokens of the tile inside the stream (0..32)
};

// One 16-byte-per-lane global -> LDS load: lane i's 16 bytes at sbase + voff
// land at LDS address lds_addr + 16 i (the address is taken from M0, which is
// restored afterwards).  The load carries the non-temporal hint: each K row is
// read once per step, and on cold rows at 1 x 1M the hint took the kernel from
// 36.8 to 33.3 us and the decode step from 58.4 to 57.1 us.  Written as inline assembly so that the compiler, which
// does not see the LDS write, adds no wait of its own for it before LDS reads:
// the pipeline below does its own counting.
__device__ __forceinline__ void dma16(const unsigned char* sbase, uint32_t voff,
                                      uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(sbase)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const unsigned char* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p));
}

// The slots this lane fills: DMA instruction j of wave w is instruction
// w + 8j of the tile (j < 5 for waves 0-3, j < 4 otherwise) and fills slots
// (w + 8j) * 64 .. +63, lane i slot (w + 8j) * 64 + i, which holds row
// slot / 72, vector (slot % 72) ^ swz(row).
struct DmaLane {
  uint32_t voff[kDmaMax];  // byte offset in a full tile
  int32_t rv[kDmaMax];     // row << 8 | vector
};

__device__ __forceinline__ DmaLane dma_lane(int64_t row_bytes, int wave, int lane) {
  DmaLane d;
#pragma unroll
  for (int j = 0; j < kDmaMax; ++j) {
    const int slot = min(wave + kMlaWaves * j, kTileInsts - 1) * kWave + lane;
    const int row = slot / kRowVecs;
    const int vec = (slot - row * kRowVecs) ^ swz(row);
    d.voff[j] = static_cast<uint32_t>(row * row_bytes) + vec * 16;
    d.rv[j] = (row << 8) | vec;
  }
  return d;
}

// Copy one tile (rows row0 .. row0+31; rows past nvalid repeat the last valid
// row) into an LDS buffer: ND instructions from this wave.
template <int ND>
__device__ __forceinline__ void dma_tile(const unsigned char* __restrict__ kbytes,
                                         int64_t row_bytes, const TileInfo& ti,
                                         const DmaLane& dl, const unsigned char* buf,
                                         int wave) {
  const uint64_t addr = reinterpret_cast<uint64_t>(kbytes) + static_cast<uint64_t>(ti.row0 * row_bytes);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  const unsigned char* sbase =
      reinterpret_cast<const unsigned char*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t lds0 = lds_address(buf) + wave * kWave * 16;
  if (ti.nvalid == kTileTokens) {
#pragma unroll
    for (int j = 0; j < ND; ++j)
      dma16(sbase, dl.voff[j], __builtin_amdgcn_readfirstlane(lds0 + j * kMlaWaves * kWave * 16));
  } else {
    const int last = ti.nvalid > 0 ? ti.nvalid - 1 : 0;
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int row = dl.rv[j] >> 8, vec = dl.rv[j] & 255;
      const uint32_t voff = static_cast<uint32_t>(min(row, last) * row_bytes) + vec * 16;
      dma16(sbase, voff, __builtin_amdgcn_readfirstlane(lds0 + j * kMlaWaves * kWave * 16));
    }
  }
}

// Copy the query rows of all heads (H rows of 1152 B, contiguous) into LDS
// at `dst` (two tile buffers hold the 64-row maximum) in the tiles' layout:
// LDS slot (row r, vector v) holds the row's vector v ^ swz(r), so that the
// operand reads below are conflict-free like the K reads.  Instruction j of
// wave w fills slots (w + 8j) * 64 .. +63.  Every wave issues kQDma
// instructions; a lane whose slot lies past the H rows re-reads the last 16
// bytes, so no read leaves the query array.
constexpr int kQDma = kMlaDqk * 2 * 64 / (kWave * 16) / kMlaWaves;  // 9
static_assert(kQDma * kMlaWaves * kWave * 16 == 2 * kBufBytes, "Q fills two tile buffers");

__device__ __forceinline__ void dma_q(const unsigned char* __restrict__ qbytes, int32_t q_bytes,
                                      const unsigned char* dst, int wave, int lane) {
  const uint64_t addr = reinterpret_cast<uint64_t>(qbytes);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(addr >> 32));
  const unsigned char* sbase =
      reinterpret_cast<const unsigned char*>((static_cast<uint64_t>(hi) << 32) | lo);
  const uint32_t lds0 = lds_address(dst);
#pragma unroll
  for (int j = 0; j < kQDma; ++j) {
    const int inst = wave + kMlaWaves * j;
    const int slot = inst * kWave + lane;
    const int row = slot / kRowVecs;
    const int32_t off =
        min(row * kPitch + ((slot - row * kRowVecs) ^ swz(row)) * 16, q_bytes - 16);
    dma16(sbase, static_cast<uint32_t>(off), __builtin_amdgcn_readfirstlane(lds0 + inst * kWave * 16));
  }
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then meet the other waves at a barrier.
#define LSA_MLA_WAIT_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" ::: "memory")
// Barrier after this wave's LDS writes have completed.
#define LSA_MLA_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// Per-lane LDS read addresses (byte offsets inside a tile buffer).
struct ReadLane {
  uint32_t k[2];  // K operand, steps s = 2q + r: k[r] + 128 q (+ 16 rows for half 1)
  uint32_t v[4];  // V^T operand, column groups cg = 4q + r: v[r] + 128 q (+ 16 rows)
};

// K operand of lane (r16, g): row r16, vector 4s + g.  V^T operand of lane
// (r16, g): rows 4g + (r16 >> 2) (and +16), the 8-byte piece 8 * (r16 & 3) of
// the 32-byte span of column group cg (vectors 2cg, 2cg + 1), in this wave's
// column half.  swz(r) depends on r & 7 only, so rows r and r + 16 share it.
__device__ __forceinline__ ReadLane read_lane(int col_half, int lane) {
  ReadLane rl;
  const int r16 = lane & 15, g = lane >> 4;
  const int fk = swz(r16);
#pragma unroll
  for (int r = 0; r < 2; ++r) rl.k[r] = r16 * kPitch + 16 * (g ^ (fk & 3)) + 64 * (r ^ (fk >> 2));
  const int row = 4 * g + (r16 >> 2);
  const int fv = swz(row);
  const int t = (r16 >> 1) & 1;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    rl.v[r] = row * kPitch + 512 * col_half + 32 * (r ^ (fv >> 1)) + 16 * (t ^ (fv & 1)) +
              8 * (r16 & 1);
  return rl;
}

// S^T for one 16-token half of a tile and the 16 heads of this wave:
// S^T[token][head] = K . Q^T over the 576 key dims (token = half*16 + lane%16,
// dims s*32 + 8g .. +7 in lane (r16, g)).  Operands are read nine at a time
// ahead of their products.
__device__ __forceinline__ f32x4 qk_half(const unsigned char* __restrict__ kt, int half,
                                         const ReadLane& rl, const bf16x8 (&qf)[kMlaDqk / 32]) {
  const unsigned char* kh = kt + half * 16 * kPitch;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < kMlaDqk / 32; s0 += 9) {
    u32x4 av[9];
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      const int s = s0 + u;
      av[u] = *reinterpret_cast<const u32x4*>(kh + rl.k[s & 1] + 128 * (s >> 1));
    }
#pragma unroll
    for (int u = 0; u < 9; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), qf[s0 + u], acc, 0, 0, 0);
  }
  return acc;
}

// Online softmax of one tile for this wave's 16 heads, given S^T of both
// halves, then O^T += V^T P^T over this wave's 256 latent columns.
// Lane (r16, g) holds tokens 4g..4g+3 (first half) and 16+4g..16+4g+3 (second
// half) of head r16, which is exactly its slice of the P^T operand.  The
// weights are taken against a reference maximum m that is raised only when a
// tile's maximum exceeds it by more than kLazyLog2, so weights stay below
// 2^kLazyLog2 and the accumulators are rescaled only on those tiles.
__device__ __forceinline__ void softmax_pv(const unsigned char* __restrict__ kt,
                                           const ReadLane& rl, f32x4 s0, f32x4 s1,
                                           int32_t nvalid, float& m, float& l,
                                           f32x4 (&o)[kMlaDv / 32], float scale_log2, int lane) {
  const int g = lane >> 4;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = ((j < 4) ? s0[j & 3] : s1[j & 3]) * scale_log2;
  if (nvalid < kTileTokens) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 16 * (j >> 2) + 4 * g + (j & 3);
      if (tok >= nvalid) x[j] = -INFINITY;
    }
  }
  float mt = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
  mt = xor32_max(xor16_max(mt));
  if (__ballot(mt > m + kLazyLog2) != 0) {
    const float m_new = (mt > m + kLazyLog2) ? mt : m;
    const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < kMlaDv / 32; ++c) o[c] *= alpha;
    m = m_new;
  }
  const float m_use = (m == -INFINITY) ? 0.f : m;
  bf16x8 pf;
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = __builtin_amdgcn_exp2f(x[j] - m_use);
    ps += p;
    pf[j] = static_cast<__bf16>(p);
  }
  l += ps;

  constexpr int kBatch = 8;  // column groups whose operands are read together
#pragma unroll
  for (int q = 0; q < kMlaDv / 32 / kBatch; ++q) {
    u32x4 vt[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const unsigned char* p0 = kt + rl.v[r & 3] + 128 * (q * (kBatch / 4) + (r >> 2));
      const u32x2 lo =
          __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 16 * kPitch)));
      vt[r] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      o[q * kBatch + r] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vt[r]), pf, o[q * kBatch + r], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kMlaThreads, 1) void attn_mla_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kBufs * kBufBytes];
  __shared__ __attribute__((aligned(16))) f32x4 s_xch[kMlaWaves][kWave];  // S^T halves
  __shared__ int32_t s_slot[kMaxRunSlots];  // the run's kept-chunk indices
  __shared__ AttnRun s_run;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int hg = wave >> 1;    // head group: heads 16 hg .. 16 hg + 15
  const int half = wave & 1;   // token half of S^T and column half of O^T

  const AttnRun run = attn_prologue(a, s_slot, &s_run);
  if (run.b < 0) return;
  const int32_t b = run.b;
  const int32_t tpc = a.tiles_per_chunk, C = a.C, H = a.H;
  const int32_t sel0 = run.sel0;
  const int32_t t_begin = run.t_begin;
  const int32_t t_end = run.t_end;
  const int32_t slot_first = run.slot_first;
  const int64_t tb = run.tb;
  const int64_t len = run.len;
  const int64_t last_chunk = len > 0 ? (len - 1) / C : 0;
  const int head = hg * 16 + r16;
  const bool active = hg * 16 < H;  // wave-uniform

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

  // Four-buffer pipeline: tiles i+1, i+2 and (issued during iteration i)
  // i+3 are in flight while tile i is computed.  Each wave issues a fixed
  // number nd of loads per tile (5 for waves 0-3, 4 for waves 4-7) and no
  // other vector-memory operation inside the loop, so "tile i has landed" is
  // "at most nd times the number of later tiles issued of this wave's loads
  // outstanding", and the first barrier makes every wave's part of tile i
  // visible.  The buffer refilled with tile i+3 held tile i-1 (for i = 0 the
  // query), which every wave finished before that barrier.  The second
  // barrier publishes the S^T halves; a half is rewritten only after the next
  // first barrier, which its reader reaches after reading it.
  const DmaLane dl = dma_lane(row_bytes, wave, lane);
  const ReadLane rl = read_lane(half, lane);
  const bool five = wave < 4;  // wave-uniform: 5 loads per tile, else 4
  auto issue = [&](int32_t t, int slot) {
    const TileInfo ti = tile_info(t_begin + t);
    if (five) dma_tile<5>(kbytes, row_bytes, ti, dl, smem + slot * kBufBytes, wave);
    else dma_tile<4>(kbytes, row_bytes, ti, dl, smem + slot * kBufBytes, wave);
    return ti.nvalid;
  };
  const int32_t n = t_end - t_begin;
  int32_t nv[kBufs] = {0, 0, 0, 0};  // valid tokens of the tile in each buffer

  // Start-up.  The query rows of the stream go to buffers 2-3 through the same
  // copy path, ahead of tiles 0 and 1 (buffers 0-1); once the query has landed
  // every wave takes its Q^T operand from LDS (lane (r16, g) holds
  // Q[head][s*32 + 8g .. +7]), and only then is tile 2 issued into buffer 2,
  // tile 3 following in the loop's first iteration.  So the first tile is
  // waited for alone rather than with all three, and one coalesced copy per
  // workgroup replaces per-wave query loads of 64-byte pieces.
  bf16x8 qf[kMlaDqk / 32];
  {
    const unsigned char* qbytes =
        static_cast<const unsigned char*>(a.q) + static_cast<int64_t>(b) * H * kMlaDqk * 2;
    const unsigned char* qs = smem + 2 * kBufBytes;
    dma_q(qbytes, H * kMlaDqk * 2, qs, wave, lane);
    if (0 < n) nv[0] = issue(0, 0);
    if (1 < n) nv[1] = issue(1, 1);
    if (n >= 2) {
      if (five) LSA_MLA_WAIT_BARRIER(10);
      else LSA_MLA_WAIT_BARRIER(8);
    } else if (n == 1) {
      if (five) LSA_MLA_WAIT_BARRIER(5);
      else LSA_MLA_WAIT_BARRIER(4);
    } else {
      LSA_MLA_WAIT_BARRIER(0);
    }
    const int qr = min(head, H - 1);
    const unsigned char* qrow = qs + qr * kPitch;
#pragma unroll
    for (int s = 0; s < kMlaDqk / 32; ++s)
      qf[s] = as_bf16x8(head < H ? *reinterpret_cast<const u32x4*>(
                                       qrow + 16 * ((4 * s + g) ^ swz(qr)))
                                 : u32x4{0u, 0u, 0u, 0u});
    LSA_MLA_BARRIER();  // buffers 2-3 are free once every wave holds its Q
    if (2 < n) nv[2] = issue(2, 2);
  }

  for (int32_t i = 0; i < n; ++i) {
    const int32_t later = min(n - 1 - i, kBufs - 2);  // tiles issued after tile i
    if (later == 2) {
      if (five) LSA_MLA_WAIT_BARRIER(10);
      else LSA_MLA_WAIT_BARRIER(8);
    } else if (later == 1) {
      if (five) LSA_MLA_WAIT_BARRIER(5);
      else LSA_MLA_WAIT_BARRIER(4);
    } else {
      LSA_MLA_WAIT_BARRIER(0);
    }
    const int buf = i & (kBufs - 1);
    const unsigned char* kt = smem + buf * kBufBytes;
    f32x4 s_mine = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      s_mine = qk_half(kt, half, rl, qf);
      s_xch[wave][lane] = s_mine;
    }
    // the copies of tile i+3 go out after this wave's S^T products, so that a
    // wave stalled on a full memory queue does not hold up its products
    // (measured: 1.2 % shorter at 1 x 1M than issuing them first)
    if (i + kBufs - 1 < n) {
      const int nb = (i + kBufs - 1) & (kBufs - 1);
      nv[nb] = issue(i + kBufs - 1, nb);
    }
    LSA_MLA_BARRIER();
    if (active) {
      const f32x4 s_other = s_xch[wave ^ 1][lane];
      softmax_pv(kt, rl, half ? s_other : s_mine, half ? s_mine : s_other, nv[buf], m, l, o,
                 a.scale_log2, lane);
    }
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
  // The output rows as bf16 (64 KiB per workgroup at 64 heads), written
  // through in 16-byte pieces.  Lane (r16, g) holds columns 4g .. 4g+3 of
  // each 16-column block; for a pair of blocks (c, c+1) one permlane16_swap
  // per 32-bit word hands an even-row lane (g = 0, 2) columns 4g .. 4g+7 of
  // block c and an odd-row lane columns 4(g-1) .. 4g+3 of block c+1.
  unsigned char* ob = reinterpret_cast<unsigned char*>(a.ws_o) + wg * H * kMlaDv * 2;
  const int odd = g & 1;
#pragma unroll
  for (int c = 0; c < kMlaDv / 32; c += 2) {
    const st_u32x2 pa = __builtin_bit_cast(st_u32x2, __builtin_convertvector(o[c], bf16x4));
    const st_u32x2 pb = __builtin_bit_cast(st_u32x2, __builtin_convertvector(o[c + 1], bf16x4));
    const auto x = __builtin_amdgcn_permlane16_swap(pa.x, pb.x, false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(pa.y, pb.y, false, false);
    const int col = half * (kMlaDv / 2) + 16 * (c + odd) + 8 * (g >> 1);
    store_through_16(reinterpret_cast<float*>(ob), static_cast<uint32_t>((head * kMlaDv + col) * 2),
                     st_u32x4{x[0], y[0], x[1], y[1]});
  }
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
