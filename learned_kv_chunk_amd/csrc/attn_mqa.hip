// attn_mqa.hip -- split-KV sparse decode attention on the matrix cores for
// multi-query attention (all query heads share one KV head), bf16 inputs,
// head_dim_qk == head_dim_v == D in {64, 128}.
//
// Dimensionstp review, section 3-2-3 steps 6-7: softmax attention restricted
// to the kept chunks.  Per 32-token tile and group of 16 heads a wave does
//   S^T[token][head] = K_tile . Q^T        (v_mfma_f32_16x16x32_bf16, K = d)
//   online softmax in fp32 (exp2 domain), weights rounded to bf16
//   O^T[col][head]  += V_tile^T . P^T       (v_mfma_f32_16x16x32_bf16, K = tokens)
// Computing the transposed products makes the softmax state line up with the
// matrix-core register layouts: in S^T's accumulator a lane holds four tokens
// of one head (head = lane % 16), which is exactly the lane's slice of the P^T
// operand of the second product, and the O^T accumulator keeps one head per
// lane, so rescaling by the running maximum needs no cross-lane traffic.
// K tiles are loaded straight from HBM into the operand registers (each load
// instruction covers 16 rows x 64 contiguous bytes); V tiles go through a
// per-wave LDS buffer because the second product contracts over tokens,
// which are strided in memory.  Each wave software-pipelines its tiles: the
// next tile's loads are in flight while the current one is computed.
// A workgroup has four waves, one per SIMD: for up to 32 heads each wave
// serves every head group, and up to 64 heads two teams of two waves each
// serve half of them.  Measured on cold K/V, four waves stream faster than
// eight (two per SIMD) even for one head group, where eight would fit: at
// 16 x 128K, 30.2 us per launch against 31.6 for eight waves, each with the
// load hints that suit it best; more loads in flight per CU only lengthen
// the memory queues (a third register set per wave: 32.4 us).  The
// waves of a team take interleaved tiles of the workgroup's run, then merge
// their (max, sum, output) states through LDS into one partial result.  When
// streams average few workgroups the stream's partials are combined by its
// last workgroup to finish (arrival counter with release / acquire ordering
// at device scope, merge_stream_block), so attention is one launch, and a
// stream served by a single workgroup writes its output directly; otherwise
// the merge launch of attn_common.hip combines them.
#include <math.h>

#include "lsa_internal.hpp"
#include "select_core.hpp"
#include "wave.hpp"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// LDS row pitch of a staged V tile: D bf16 plus 32 bytes, so that the eight
// rows one transposed read touches per half-wave start in distinct 8-bank
// windows.
template <int D>
constexpr int v_row_bytes() { return 2 * D + 32; }


__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
struct TileRegs {
  u32x4 k[2][D / 32];  // K operand: token block (16 rows) x 32-wide d step
  u32x4 v[D / 16];     // V tile pieces (16 bytes each), written to LDS later
};

struct TileInfo {
  int64_t row0;    // element row of the tile's first token in the K/V base
  int32_t nvalid;  // tokens of the tile inside the stream (0..32)
};

// Loads are unconditional so that the compiler can count them and keep the
// next tile in flight: rows past the tile's valid tokens re-read its last
// valid row (their logits are masked and their weights are zero).  V is read
// with the non-temporal hint.  K carries it too when a wave serves one head
// group (KNT): each K load instruction covers half of every 128-byte line it
// touches and the next one the other half, and measured on cold K/V the hint
// pays only there (16 x 128K: 30.2 us against 31.4 without it; 32 ragged
// streams: 65.5 against 64.7, a 1 % loss; eight waves per workgroup: 32.7
// against 31.6; a wave serving two groups, 4 x 512K pool: 28.3 against 27.5).
template <int D, bool KNT>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ kb,
                                           const uint16_t* __restrict__ vb, int32_t k_row,
                                           int32_t v_row, const TileInfo& ti, TileRegs<D>& r,
                                           int lane) {
  constexpr int PR = D / 8;  // 16-byte pieces per row
  const int r16 = lane & 15, g = lane >> 4;
  const int last = ti.nvalid > 0 ? ti.nvalid - 1 : 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int row = min(blk * 16 + r16, last);
    const u32x4* src = reinterpret_cast<const u32x4*>(kb + (ti.row0 + row) * k_row) + g;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      r.k[blk][s] = KNT ? __builtin_nontemporal_load(src + s * 4) : src[s * 4];
  }
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int flat = i * kWave + lane;
    const int row = min(flat / PR, last), c16 = flat % PR;
    r.v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(vb + (ti.row0 + row) * v_row) + c16);
  }
}

template <int D, int NHG>
__device__ __forceinline__ void compute_tile(const TileRegs<D>& r, int32_t nvalid,
                                             const bf16x8 (&qf)[NHG][D / 32], float (&m)[NHG],
                                             float (&l)[NHG], f32x4 (&o)[NHG][D / 16],
                                             unsigned char* __restrict__ sv, float scale_log2,
                                             int lane) {
  constexpr int PR = D / 8;
  constexpr int ROWB = v_row_bytes<D>();
  const int r16 = lane & 15, g = lane >> 4;

  // S^T = K Q^T for both 16-token blocks and every head group
  f32x4 sacc[NHG][2];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[blk][s]), qf[hg][s], acc, 0,
                                                      0, 0);
      sacc[hg][blk] = acc;
    }

  // V tile -> this wave's LDS buffer (row-major, padded rows)
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int flat = i * kWave + lane;
    const int row = flat / PR, c16 = flat % PR;
    *reinterpret_cast<u32x4*>(sv + row * ROWB + c16 * 16) = r.v[i];
  }

  // online softmax; the lane's eight weights form its P^T operand directly
  bf16x8 pf[NHG];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 16 * (j >> 2) + 4 * g + (j & 3);
      x[j] = (tok < nvalid) ? sacc[hg][j >> 2][j & 3] * scale_log2 : -INFINITY;
    }
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt = xor32_max(xor16_max(mt));
    const float m_new = fmaxf(m[hg], mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m[hg] - m_use);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(x[j] - m_use);
      ps += p;
      pf[hg][j] = static_cast<__bf16>(p);
    }
    l[hg] = fmaf(l[hg], alpha, ps);
    m[hg] = m_new;
#pragma unroll
    for (int cg = 0; cg < D / 16; ++cg) o[hg][cg] *= alpha;
  }

  // O^T += V^T P^T.  The V^T operand of a lane is column cg*16 + lane%16 at
  // the eight tokens that pair with its weights (4g..4g+3, 16+4g..16+4g+3).
  // ds_read_b64_tr_b16 gives lane i of a 16-lane group element (i & 3) of the
  // 8-byte chunk addressed by lane 4j + (i >> 2) of the group, as its element
  // j; so lane s of group g addresses row 4g + (s >> 2) (+16), columns
  // cg*16 + 4*(s & 3) .. +3.
  const unsigned char* vrow = sv + (4 * g + (r16 >> 2)) * ROWB + 8 * (r16 & 3);
#pragma unroll
  for (int cg = 0; cg < D / 16; ++cg) {
    const unsigned char* p0 = vrow + cg * 32;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(p0 + 16 * ROWB));
    u32x4 packed;
    packed.x = static_cast<uint16_t>(lo.x) | (static_cast<uint32_t>(static_cast<uint16_t>(lo.y)) << 16);
    packed.y = static_cast<uint16_t>(lo.z) | (static_cast<uint32_t>(static_cast<uint16_t>(lo.w)) << 16);
    packed.z = static_cast<uint16_t>(hi.x) | (static_cast<uint32_t>(static_cast<uint16_t>(hi.y)) << 16);
    packed.w = static_cast<uint16_t>(hi.z) | (static_cast<uint32_t>(static_cast<uint16_t>(hi.w)) << 16);
    const bf16x8 vt = as_bf16x8(packed);
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
      o[hg][cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pf[hg], o[hg][cg], 0, 0, 0);
  }
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Waves per workgroup: one per SIMD.
template <int NHG>
constexpr int mqa_waves() { return 4; }
constexpr int kMqaThreads = 4 * kWave;

template <int D, int NHG>
struct MqaLds {
  static constexpr int kWaves = mqa_waves<NHG>();
  static constexpr int kRowBytes = v_row_bytes<D>();
  static constexpr int kTileBytes = kTileTokens * kRowBytes;              // per wave
  static constexpr int kStateO = NHG * (D / 16) * kWave * 16;            // lane-major o
  static constexpr int kStateBytes = kStateO + 2 * NHG * kWave * 4;      // + m, l
  static constexpr int kBytes = cmax(kWaves * kTileBytes, kWaves * kStateBytes);
};

template <int D, int NHG>
__device__ __forceinline__ void store_state(unsigned char* base, const float (&m)[NHG],
                                            const float (&l)[NHG], const f32x4 (&o)[NHG][D / 16],
                                            int lane) {
  using L = MqaLds<D, NHG>;
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
#pragma unroll
    for (int cg = 0; cg < D / 16; ++cg)
      reinterpret_cast<f32x4*>(base)[(hg * (D / 16) + cg) * kWave + lane] = o[hg][cg];
    reinterpret_cast<float*>(base + L::kStateO)[hg * kWave + lane] = m[hg];
    reinterpret_cast<float*>(base + L::kStateO)[(NHG + hg) * kWave + lane] = l[hg];
  }
}

// Combines the WPG states a team stored (store_state, one slot per wave from
// `team`) for column blocks cb0 .. cb0 + CPW - 1 of every head group: per
// lane the maximum m, the rescaled sum l over the head's lanes (lt), and
// the rescaled output blocks (os).
template <int D, int NHG, int WPG, int CPW>
__device__ __forceinline__ void team_states(const unsigned char* team, int cb0, float (&m)[NHG],
                                            float (&lt)[NHG], f32x4 (&os)[NHG][CPW], int lane) {
  using L = MqaLds<D, NHG>;
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    float mw[WPG], fw[WPG];
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPG; ++w) {
      mw[w] = reinterpret_cast<const float*>(team + w * L::kStateBytes + L::kStateO)[hg * kWave +
                                                                                    lane];
      mx = fmaxf(mx, mw[w]);
    }
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < WPG; ++w) {
      fw[w] = __builtin_amdgcn_exp2f(mw[w] - mu);
      ls = fmaf(reinterpret_cast<const float*>(team + w * L::kStateBytes +
                                               L::kStateO)[(NHG + hg) * kWave + lane],
                fw[w], ls);
    }
    m[hg] = mx;
    lt[hg] = xor32_sum(xor16_sum(ls));
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < WPG; ++w)
        acc += reinterpret_cast<const f32x4*>(team + w * L::kStateBytes)
                   [(hg * (D / 16) + cb0 + c) * kWave + lane] * fw[w];
      os[hg][c] = acc;
    }
  }
}

// Each wave serves NHG groups of 16 heads.  The workgroup's waves form HS
// teams; team t serves head groups t*NHG .. t*NHG + NHG - 1 and its waves
// interleave the run's tiles among themselves, so a tile is read once per team
// (HS = 1 except for more than 32 heads).
// KSEL > 0: the workgroup ranks its stream's kept chunks itself in the
// prologue (KSEL keys per thread, attn_select_stream) instead of reading them.
template <int D, int NHG, int HS, int KSEL>
__global__ __launch_bounds__(mqa_waves<NHG>() * kWave, 1) void attn_mqa_kernel(
    AttnArgs a) {
  using L = MqaLds<D, NHG>;
  constexpr int NW = L::kWaves;
  constexpr int WPG = NW / HS;  // waves per team
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::kBytes];
  __shared__ int32_t s_slot[kMaxRunSlots];  // the run's kept-chunk indices
  __shared__ AttnRun s_run;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int grp = wave / WPG;  // team of this wave
  const int wl = wave % WPG;   // index among the team's waves

  const AttnRun run = attn_prologue(a, s_slot, &s_run);
  if (run.b < 0) return;
  const int32_t b = run.b;
  const int32_t tpc = a.tiles_per_chunk, C = a.C, H = a.H;

  // Q^T operand: lane holds Q[head][s*32 + 8*(lane/16) + 0..7] for the heads
  // (grp*NHG + hg)*16 + lane%16 of its team (loaded before an in-kernel
  // top-k, whose latency then covers theirs)
  const int head0 = grp * NHG * 16 + r16;
  const uint16_t* __restrict__ qb = static_cast<const uint16_t*>(a.q);
  bf16x8 qf[NHG][D / 32];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int head = head0 + hg * 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(
                           qb + (static_cast<int64_t>(b) * H + min(head, H - 1)) * D) + g;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[hg][s] = as_bf16x8(head < H ? src[s * 4] : u32x4{0u, 0u, 0u, 0u});
  }
  if constexpr (KSEL > 0)  // the V tile buffers are free until the first tile
    attn_select_stream<NW * kWave, KSEL>(a, run, s_slot,
                                         *reinterpret_cast<SelectLds<NW * kWave>*>(smem));
  const int32_t sel0 = run.sel0;
  const int32_t t_begin = run.t_begin;
  const int32_t t_end = run.t_end;
  // s_slot holds the run's kept chunks, or the whole stream's when selected here
  const int32_t slot_first = KSEL > 0 ? 0 : run.slot_first;
  const int64_t tb = run.tb;
  const int64_t len = run.len;
  const int64_t last_chunk = len > 0 ? (len - 1) / C : 0;

  // Tile i of this wave is t_begin + wl + WPG*i.  An empty tile (past the end
  // of a partial chunk) points at its chunk's first row with nvalid = 0.
  // A team whose heads all lie past H (only with HS > 1) skips the work.
  const int32_t n_mine = grp * NHG * 16 < H ? (t_end - t_begin - wl + WPG - 1) / WPG : 0;
  auto tile_info = [&](int32_t i) {
    TileInfo ti;
    const int32_t t = t_begin + wl + WPG * i;
    const int32_t j = t / tpc;
    const int32_t sub = t - j * tpc;
    // a kept index outside [0, N_b) (a violated precondition) is clamped so
    // that no read leaves the stream
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

  const uint16_t* __restrict__ kb = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vb = static_cast<const uint16_t*>(a.v);
  unsigned char* sv = smem + wave * L::kTileBytes;

  float m[NHG], l[NHG];
  f32x4 o[NHG][D / 16];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    m[hg] = -INFINITY;
    l[hg] = 0.f;
#pragma unroll
    for (int cg = 0; cg < D / 16; ++cg) o[hg][cg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Software pipeline, two register sets: the loads of tile i+1 are in flight
  // while tile i is computed.  Past the last tile the prefetch still issues
  // the same loads, all of them at the current tile's first row (nvalid = 0:
  // every row re-reads row 0), so that the compiler can count them; a re-read
  // of the whole last tile instead, with the non-temporal hint, missed the
  // caches and fetched 16 KiB per wave again (16 x 128K: 158.6 MB counted
  // against 145.7 MB expected per launch).
  if (n_mine > 0) {
    auto step = [&](TileRegs<D>& rc, const TileInfo& ic, TileRegs<D>& rn, TileInfo& in,
                    int32_t next) {
      if (next < n_mine) {
        in = tile_info(next);
      } else {
        in.row0 = ic.row0;
        in.nvalid = 0;
      }
      issue_tile<D, NHG == 1>(kb, vb, a.k_row, a.v_row, in, rn, lane);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
      compute_tile<D, NHG>(rc, ic.nvalid, qf, m, l, o, sv, a.scale_log2, lane);
    };
    TileRegs<D> ra, rb;
    TileInfo ia = tile_info(0), ib;
    issue_tile<D, NHG == 1>(kb, vb, a.k_row, a.v_row, ia, ra, lane);
    for (int32_t i = 0;; i += 2) {
      step(ra, ia, rb, ib, i + 1);
      if (i + 1 >= n_mine) break;
      step(rb, ib, ra, ia, i + 2);
      if (i + 2 >= n_mine) break;
    }
  }

  // Every wave stores its state; then wave wl of a team combines the team's
  // WPG states for its own slice of the output columns, CPW 16-column blocks
  // of every head, and writes that slice: one barrier, and the partial's
  // stores spread over the waves (a tree merge into the first wave took two
  // rounds of two barriers, and that wave stored the whole partial)
  constexpr int CB = D / 16;
  constexpr int CPW = CB / WPG;
  static_assert(CPW * WPG == CB, "the column blocks split evenly over a team's waves");
  __syncthreads();  // every wave is done with its tile buffers
  store_state<D, NHG>(smem + wave * L::kStateBytes, m, l, o, lane);
  __syncthreads();
  float lt[NHG];
  f32x4 os[NHG][CPW];
  team_states<D, NHG, WPG, CPW>(smem + grp * WPG * L::kStateBytes, wl * CPW, m, lt, os, lane);

  const int64_t wg = blockIdx.x;
  if (a.fuse_merge && run.wgs == 1) {
    // the stream's only workgroup holds its whole softmax state: normalise
    // and write the output directly, no partial and no merge
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const int head = head0 + hg * 16;
      if (head >= H) continue;
      const float inv = lt[hg] > 0.f ? 1.f / lt[hg] : 0.f;
      const int64_t orow = static_cast<int64_t>(b) * H + head;
      if (wl == 0 && g == 0 && a.lse != nullptr)
        a.lse[orow] =
            lt[hg] > 0.f ? (m[hg] + log2f(lt[hg])) * 0.69314718055994530942f : -INFINITY;
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        *reinterpret_cast<f32x4*>(a.out + orow * D + (wl * CPW + c) * 16 + 4 * g) =
            os[hg][c] * inv;
    }
    return;
  }
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int head = head0 + hg * 16;
    if (head >= H) continue;
    float* om = a.ws_m + wg * H + head;
    float* ol = a.ws_l + wg * H + head;
    if (wl == 0 && g == 0) {
      if (a.fuse_merge) {  // the stream's last workgroup reads these at device scope
        store_coherent(om, m[hg]);
        store_coherent(ol, lt[hg]);
      } else {
        *om = m[hg];
        *ol = lt[hg];
      }
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int col = (wl * CPW + c) * 16 + 4 * g;
      // sc1 (written through) for the in-kernel merge, which reads them at
      // device scope, and for the two-group kernel's 16 KiB per workgroup
      if (a.fuse_merge || NHG > 1)
        store_through_16(a.ws_o + wg * H * D, static_cast<uint32_t>((head * D + col) * 4),
                         __builtin_bit_cast(st_u32x4, os[hg][c]));
      else
        *reinterpret_cast<f32x4*>(a.ws_o + (wg * H + head) * D + col) = os[hg][c];
    }
  }
  if (!a.fuse_merge) return;
  // the stream's last workgroup to finish merges its partials (no merge launch)
  __shared__ int32_t s_last;
  if (!arrive_last(a, b, run.wgs, &s_last)) return;
  merge_stream_block<NW * kWave>(a, b, wg - run.local, run.wgs);
  if (tid == 0)
    __hip_atomic_store(a.counters + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int KSEL>
hipError_t launch_mqa_dk(const AttnArgs& a, int64_t grid, hipStream_t st) {
  const int nhg = (a.H + 15) / 16;
  dim3 g(static_cast<uint32_t>(grid));
  if (nhg == 1)
    hipLaunchKernelGGL((attn_mqa_kernel<D, 1, 1, KSEL>), g, dim3(mqa_waves<1>() * kWave), 0, st,
                       a);
  else if (nhg == 2)
    hipLaunchKernelGGL((attn_mqa_kernel<D, 2, 1, KSEL>), g, dim3(mqa_waves<2>() * kWave), 0, st,
                       a);
  else if (nhg <= 4)
    hipLaunchKernelGGL((attn_mqa_kernel<D, 2, 2, KSEL>), g, dim3(mqa_waves<2>() * kWave), 0, st,
                       a);
  else return hipErrorNotSupported;
  return hipGetLastError();
}

template <int D>
hipError_t launch_mqa_d(const AttnArgs& a, int32_t max_chunks, hipStream_t st,
                        int64_t grid) {
  if (a.sel_scores == nullptr) return launch_mqa_dk<D, 0>(a, grid, st);
  if (max_chunks <= kMqaThreads * 8) return launch_mqa_dk<D, 8>(a, grid, st);
  if (max_chunks <= kMqaThreads * 16) return launch_mqa_dk<D, 16>(a, grid, st);
  return hipErrorNotSupported;
}

}  // namespace

bool mqa_select_in_kernel_supported(const lsa_shape& s) {
  return mqa_attn_supported(s) && s.max_chunks <= kMqaThreads * 16 && s.max_k <= kMaxRunSlots;
}

bool mqa_attn_supported(const lsa_shape& s) {
  return s.dtype == LSA_DTYPE_BF16 && !s.v_aliases_k && s.head_dim_qk == s.head_dim_v &&
         (s.head_dim_qk == 64 || s.head_dim_qk == 128) && s.num_q_heads >= 1 &&
         s.num_q_heads <= 64;
}

hipError_t launch_attn_mqa(const lsa_shape& s, const AttnArgs& a, int64_t grid, hipStream_t st) {
  if (a.sel_scores != nullptr && !mqa_select_in_kernel_supported(s)) return hipErrorNotSupported;
  if (s.head_dim_qk == 128) return launch_mqa_d<128>(a, s.max_chunks, st, grid);
  if (s.head_dim_qk == 64) return launch_mqa_d<64>(a, s.max_chunks, st, grid);
  return hipErrorNotSupported;
}

}  // namespace lsa
