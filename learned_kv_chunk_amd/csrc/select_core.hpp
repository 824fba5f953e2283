// select_core.hpp -- top-k of one stream's fp32 scores by one workgroup (or
// one wave).
//
// Dimensionstp review, section 3-2-3 step 5: keep the top-k chunks.  Ties go
// to the lower chunk index, NaN ranks below every number and -0.0 equals
// +0.0; kept indices come out in ascending order.
//
// THREADS threads (64: a single wave, no barriers) hold KPT consecutive
// scores each ([t*KPT, t*KPT+KPT)) as order-preserving 32-bit keys.  An
// MSB-first radix select runs up to four 8-bit digit passes, each into its
// own LDS histogram, and stops early once every key of the chosen digit is
// kept (with continuous scores, usually after three).  In the first pass (sign and top exponent bits: few distinct
// digits) the lanes holding the first participating lane's digit (usually the
// wave's most common one) add their count once, so few lanes of a wave hit the
// same LDS word; later passes only see keys that share the digits chosen so
// far and add directly.  After a pass every wave reads the 256 counts (four per
// lane), scans them with DPP row shifts and lane reads, and finds the digit
// holding the k-th largest key without another barrier.  A block-wide
// exclusive scan of (#keys > T, #keys == T) then places every kept chunk at
// its output position: ascending indices and the lower-index tie rule with no
// sort.
//
// With eight or more keys per thread a bucket pass is tried first: the stream's finite
// scores are spread over 1024 equal-width bins between their minimum and
// maximum (a monotone map, so the bins are ordered like the keys), one
// histogram finds the bin holding the k-th largest key, and when that bin has
// at most 64 keys one wave ranks them exactly by (key desc, index asc).  For
// scores from a continuous distribution the boundary bin holds a few keys, so
// one histogram replaces four; otherwise (ties, infinities, a very skewed
// spread) the radix passes run.
#pragma once

#include "lsa_internal.hpp"
#include "wave.hpp"

namespace lsa {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;       // NaN: below every number
  if ((u << 1) == 0u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelectBins = 1024;     // bucket pass bins (the four radix histograms' words)
constexpr int kSelectMaxCand = 64;    // keys the bucket pass ranks in one wave

template <int THREADS>
struct SelectLds {
  alignas(16) uint32_t hist[4][256];
  uint32_t tot[2 * (THREADS / kWave)];
  uint32_t cand_key[kSelectMaxCand];
  int32_t cand_idx[kSelectMaxCand];
  uint32_t misc[4];  // candidate count; threshold key and its kept count
};

// Value of a non-zero order key (the inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Barrier among the THREADS threads taking part (a single wave needs only
// its LDS operations ordered).
template <int THREADS>
__device__ __forceinline__ void select_sync() {
  if (THREADS == kWave) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  } else {
    __syncthreads();
  }
}

// Exclusive scan of two counters over the THREADS threads.
template <int THREADS>
__device__ __forceinline__ void select_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* ea,
                                                       uint32_t* eb, uint32_t* s_tot) {
  const int wave = threadIdx.x / kWave;
  const uint32_t ia = wave_inclusive_scan(a);
  const uint32_t ib = wave_inclusive_scan(b);
  uint32_t ba = 0, bb = 0;
  if (THREADS > kWave) {
    if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
      s_tot[2 * wave] = ia;
      s_tot[2 * wave + 1] = ib;
    }
    select_sync<THREADS>();
#pragma unroll
    for (int w = 0; w < THREADS / kWave; ++w) {
      if (w < wave) {
        ba += s_tot[2 * w];
        bb += s_tot[2 * w + 1];
      }
    }
  }
  *ea = ba + ia - a;
  *eb = bb + ib - b;
}

// Loads scores[0..n) as order keys, KPT consecutive ones per thread (keys
// past n are 0 and never counted).  With KPT a multiple of four every load is
// a 16-byte load of an aligned block, whatever the alignment of the stream's
// first score: a thread reads the KPT / 4 blocks that cover its scores, one
// more when the stream starts r floats into a block, and picks its scores
// from offset r (r is the same for the whole workgroup, so the pick is a
// uniform branch).  A block holding none of the stream's scores is not read,
// so no access leaves the aligned blocks of the stream's own scores.  (One
// 4-byte load per score instead -- the form for a misaligned stream before --
// took twice as long for 4096 scores: each instruction touched 64 lines.)
// `meanwhile` runs once the loads are issued, before their data is used.
struct NoWork {
  __device__ void operator()() const {}
};
template <int THREADS, int KPT, typename F = NoWork>
__device__ __forceinline__ void select_load_keys(const float* __restrict__ scores, int32_t n,
                                                 uint32_t (&key)[KPT], F meanwhile = F()) {
  const int tid = threadIdx.x;
  float sv[KPT];
  if constexpr (KPT % 4 == 0) {
    constexpr int NB = KPT / 4 + 1;
    const int r = static_cast<int>((reinterpret_cast<uintptr_t>(scores) >> 2) & 3u);
    const float4* blk = reinterpret_cast<const float4*>(scores - r) + tid * (KPT / 4);
    float v[4 * NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      // the block's first float is score tid * KPT + 4q - r: read it only if
      // the block holds a score of the stream
      const bool need = (q < KPT / 4 || r != 0) && tid * KPT + 4 * q - r < n;
      const float4 f = need ? blk[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[4 * q] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
    meanwhile();
    switch (r) {
#define LSA_PICK(R)                                     \
  case R:                                               \
    _Pragma("unroll") for (int i = 0; i < KPT; ++i) sv[i] = v[(R) + i]; \
    break;
      LSA_PICK(0)
      LSA_PICK(1)
      LSA_PICK(2)
      LSA_PICK(3)
#undef LSA_PICK
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) sv[i] = scores[min(tid * KPT + i, n - 1)];
    meanwhile();
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = (tid * KPT + i < n) ? order_key(sv[i]) : 0u;
}

// Zeroes the radix histograms (every one of the THREADS threads; a barrier
// must follow before the passes).
template <int THREADS>
__device__ __forceinline__ void select_clear_hist(SelectLds<THREADS>& lds) {
  for (int i = threadIdx.x; i < 4 * 256; i += THREADS) (&lds.hist[0][0])[i] = 0u;
}

// Radix passes: the key T of the k-th largest key (`prefix`) and how many
// keys equal to T are kept (`remaining`), T compared on the bits of `mask`.
// The passes stop as soon as every key of the chosen digit is kept: then the
// digits resolved so far already separate the kept keys (T is a prefix, and
// all keys sharing it are kept).  cleared: the histograms are already zero
// (select_clear_hist and a barrier).
template <int THREADS, int KPT>
__device__ __forceinline__ void select_radix(const uint32_t (&key)[KPT], int32_t n, int32_t k,
                                             SelectLds<THREADS>& lds, uint32_t* prefix_out,
                                             uint32_t* remaining_out, uint32_t* mask_out,
                                             bool cleared = false) {
  const int tid = threadIdx.x;
  if (!cleared) {
    select_clear_hist<THREADS>(lds);
    select_sync<THREADS>();
  }

  const uint64_t below = lanemask_lt();
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(k);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* hist = lds.hist[pass];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool part = (tid * KPT + i < n) && ((key[i] & mask) == prefix);
      const uint32_t d = (key[i] >> shift) & 0xffu;
      const uint64_t pm = __ballot(part);
      if (pm == 0) continue;
      if (pass == 0) {
        // the leading digit is shared by most lanes: the lanes holding the
        // first participating lane's digit add as one (the lowest of them
        // adds their count), the others directly -- one predicated atomic
        const uint32_t lead = __builtin_amdgcn_readlane(d, __ffsll(static_cast<long long>(pm)) - 1);
        const bool is_lead = part && d == lead;
        const uint64_t same = __ballot(is_lead);
        const uint32_t add = is_lead ? ((same & below) == 0 ? static_cast<uint32_t>(__popcll(same)) : 0u)
                                     : (part ? 1u : 0u);
        if (add != 0u) atomicAdd(&hist[d], add);
      } else {
        // few keys still take part: the others add zero, which keeps the
        // atomic unconditional (no exec-mask branches around it)
        atomicAdd(&hist[d], part ? 1u : 0u);
      }
    }
    select_sync<THREADS>();
    // digit d* with #(digit > d*) < remaining <= #(digit >= d*); lane l owns
    // digits 4l..4l+3 (higher lanes hold higher digits)
    const uint32_t lane = tid & (kWave - 1);
    const uint4 c = reinterpret_cast<const uint4*>(hist)[lane];
    const uint32_t tot = c.x + c.y + c.z + c.w;
    const uint32_t incl = wave_inclusive_scan(tot);
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    uint32_t ge = total - incl;  // keys whose digit is above this lane's four
    const uint32_t cnt[4] = {c.x, c.y, c.z, c.w};
    // the ranges (gt, gt + cnt] of the digits are disjoint and cover
    // (0, total], so exactly one digit holds `remaining`: selects, no branches
    uint32_t pick = 0, gt_pick = 0, n_pick = 0;
    bool found = false;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      const uint32_t gt = ge;
      ge += cnt[j];
      const bool here = gt < remaining && remaining <= ge;
      pick = here ? 4u * lane + j : pick;
      gt_pick = here ? gt : gt_pick;
      n_pick = here ? cnt[j] : n_pick;
      found = found || here;
    }
    const uint64_t hit = __ballot(found);
    const int src = __ffsll(static_cast<long long>(hit)) - 1;
    pick = __builtin_amdgcn_readlane(pick, src);
    gt_pick = __builtin_amdgcn_readlane(gt_pick, src);
    n_pick = __builtin_amdgcn_readlane(n_pick, src);
    prefix |= pick << shift;
    mask |= 0xffu << shift;
    remaining -= gt_pick;
    if (n_pick == remaining) break;  // workgroup-uniform: every wave scanned the same counts
  }

  *prefix_out = prefix;
  *remaining_out = remaining;
  *mask_out = mask;
}

// Bucket pass (see the file comment): returns false, with the workgroup in
// step and the histograms free, when the radix passes must decide instead.
template <int THREADS, int KPT>
__device__ __forceinline__ bool select_buckets(const uint32_t (&key)[KPT], int32_t n, int32_t k,
                                               SelectLds<THREADS>& lds, uint32_t* prefix_out,
                                               uint32_t* remaining_out) {
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const uint32_t lane = tid & (kWave - 1);
  uint32_t* hist = &lds.hist[0][0];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (tid * KPT + i < n && key[i] != 0u) {  // NaN (key 0) takes no part in the range
      lo = min(lo, key[i]);
      hi = max(hi, key[i]);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  for (int i = tid; i < kSelectBins; i += THREADS) hist[i] = 0u;
  if (tid == 0) lds.misc[0] = 0u;
  if (THREADS > kWave) {
    if (lane == 0) {
      lds.tot[2 * wave] = lo;
      lds.tot[2 * wave + 1] = hi;
    }
    select_sync<THREADS>();
#pragma unroll
    for (int w = 0; w < THREADS / kWave; ++w) {
      lo = min(lo, lds.tot[2 * w]);
      hi = max(hi, lds.tot[2 * w + 1]);
    }
  } else {
    select_sync<THREADS>();
  }
  if (hi <= lo) return false;  // one distinct number (or none)
  const float fl = key_value(lo), fh = key_value(hi);
  const float range = fh - fl;
  const float scale = static_cast<float>(kSelectBins) / range;
  if (!(range > 0.f) || !__builtin_isfinite(range) || !__builtin_isfinite(scale)) return false;
  // bin of a key: monotone in the key; NaN joins the lowest bin
  auto bin_of = [&](uint32_t kv) -> int {
    return kv == 0u ? 0
                    : min(kSelectBins - 1, static_cast<int>((key_value(kv) - fl) * scale));
  };
  int bin[KPT];  // kept for the candidate pass
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    bin[i] = bin_of(key[i]);
    if (tid * KPT + i < n) atomicAdd(&hist[bin[i]], 1u);
  }
  select_sync<THREADS>();
  // bin d* with #(bin > d*) < k <= #(bin >= d*); lane l owns bins 16l..16l+15
  uint32_t cnt[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 c4 = reinterpret_cast<const uint4*>(hist)[4 * lane + q];
    cnt[4 * q] = c4.x;
    cnt[4 * q + 1] = c4.y;
    cnt[4 * q + 2] = c4.z;
    cnt[4 * q + 3] = c4.w;
  }
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) tot += cnt[j];
  const uint32_t incl = wave_inclusive_scan(tot);
  const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
  uint32_t ge = total - incl;
  uint32_t pick = 0, gt_pick = 0;
  bool found = false;
#pragma unroll
  for (int j = 15; j >= 0; --j) {  // exactly one bin holds the k-th key (as in the radix pass)
    const uint32_t gt = ge;
    ge += cnt[j];
    const bool here = gt < static_cast<uint32_t>(k) && static_cast<uint32_t>(k) <= ge;
    pick = here ? 16u * lane + j : pick;
    gt_pick = here ? gt : gt_pick;
    found = found || here;
  }
  const uint64_t hit = __ballot(found);
  const int src = __ffsll(static_cast<long long>(hit)) - 1;
  pick = __builtin_amdgcn_readlane(pick, src);
  gt_pick = __builtin_amdgcn_readlane(gt_pick, src);
  const uint32_t in_bin = hist[pick];
  if (in_bin > static_cast<uint32_t>(kSelectMaxCand)) {
    select_sync<THREADS>();  // every wave has read the histogram
    return false;
  }
  const uint32_t remaining = static_cast<uint32_t>(k) - gt_pick;  // kept from bin d*
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (tid * KPT + i < n && bin[i] == static_cast<int>(pick)) {
      const uint32_t slot = atomicAdd(&lds.misc[0], 1u);
      lds.cand_key[slot] = key[i];
      lds.cand_idx[slot] = tid * KPT + i;
    }
  }
  select_sync<THREADS>();
  if (wave == 0) {
    // rank of each candidate by (key desc, index asc) among the in_bin ones
    const bool mine = lane < in_bin;
    const uint32_t kk = mine ? lds.cand_key[lane] : 0u;
    const int32_t ii = mine ? lds.cand_idx[lane] : 0x7fffffff;
    uint32_t rank = 0;
    for (uint32_t j = 0; j < in_bin; ++j) {
      const uint32_t kj = __builtin_amdgcn_readlane(kk, j);
      const int32_t ij = __builtin_amdgcn_readlane(ii, j);
      rank += (kj > kk || (kj == kk && ij < ii)) ? 1u : 0u;
    }
    const uint64_t at = __ballot(mine && rank == remaining - 1);
    const uint32_t t_key = __builtin_amdgcn_readlane(kk, __ffsll(static_cast<long long>(at)) - 1);
    const uint32_t above = static_cast<uint32_t>(__popcll(__ballot(mine && kk > t_key)));
    if (lane == 0) {
      lds.misc[1] = t_key;
      lds.misc[2] = remaining - above;
    }
  }
  select_sync<THREADS>();
  *prefix_out = lds.misc[1];
  *remaining_out = lds.misc[2];
  return true;
}

// Top-k of the n keys held as select_load_keys leaves them, written ascending
// to out[0..k); 0 < k < n.  Every one of the THREADS threads (threads
// 0..THREADS-1 of the workgroup) must call it.
template <int THREADS, int KPT, bool BUCKETS = (KPT >= 8)>
__device__ __forceinline__ void select_topk_keys(const uint32_t (&key)[KPT], int32_t n,
                                                 int32_t k, int32_t* __restrict__ out,
                                                 SelectLds<THREADS>& lds, bool cleared = false) {
  const int tid = threadIdx.x;
  uint32_t prefix, remaining, mask = 0xffffffffu;
  // the bucket pass pays off from eight keys per thread (streams of several
  // thousand chunks); below that the radix passes are as fast.  cleared: the
  // radix histograms are zero already (not after a bucket pass, which uses
  // their words)
  if (!BUCKETS || !select_buckets<THREADS, KPT>(key, n, k, lds, &prefix, &remaining))
    select_radix<THREADS, KPT>(key, n, k, lds, &prefix, &remaining, &mask, cleared && !BUCKETS);

  // keys above T (on the bits of mask) are kept, and the first `remaining`
  // keys equal to T in index order
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool v = tid * KPT + i < n;
    n_gt += (v && (key[i] & mask) > prefix) ? 1u : 0u;
    n_eq += (v && (key[i] & mask) == prefix) ? 1u : 0u;
  }
  uint32_t gt_before, eq_before;
  select_exclusive_scan2<THREADS>(n_gt, n_eq, &gt_before, &eq_before, lds.tot);
  // a kept key's slot is the number of kept keys before it; one predicated
  // store per key and no nested branches (a thread's keys are processed in
  // order, so the counts before each follow by increments)
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int32_t idx = tid * KPT + i;
    const uint32_t km = key[i] & mask;
    const bool gt = idx < n && km > prefix;
    const bool eq = idx < n && km == prefix;
    const uint32_t pos = gt_before + min(eq_before, remaining);
    if (gt || (eq && eq_before < remaining)) out[pos] = idx;
    gt_before += gt ? 1u : 0u;
    eq_before += eq ? 1u : 0u;
  }
}

// Top-k of scores[0..n) written ascending to out[0..k); 0 < k < n.
template <int THREADS, int KPT, bool BUCKETS = (KPT >= 8)>
__device__ __forceinline__ void select_topk_block(const float* __restrict__ scores, int32_t n,
                                                  int32_t k, int32_t* __restrict__ out,
                                                  SelectLds<THREADS>& lds) {
  uint32_t key[KPT];
  if constexpr (BUCKETS) {
    select_load_keys<THREADS, KPT>(scores, n, key);
    select_topk_keys<THREADS, KPT, BUCKETS>(key, n, k, out, lds);
  } else {
    // the histograms are cleared while the scores are in flight
    select_load_keys<THREADS, KPT>(scores, n, key, [&]() {
      select_clear_hist<THREADS>(lds);
      select_sync<THREADS>();
    });
    select_topk_keys<THREADS, KPT, BUCKETS>(key, n, k, out, lds, true);
  }
}

// The kept set of an attention workgroup's stream, ranked in its prologue by
// all THREADS threads (the same keys, rule and algorithm as lsa_select_topk,
// so the same set): kept[0 .. k_b) (LDS) receives the stream's kept chunk
// indices in ascending order, and the stream's first workgroup also writes
// them to sel_idx_out.  Requires N_b <= THREADS * KPT and k_b <= kMaxRunSlots
// (checked on the host); ends with a barrier.  lds may alias LDS that the
// caller uses only afterwards.
template <int THREADS, int KPT>
__device__ __forceinline__ void attn_select_stream(const AttnArgs& a, const AttnRun& run,
                                                   int32_t* kept, SelectLds<THREADS>& lds) {
  const int32_t n = run.cn < 0 ? 0 : (run.cn > THREADS * KPT ? THREADS * KPT : run.cn);
  int32_t k = run.kb < 0 ? 0 : (run.kb > kMaxRunSlots ? kMaxRunSlots : run.kb);
  if (k > n) k = n;
  if (k > 0 && k < n) {
    // the radix passes: the bucket pass is slower for streams of up to
    // 2048 chunks (eight keys per thread here)
    select_topk_block<THREADS, KPT, (KPT > 8)>(a.sel_scores + run.cbase, n, k, kept, lds);
  } else {
    for (int32_t i = threadIdx.x; i < k; i += THREADS) kept[i] = i;
  }
  __syncthreads();
  if (run.local == 0)
    for (int32_t i = threadIdx.x; i < k; i += THREADS) a.sel_idx_out[run.sel0 + i] = kept[i];
}

}  // namespace lsa
