// Radix-select building blocks shared by the top-B kernels of select2.hip.
//
// Order: 64-bit composites, the order-preserving 32-bit key of an fp32 score
// in the high half and the inverted position in the low half (higher score
// first, then lower position).  All composites of a row differ, so the B-th
// largest one splits the row exactly: selected <=> composite >= tau.
//
// tau is found by range refinement: the composites still in play lie in
// [lo, hi]; a pass histograms (c - lo) >> s into 1024 LDS bins (s is the
// smallest shift that fits the range into them), finds the bin holding the
// need-th largest and narrows [lo, hi] to that bin.  The first range is the
// row's own [min, max], so the bins follow the data instead of fixed key
// digits, and each pass shrinks the range by up to 1024x (10 bits).  Once the bin's
// population is small it is gathered into LDS and the passes continue there.
//
// With one or two waves per SIMD nothing hides latency, so every step here is
// built to keep dependent LDS round trips and barriers few: wave scans use
// DPP and lane reads instead of LDS shuffles, histogram copies are folded
// while picking the bin (vector LDS reads), gathers take one LDS atomic per
// wave, and the ordered emit needs a single barrier.
#pragma once

#include "device_common.hpp"

namespace fasa {

// Histogram of one refinement pass: 1024 bins (10 bits per pass).
constexpr int kSelBits = 10;
constexpr int kSelBins = 1 << kSelBits;

struct BinPick {
  uint32_t bin, above, count;
};

// Slabs of 4 elements per thread a register-resident select holds, at most.
constexpr int kMaxSlabs = 12;

// Scratch of a register-resident select with NT threads.
template <int NT, int COPIES, int CAP>
struct RegSelectLds {
  static constexpr int kWaves = NT / kWave;
  // Each copy has kWave spare words past the bins: lanes that count nothing
  // add 0 there (one word per lane) instead of hammering one bin address.
  uint32_t hist[COPIES][kSelBins + kWave];
  uint64_t cand[CAP];
  uint32_t wsum[kWaves];
  uint32_t slab_cnt[kMaxSlabs][kWaves];
  uint32_t rmin[kWaves], rmax[kWaves];
  uint64_t tau;
  uint32_t pick[4];
  uint32_t cand_n;
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_shr0(uint32_t v) {
  // Lanes with no source lane in their row read 0 (bound_ctrl).
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes: DPP shifts within each 16-lane
// row, then the earlier rows' totals read from lanes 15, 31 and 47.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += dpp_shr0<0x111>(v);  // row_shr:1
  v += dpp_shr0<0x112>(v);  // row_shr:2
  v += dpp_shr0<0x114>(v);  // row_shr:4
  v += dpp_shr0<0x118>(v);  // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const int row = lane_id() >> 4;
  return v + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

__device__ __forceinline__ uint64_t lanes_below() { return (1ull << lane_id()) - 1ull; }

// Zeroes the bins of `copies` histogram copies (vector LDS stores); ends with
// a barrier.
template <int NT, int COPIES, int CAP>
__device__ __forceinline__ void zero_hist(RegSelectLds<NT, COPIES, CAP>& L, int copies) {
  constexpr int kRow4 = (kSelBins + kWave) / 4;
  uint4* h = reinterpret_cast<uint4*>(&L.hist[0][0]);
  for (int i = threadIdx.x; i < copies * kRow4; i += NT)
    if (i % kRow4 < kSelBins / 4) h[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
}

// Sums `copies` histogram copies and finds, scanning from the top bin down,
// the bin where the running count reaches `need` (1 <= need <= total).
// Thread t owns the PER = kSelBins / NT bins of ranks PER t .. PER t + PER - 1
// (rank 0 = the top bin); a wave scan and the waves' totals in LDS give each
// thread its running count.  Two barriers, few registers.
template <int NT, int COPIES, int CAP>
__device__ __forceinline__ BinPick fold_and_pick(RegSelectLds<NT, COPIES, CAP>& L, int copies,
                                                 uint32_t need) {
  constexpr int PER = kSelBins / NT;
  static_assert(PER >= 1 && PER * NT == kSelBins, "bins per thread");
  const int t = threadIdx.x;
  const int lo = kSelBins - PER * (t + 1);  // lowest bin of this thread's ranks
  uint32_t c[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) c[r] = 0u;
  for (int k = 0; k < copies; ++k)
#pragma unroll
    for (int r = 0; r < PER; ++r) c[r] += L.hist[k][lo + PER - 1 - r];  // rank order
  uint32_t local = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) local += c[r];
  const uint32_t incl = wave_scan_incl(local);
  const int wave = t / kWave;
  if (lane_id() == kWave - 1) L.wsum[wave] = incl;
  if (t == 0) L.cand_n = 0;  // for the gather_cand that may follow
  __syncthreads();
  uint32_t before = incl - local;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) before += (w < wave) ? L.wsum[w] : 0u;
  if (before < need && need <= before + local) {
    uint32_t acc = before;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      if (acc < need && need <= acc + c[r]) {
        L.pick[0] = (uint32_t)(lo + PER - 1 - r);
        L.pick[1] = acc;
        L.pick[2] = c[r];
      }
      acc += c[r];
    }
  }
  __syncthreads();
  return BinPick{L.pick[0], L.pick[1], L.pick[2]};
}

// Block-wide min and max of lo / hi (in place).  One barrier.
template <int NT, int COPIES, int CAP>
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi,
                                             RegSelectLds<NT, COPIES, CAP>& L) {
  wave_minmax(lo, hi);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) {
    L.rmin[wave] = lo;
    L.rmax[wave] = hi;
  }
  __syncthreads();
  lo = L.rmin[0];
  hi = L.rmax[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) {
    lo = min(lo, L.rmin[w]);
    hi = max(hi, L.rmax[w]);
  }
}

// The fp32 score of an order-preserving key (inverse of score_key; -0 reads
// as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Shift that maps [lo, lo + span] onto at most kSelBins bins.
__device__ __forceinline__ int range_shift(uint64_t span) {
  return span < (uint64_t)kSelBins ? 0 : (64 - __clzll(span) - kSelBits);
}

// Gathers the thread's elements that satisfy `in(e)` into L.cand (one LDS
// atomic per wave reserves the wave's slots) and returns how many the block
// gathered (all of them fit: the caller knows the count is <= CAP).  L.cand_n
// must be 0 on entry (the fold_and_pick before it clears it).  One barrier.
template <int NT, int E, int COPIES, int CAP, class Src, class In>
__device__ __forceinline__ uint32_t gather_cand(const Src& src, In in,
                                                RegSelectLds<NT, COPIES, CAP>& L) {
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) mine += in(e) ? 1u : 0u;
  const uint32_t incl = wave_scan_incl(mine);
  uint32_t base = 0;
  if (lane_id() == kWave - 1 && incl) base = atomicAdd(&L.cand_n, incl);
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
  uint32_t slot = base + incl - mine;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (in(e)) {
      if (slot < (uint32_t)CAP) L.cand[slot] = ((uint64_t)src.key(e) << 32) | src.low(e);
      ++slot;
    }
  }
  __syncthreads();
  return min(L.cand_n, (uint32_t)CAP);
}

// Candidates at most this many are resolved by direct ranking.
constexpr uint32_t kRankMax = 128;

// The need-th largest of the M (<= kRankMax) distinct composites in L.cand:
// thread i counts the candidates above candidate i.  One barrier.
template <int NT, int COPIES, int CAP>
__device__ __forceinline__ uint64_t rank_resolve(uint32_t M, uint32_t need,
                                                 RegSelectLds<NT, COPIES, CAP>& L) {
  const uint32_t i = threadIdx.x;
  if (i < M) {
    const uint64_t c = L.cand[i];
    uint32_t above = 0;
    for (uint32_t j = 0; j < M; ++j) above += (L.cand[j] > c) ? 1u : 0u;
    if (above == need - 1) L.tau = c;
  }
  __syncthreads();
  return L.tau;
}

// The need-th largest of the composites in [lo, hi], held by the threads'
// elements (in_lds = false) or by L.cand[0..M) (in_lds = true): range
// refinement, see adaptive_select.
template <int NT, int E, int COPIES, int CAP, class Src>
__device__ __forceinline__ uint64_t refine(const Src& src, uint32_t need, uint64_t lo, uint64_t hi, bool in_lds,
                           uint32_t M, RegSelectLds<NT, COPIES, CAP>& L) {
  const int tid = threadIdx.x;
  const int copy = (tid / kWave) % COPIES;
  for (;;) {
    if (in_lds && M <= kRankMax) return rank_resolve(M, need, L);
    const int s = range_shift(hi - lo);
    const bool keyed = s >= 32;
    const uint32_t klo = (uint32_t)(lo >> 32), khi = (uint32_t)(hi >> 32);
    const int ks = keyed ? s - 32 : 0;
    if (!in_lds) {
      zero_hist(L, COPIES);
      const uint32_t spare = (uint32_t)(kSelBins + lane_id());
      if (keyed) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t k = src.key(e);
          const bool take = k >= klo && k <= khi;
          atomicAdd(&L.hist[copy][take ? (k - klo) >> ks : spare], take ? 1u : 0u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t c = ((uint64_t)src.key(e) << 32) | src.low(e);
          const bool take = src.key(e) != 0u && c >= lo && c <= hi;
          atomicAdd(&L.hist[copy][take ? (uint32_t)((c - lo) >> s) : spare], take ? 1u : 0u);
        }
      }
    } else {
      zero_hist(L, 1);
      for (uint32_t i = tid; i < M; i += NT) {
        const uint64_t c = L.cand[i];
        if (c >= lo && c <= hi) atomicAdd(&L.hist[0][(uint32_t)((c - lo) >> s)], 1u);
      }
    }
    __syncthreads();
    const BinPick p = fold_and_pick(L, in_lds ? 1 : COPIES, need);
    const uint64_t blo = lo + ((uint64_t)p.bin << s);
    need -= p.above;
    if (p.count == need) return blo;  // the whole bin is taken
    // A bin of one value (s == 0) holds one composite, so it ends above.
    const uint64_t bhi = blo + ((1ull << s) - 1ull);
    lo = blo;
    hi = bhi < hi ? bhi : hi;
    if (!in_lds && p.count <= (uint32_t)CAP) {
      const uint64_t glo = lo, ghi = hi;
      const bool gkeyed = (uint32_t)glo == 0u && (uint32_t)ghi == 0xffffffffu;
      M = gather_cand<NT, E>(src, [&](int e) {
        const uint32_t k = src.key(e);
        if (gkeyed) return k >= (uint32_t)(glo >> 32) && k <= (uint32_t)(ghi >> 32);
        const uint64_t c = ((uint64_t)k << 32) | src.low(e);
        return k != 0u && c >= glo && c <= ghi;
      }, L);
      in_lds = true;
    }
  }
}

// tau = the need-th largest composite of the row (1 <= need <= the number of
// valid elements); selected <=> composite >= tau, and tau >= 2^32.
//
// Src gives the thread's elements for compile-time e < E (so they stay in
// registers): key(e), the high half of the composite, 0 for an invalid
// element and >= 1 otherwise, and low(e), the low half.
//
// First pass, when every score is finite: 1024 bins linear in the score over
// [min, max] (fp32 arithmetic, monotone in the score, so a bin is a run of
// the order), which spreads typical score distributions over many bins; the
// bin holding the need-th largest is gathered into LDS and resolved there.
// Otherwise, or when that bin is too large, range refinement on keys: the
// range spans whole keys, [kmin << 32, (kmax << 32) | 0xffffffff], and bins
// of 2^s with s >= 32 keep it key-aligned, so while s >= 32 every test and bin
// needs the 32-bit key alone; only a range inside one key (ties) uses both
// halves.  Invalid elements (key 0) fall below every range.
template <int NT, int E, int COPIES, int CAP, class Src>
__device__ __forceinline__ uint64_t adaptive_select(const Src& src, uint32_t need,
                                    RegSelectLds<NT, COPIES, CAP>& L) {
  const int copy = (threadIdx.x / kWave) % COPIES;
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t k = src.key(e);
    kmin = min(kmin, k ? k : ~0u);
    kmax = max(kmax, k);
  }
  block_minmax(kmin, kmax, L);
  // Keys order the scores, so the extreme keys give the extreme scores, and
  // every score lies between them: all are finite when both ends are.
  const float vmin = key_value(kmin), vmax = key_value(kmax);
  const bool fin = isfinite(vmin) && isfinite(vmax);
  const float span = vmax - vmin;
  const float scale = (float)kSelBins / span;
  if (fin && span > 0.0f && isfinite(span) && isfinite(scale)) {
    auto bin_of = [&](uint32_t k) {
      return min(kSelBins - 1, (int)((key_value(k) - vmin) * scale));
    };
    zero_hist(L, COPIES);
    // Each element's bin, kept for the gather up to 32 elements per thread
    // (past that, registers are short and the gather computes it again, with
    // the same operations): invalid elements get the lane's spare word, which
    // is past every bin a pick can return.
    constexpr bool kKeepBins = E <= 32;
    const uint32_t spare = (uint32_t)(kSelBins + lane_id());
    uint32_t bins[kKeepBins ? E : 1];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = src.key(e);
      const uint32_t bn = k ? (uint32_t)bin_of(k) : spare;
      if constexpr (kKeepBins) bins[e] = bn;
      atomicAdd(&L.hist[copy][bn], k ? 1u : 0u);
    }
    __syncthreads();
    const BinPick p = fold_and_pick(L, COPIES, need);
    if (p.count <= (uint32_t)CAP) {
      const uint32_t M = gather_cand<NT, E>(src, [&](int e) {
        if constexpr (kKeepBins) return bins[e] == p.bin;
        const uint32_t k = src.key(e);
        return k != 0u && (uint32_t)bin_of(k) == p.bin;
      }, L);
      const uint32_t rest = need - p.above;
      if (M <= kRankMax) return rank_resolve(M, rest, L);
      // Range of the gathered composites, then refinement in LDS.
      uint32_t glo = ~0u, ghi = 0u;
      for (uint32_t i = threadIdx.x; i < M; i += NT) {
        const uint32_t k = (uint32_t)(L.cand[i] >> 32);
        glo = min(glo, k);
        ghi = max(ghi, k);
      }
      block_minmax(glo, ghi, L);
      return refine<NT, E>(src, rest, (uint64_t)glo << 32, ((uint64_t)ghi << 32) | 0xffffffffull,
                           true, M, L);
    }
  }
  return refine<NT, E>(src, need, (uint64_t)kmin << 32, ((uint64_t)kmax << 32) | 0xffffffffull,
                       false, 0u, L);
}

// Whether element e is selected by threshold tau (>= 2^32): 32-bit tests.
template <class Src>
__device__ __forceinline__ bool is_selected(const Src& src, int e, uint64_t tau) {
  const uint32_t tk = (uint32_t)(tau >> 32), tl = (uint32_t)tau;
  const uint32_t k = src.key(e);
  return k > tk || (k == tk && src.low(e) >= tl);
}

// Output offsets for an ordered compaction over S slabs: element e of slab s
// of thread t has order (s, t, e); sel[s] is the thread's 4-bit mask of
// selected elements in slab s.  off[s] receives the output index of the
// thread's first selected element of slab s; the return value is the total.
// One barrier.
//
// Within a wave, ballots and lane-masked bit counts give each thread its
// rank.  Across waves, the S * NW (slab, wave) counts lie in LDS slab-major;
// every wave reads them 64 at a time (lane s * NW + w of a group of 64 holds
// wave w's count for slab s), and one scan over each slab's NW lanes (DPP
// shifts, masked at the slab's edge) gives every wave its start in each
// slab, read out with lane reads.
//
// `tab` is LDS of S * NT / 64 words (the (slab, wave) counts, slab-major).
template <int NT, int S>
__device__ __forceinline__ uint32_t ordered_offsets_tab(const uint32_t (&sel)[S],
                                                        uint32_t (&off)[S], uint32_t* tab) {
  static_assert(S <= kMaxSlabs, "slab table size");
  constexpr int NW = NT / kWave;
  static_assert(NW == 8 || NW == 16, "a slab's counts fill part of one 16-lane row or all of it");
  constexpr int SPG = kWave / NW;           // slabs per group of 64 counts
  constexpr int NG = (S + SPG - 1) / SPG;   // groups
  const int wave = threadIdx.x / kWave, lane = lane_id();
  uint32_t pre[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint32_t p = 0, tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((sel[s] >> e) & 1u);
      p = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                    __builtin_amdgcn_mbcnt_lo((uint32_t)bal, p));
      tot += (uint32_t)__popcll(bal);
    }
    pre[s] = p;
    if (lane == 0) tab[s * NW + wave] = tot;
  }
  __syncthreads();
  const int lw = lane % NW;
  uint32_t incl[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int i = g * kWave + lane;
    uint32_t x = (i < S * NW) ? tab[i] : 0u;
    uint32_t t;
    t = dpp_shr0<0x111>(x);  // row_shr:1
    x += (lw >= 1) ? t : 0u;
    t = dpp_shr0<0x112>(x);  // row_shr:2
    x += (lw >= 2) ? t : 0u;
    t = dpp_shr0<0x114>(x);  // row_shr:4
    x += (lw >= 4) ? t : 0u;
    if constexpr (NW == 16) {
      t = dpp_shr0<0x118>(x);  // row_shr:8
      x += (lw >= 8) ? t : 0u;
    }
    incl[g] = x;
  }
  const int w = __builtin_amdgcn_readfirstlane(wave);
  uint32_t base = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int g = s / SPG, l0 = (s % SPG) * NW;
    const uint32_t before =
        w > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)incl[g], l0 + w - 1) : 0u;
    off[s] = base + before + pre[s];
    base += (uint32_t)__builtin_amdgcn_readlane((int)incl[g], l0 + NW - 1);
  }
  return base;
}

// ordered_offsets_tab with the scratch's slab table.
template <int NT, int S, int COPIES, int CAP>
__device__ __forceinline__ uint32_t ordered_offsets(const uint32_t (&sel)[S], uint32_t (&off)[S],
                                                    RegSelectLds<NT, COPIES, CAP>& L) {
  return ordered_offsets_tab<NT, S>(sel, off, &L.slab_cnt[0][0]);
}

}  // namespace fasa
