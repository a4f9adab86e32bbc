// Filtered top-B selection of a decode step, fused with FAC.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC bullets: the critical token set T_t is chosen from the TIP
// scores (the min(B, n) highest of each (sequence, query head) row, equal
// scores to the lower position, listed ascending), then full attention runs
// over T_t only.  Selection is exact, over the 64-bit composites of
// select_common.hpp: selected <=> composite >= tau, tau the B-th largest.
//
// In a filtered decode step the TIP launch has also written the largest
// score key of every 8-token group of each row.  Group maxima are scores of
// distinct tokens, so the B-th largest of them is at most tau, and every
// token >= tau lies in a group whose maximum is >= it.  Here:
//   1. one histogram pass over the row's group maxima (bins linear in the
//      score between their min and max) finds the bin P holding the B-th
//      largest; every group whose maximum falls in bin P or above survives
//      (about B groups);
//   2. the survivors' scores (8 each, 32 contiguous bytes) are gathered, those
//      below bin P dropped, and tau is the B-th largest of the rest, exactly;
//      T_t is emitted in position order (groups ascending, then positions);
//   3. rows where that would not fit (ties spread over too many groups, or a
//      degenerate score range) are selected by streaming range refinement
//      over their scores and an ordered streaming emit.
// Rows of at most B groups skip step 1 (every group survives).
//
// One 512-thread workgroup per row, or S per row for the fused FAC's column
// split (each part makes the same selection); part 0 writes idx, the advanced
// length and flags.  No workgroup waits on another.

#include "attention_common.hpp"
#include "budget.hpp"
#include "fasa_internal.hpp"
#include "select_common.hpp"
#include "select_src.hpp"

namespace fasa {

constexpr int kFilterThreads = kFilterSelectThreads;
constexpr int kFilterWaves = kFilterThreads / kWave;
constexpr int kFilterHistCopies = 4;
constexpr int kFilterCandCap = 4096;
// Most surviving groups: 24 survivor slots per thread, 8 per group.
constexpr int kFilterMaxSurvivors = kFilterThreads * 24 / kGroupTokens;
static_assert(kGroupTokens == 8 && kFilterThreads % 2 == 0, "two threads per group");
// LDS the fused FAC needs for its state merge, worst case over the head
// sizes and dtypes built (bf16, d = 64: 128 states of 64 dims).
constexpr int kFilterAttendScratch = 9728;

using FilterSelLds = RegSelectLds<kFilterThreads, kFilterHistCopies, kFilterCandCap>;

struct FilterLds {
  union {
    FilterSelLds s;  // streaming passes, LDS refinement, pivot-bin gather, ordered emits
    float att[kFilterAttendScratch];
  };
  // Histograms of the group maxima and of the survivors, cleared at the
  // kernel's start (a spare word per lane past the bins, as in RegSelectLds).
  alignas(16) uint32_t hist1[kSelBins + kWave];
  alignas(16) uint32_t hist2[kSelBins + kWave];
  int32_t sel[kFusedMaxBudget];
  int32_t grp[kFilterMaxSurvivors];  // surviving groups, ascending
  uint32_t kpmin[kFilterWaves];      // per-wave smallest surviving group maximum
};

struct WavePick {
  uint32_t bin, above, count;
  bool ok;  // false when the histogram holds fewer than `need`
};

// The bin where the running count from the top bin down reaches `need`,
// found by each wave on its own (no barrier): lane l sums the 16 bins of
// ranks 16 l .. 16 l + 15 from the top, a wave scan gives each lane its
// running count, and the lane holding the target walks its 16 bins.
__device__ __forceinline__ WavePick wave_pick(const uint32_t* hist, uint32_t need) {
  const int l = lane_id();
  const uint4* h4 = reinterpret_cast<const uint4*>(hist + (kSelBins - 16 * (l + 1)));
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 x = h4[i];
    // word w of the 16 holds bin kSelBins - 16 (l + 1) + w, rank 15 - w
    c[15 - 4 * i] = x.x;
    c[14 - 4 * i] = x.y;
    c[13 - 4 * i] = x.z;
    c[12 - 4 * i] = x.w;
  }
  uint32_t local = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) local += c[r];
  const uint32_t incl = wave_scan_incl(local);
  const uint32_t before = incl - local;
  const uint64_t bal = __ballot(before < need && need <= incl);
  WavePick p{0u, 0u, 0u, bal != 0ull};
  if (!p.ok) return p;
  uint32_t bin = 0, above = 0, count = 0, acc = before;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (acc < need && need <= acc + c[r]) {
      bin = (uint32_t)(kSelBins - 1 - 16 * l - r);
      above = acc;
      count = c[r];
    }
    acc += c[r];
  }
  const int src = (int)__builtin_ctzll(bal);
  p.bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
  p.above = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
  p.count = (uint32_t)__builtin_amdgcn_readlane((int)count, src);
  return p;
}

// The need-th largest of the M (<= kWave) composites in cand[0 .. M), found
// by each wave on its own: lane i counts the candidates above candidate i.
__device__ __forceinline__ uint64_t wave_rank(const uint64_t* cand, uint32_t M, uint32_t need) {
  const uint32_t i = (uint32_t)lane_id();
  const uint64_t c = i < M ? cand[i] : 0ull;
  uint32_t above = 0;
  for (uint32_t j = 0; j < M; ++j) above += (cand[j] > c) ? 1u : 0u;
  const uint64_t bal = __ballot(i < M && above == need - 1);
  const int src = (int)__builtin_ctzll(bal);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// The surviving groups' scores held for the exact select: slot e of thread t
// is virtual element 4 (s NT + t) + e % 4 (s = e / 4), i.e. list entry
// (s NT + t) / 2 and offset 4 (t % 2) + e % 4 in its group, so (slab, thread,
// e) order is position order.  Key 0 marks no element.
template <int E>
struct SurvivorSrc {
  uint32_t k[E];
  int g[E / 4];  // group of slab s (any value where the slab holds none)
  __device__ __forceinline__ int pos(int e) const {
    return g[e / 4] * kGroupTokens + 4 * (int)(threadIdx.x & 1) + (e & 3);
  }
  __device__ __forceinline__ uint32_t key(int e) const { return k[e]; }
  __device__ __forceinline__ uint32_t low(int e) const { return 0xffffffffu - (uint32_t)pos(e); }
};

// Streaming passes over a row's n scores (8192 per round: 4 float4 slabs per
// thread, slab layout), for rows whose saturated tiles do not fit registers.
constexpr int kStreamSlabs = 4;
constexpr int kStreamChunk = kFilterThreads * 4 * kStreamSlabs;

struct StreamChunk {
  uint32_t k[4 * kStreamSlabs];  // keys, 0 past n
  int first;                     // position of element 0 of this thread
  __device__ __forceinline__ int pos(int e) const {
    return first + (e / 4) * 4 * kFilterThreads + (e & 3);
  }
};

__device__ __forceinline__ void stream_load(StreamChunk& c, __amdgpu_buffer_rsrc_t rs, int base,
                                            int n) {
  const int t = threadIdx.x;
  c.first = base + 4 * t;
#pragma unroll
  for (int g = 0; g < kStreamSlabs; ++g) {
    const int p0 = base + 4 * (g * kFilterThreads + t);
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)p0 * 4u, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = score_key(__uint_as_float(x[e]));
      c.k[4 * g + e] = (p0 + e < n) ? (k ? k : 1u) : 0u;
    }
  }
}

// tau over the row's scores: the need-th largest composite in [lo, hi]
// (which holds at least need of them, and every composite above hi is out):
// 1024-bin range refinement, each pass a streaming histogram of the row;
// once the pivot bin holds at most kFilterCandCap elements they are gathered
// into LDS and the refinement ends there.
// A register source with no elements: the LDS-only refinement below never
// reads one.
struct NoSrc {
  __device__ __forceinline__ uint32_t key(int) const { return 0u; }
  __device__ __forceinline__ uint32_t low(int) const { return 0u; }
};

__device__ __forceinline__ uint64_t stream_select(const float* row, int n, uint32_t need,
                                                  uint64_t lo, uint64_t hi, FilterSelLds& L,
                                                  uint32_t* err) {
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row, ((n + 3) & ~3) * 4);
  const int copy = (threadIdx.x / kWave) % kFilterHistCopies;
  const uint32_t spare = (uint32_t)(kSelBins + lane_id());
  // Each pass narrows the 64-bit range by 10 bits or ends it, so 7 passes
  // always suffice when [lo, hi] holds `need` composites; the cap only
  // guards the loop should that ever not hold.
  for (int pass = 0;; ++pass) {
    if (pass == 8) {
      if (threadIdx.x == 0) raise_flag(err, FASA_DEVFLAG_SELECT);
      return lo;
    }
    const int s = range_shift(hi - lo);
    zero_hist(L, kFilterHistCopies);
    for (int base = 0; base < n; base += kStreamChunk) {
      StreamChunk c;
      stream_load(c, rs, base, n);
#pragma unroll
      for (int e = 0; e < 4 * kStreamSlabs; ++e) {
        const uint64_t cc = composite(c.k[e], (uint32_t)c.pos(e));
        const bool take = c.k[e] != 0u && cc >= lo && cc <= hi;
        atomicAdd(&L.hist[copy][take ? (uint32_t)((cc - lo) >> s) : spare], take ? 1u : 0u);
      }
    }
    __syncthreads();
    const BinPick p = fold_and_pick(L, kFilterHistCopies, need);
    const uint64_t blo = lo + ((uint64_t)p.bin << s);
    need -= p.above;
    if (p.count == need) return blo;  // the whole bin is taken
    const uint64_t bhi = blo + ((1ull << s) - 1ull);
    lo = blo;
    hi = bhi < hi ? bhi : hi;
    if (p.count <= (uint32_t)kFilterCandCap) {
      // Gather the bin (L.cand_n was cleared by fold_and_pick).
      for (int base = 0; base < n; base += kStreamChunk) {
        StreamChunk c;
        stream_load(c, rs, base, n);
        uint32_t mine = 0;
#pragma unroll
        for (int e = 0; e < 4 * kStreamSlabs; ++e) {
          const uint64_t cc = composite(c.k[e], (uint32_t)c.pos(e));
          mine += (c.k[e] != 0u && cc >= lo && cc <= hi) ? 1u : 0u;
        }
        const uint32_t incl = wave_scan_incl(mine);
        uint32_t at = 0;
        if (lane_id() == kWave - 1 && incl) at = atomicAdd(&L.cand_n, incl);
        at = (uint32_t)__builtin_amdgcn_readlane((int)at, kWave - 1);
        uint32_t slot = at + incl - mine;
#pragma unroll
        for (int e = 0; e < 4 * kStreamSlabs; ++e) {
          const uint64_t cc = composite(c.k[e], (uint32_t)c.pos(e));
          if (c.k[e] != 0u && cc >= lo && cc <= hi) {
            if (slot < (uint32_t)kFilterCandCap) L.cand[slot] = cc;
            ++slot;
          }
        }
      }
      __syncthreads();
      const uint32_t M = L.cand_n < (uint32_t)kFilterCandCap ? L.cand_n : (uint32_t)kFilterCandCap;
      return refine<kFilterThreads, 4>(NoSrc{}, need, lo, hi, true, M, L);
    }
  }
}

// Calls f(rank, position) for the row's composites >= tau in ascending
// position order, the first `limit` of them: one streaming pass, each round
// an ordered compaction.
template <class F>
__device__ __forceinline__ void stream_emit(const float* row, int n, uint64_t tau, uint32_t limit, FilterSelLds& L,
                            F f) {
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row, ((n + 3) & ~3) * 4);
  uint32_t done = 0;
  for (int base = 0; base < n && done < limit; base += kStreamChunk) {
    StreamChunk c;
    stream_load(c, rs, base, n);
    uint32_t m4[kStreamSlabs], off[kStreamSlabs];
#pragma unroll
    for (int g = 0; g < kStreamSlabs; ++g) {
      m4[g] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = c.k[4 * g + e];
        const bool in = k != 0u && composite(k, (uint32_t)c.pos(4 * g + e)) >= tau;
        m4[g] |= (in ? 1u : 0u) << e;
      }
    }
    const uint32_t tot = ordered_offsets<kFilterThreads>(m4, off, L);
#pragma unroll
    for (int g = 0; g < kStreamSlabs; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((m4[g] >> e) & 1u) {
          const uint32_t r = done + off[g];
          if (r < limit) f(r, c.pos(4 * g + e));
          ++off[g];
        }
    done += tot;
    __syncthreads();  // the slab counts are rewritten next round
  }
}

// T_t of row (b, h) from the group maxima (see the file comment), written to
// idx (part 0, if given) and attended (fused FAC) by every part for its
// columns.  E1 group maxima per thread (E1 NT >= the row's groups), E2
// survivor slots per thread (E2 NT / 8 groups).
template <bool BF16, int D, int E1, int E2, int S>
__global__ void __launch_bounds__(kFilterThreads)
filter_select_kernel(const uint32_t* __restrict__ gmax, int gstride,
                     const float* __restrict__ scores, const int32_t* __restrict__ nb,
                     int max_seq_len, int hq, int cap, int budget,
                     const int32_t* __restrict__ head_budget, int32_t* __restrict__ idx,
                     const void* __restrict__ k_cache, const void* __restrict__ v_cache,
                     const float* __restrict__ qrot, int hkv, int G, float* __restrict__ out,
                     int32_t* __restrict__ advance, uint32_t* err) {
  constexpr int NT = kFilterThreads;
  constexpr int NW = kFilterWaves;
  constexpr int kCapGroups = E2 * NT / kGroupTokens;
  static_assert(kCapGroups <= kFilterMaxSurvivors, "survivor list");
  static_assert(NW * RowGeom<BF16, D>::RS * (D + 3) + 1 + NT <= kFilterAttendScratch,
                "attend_rows scratch");
  static_assert(E1 % 4 == 0 && E1 / 4 <= kMaxSlabs && E2 % 4 == 0 && E2 / 4 <= kMaxSlabs,
                "slabs");
  __shared__ FilterLds L;
  const int part = S > 1 ? (int)blockIdx.x / hq : 0;
  const int h = S > 1 ? (int)blockIdx.x % hq : (int)blockIdx.x, b = blockIdx.y;
  const bool lead = part == 0;
  const size_t row = (size_t)b * hq + h;
  const int t = threadIdx.x;

  // The row's group maxima go out before n_b arrives (bounded by the
  // launch's longest row); groups past the row's own length are masked once
  // it is known.
  const int groups_max = (min(max_seq_len, cap) + kGroupTokens - 1) / kGroupTokens;
  uint4 graw[E1 / 4];
  {
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(gmax + row * (size_t)gstride, groups_max * 4);
#pragma unroll
    for (int g = 0; g < E1 / 4; ++g) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(4 * (g * NT + t)) * 4u,
                                                           0, 0);
      graw[g] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  }
  // Both histograms and the pivot gather's counter are cleared while the
  // loads fly (the first barrier below orders that before any count).
  {
    uint4* h1 = reinterpret_cast<uint4*>(L.hist1);
    uint4* h2 = reinterpret_cast<uint4*>(L.hist2);
    for (int i = t; i < kSelBins / 4; i += NT) {
      h1[i] = make_uint4(0, 0, 0, 0);
      h2[i] = make_uint4(0, 0, 0, 0);
    }
    if (t == 0) L.s.cand_n = 0u;
  }
  const int n = checked_len(nb, b, max_seq_len, cap, err, lead && h == 0 && t == 0);
  if (advance != nullptr && lead && h == 0 && t == 0 && n > 0) advance[b] = n;
  int32_t* o = (idx && lead) ? idx + row * budget : nullptr;
  const int bh = row_budget(head_budget, h, budget, err, lead && b == 0 && t == 0);
  const int take = n < bh ? n : bh;
  const bool whole = n <= bh || bh == 0;  // every position, or none

  // Every slot FAC may read starts at position 0 (always a token), so no
  // selection outcome can send its gather out of the row.
  for (int j = t; j < take; j += NT) L.sel[j] = 0;
  if (whole) {
    for (int j = t; j < budget; j += NT) {
      if (o) o[j] = (j < take) ? j : -1;
      if (j < kFusedMaxBudget) L.sel[j] = j;
    }
  } else {
    const float* row_scores = scores + row * cap;
    const int ng = (n + kGroupTokens - 1) / kGroupTokens;
    const uint32_t spare = (uint32_t)(kSelBins + lane_id());
    uint32_t gk[E1];
#pragma unroll
    for (int g = 0; g < E1 / 4; ++g) {
      const uint32_t w4[4] = {graw[g].x, graw[g].y, graw[g].z, graw[g].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) gk[4 * g + e] = (4 * (g * NT + t) + e < ng) ? w4[e] : 0u;
    }

    // 1. Bin P of the bh-th largest group maximum (1024 bins linear in the
    // score over the maxima's range); groups at bin P or above survive.
    // Rows of at most bh groups keep every group.
    bool stream = false;
    const bool filter = ng > bh;
    uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
    for (int e = 0; e < E1; ++e) {
      kmin = min(kmin, gk[e] ? gk[e] : ~0u);
      kmax = max(kmax, gk[e]);
    }
    block_minmax(kmin, kmax, L.s);  // barrier 1
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float span = vmax - vmin;
    const float scale = (float)kSelBins / span;
    uint32_t pbin = 0;
    if (filter) {
      if (isfinite(vmin) && isfinite(vmax) && span > 0.0f && isfinite(span) && isfinite(scale)) {
#pragma unroll
        for (int e = 0; e < E1; ++e) {
          const uint32_t k = gk[e];
          const uint32_t bn = (uint32_t)min(kSelBins - 1, (int)((key_value(k) - vmin) * scale));
          atomicAdd(&L.hist1[k ? bn : spare], 1u);
        }
        __syncthreads();  // barrier 2
        const WavePick p = wave_pick(L.hist1, (uint32_t)bh);
        pbin = p.bin;
        stream = !p.ok || p.above + p.count > (uint32_t)kCapGroups;
      } else {
        stream = true;  // one score value, or non-finite ones
      }
    } else {
      stream = ng > kCapGroups;
    }
    if (!stream) {
      // The surviving groups, ascending, into L.grp (barriers 3, 4).
      // kp: the smallest surviving group maximum (its wave minima ride along
      // with the compaction's barriers).  Every token >= tau has a key >= kp.
      uint32_t m4[E1 / 4], off[E1 / 4];
      uint32_t kmine = ~0u;
#pragma unroll
      for (int g = 0; g < E1 / 4; ++g) {
        m4[g] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = gk[4 * g + e];
          const bool in =
              k != 0u && (!filter || min(kSelBins - 1, (int)((key_value(k) - vmin) * scale)) >=
                                         (int)pbin);
          m4[g] |= (in ? 1u : 0u) << e;
          kmine = in ? min(kmine, k) : kmine;
        }
      }
      {
        uint32_t unused = 0u;
        wave_minmax(kmine, unused);
        if (lane_id() == 0) L.kpmin[t / kWave] = kmine;
      }
      const uint32_t ns = ordered_offsets<NT>(m4, off, L.s);
#pragma unroll
      for (int g = 0; g < E1 / 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((m4[g] >> e) & 1u) {
            if (off[g] < (uint32_t)kCapGroups) L.grp[off[g]] = 4 * (g * NT + t) + e;
            ++off[g];
          }
      __syncthreads();
      uint32_t kp = 1u;  // rows kept whole: every token in play
      if (filter) {
        kp = ~0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) kp = min(kp, L.kpmin[w]);
      }

      // 2. The survivors' scores: thread t holds half of list entry
      // (s NT + t) / 2 in slab s.  Keys below kp are out of play.
      SurvivorSrc<E2> src;
      {
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row_scores, ((n + 3) & ~3) * 4);
        float4 sv[E2 / 4];
#pragma unroll
        for (int s = 0; s < E2 / 4; ++s) {
          const uint32_t li = (uint32_t)(s * NT + t) / 2;
          const int g = li < ns ? L.grp[li] : 0;
          src.g[s] = g;
          const uint32_t at = li < ns ? (uint32_t)(g * kGroupTokens + 4 * (t & 1)) * 4u
                                      : 0xfffffff0u;  // past the range: reads zeros
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, at, 0, 0);
          sv[s] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                              __uint_as_float(x[2]), __uint_as_float(x[3]));
        }
#pragma unroll
        for (int s = 0; s < E2 / 4; ++s) {
          const bool slab = (uint32_t)(s * NT + t) / 2 < ns;
          const int p0 = src.g[s] * kGroupTokens + 4 * (t & 1);
          const float f[4] = {sv[s].x, sv[s].y, sv[s].z, sv[s].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t k0 = score_key(f[e]);
            const uint32_t k = k0 ? k0 : 1u;
            src.k[4 * s + e] = (slab && p0 + e < n && k >= kp) ? k : 0u;
          }
        }
      }
      // Exact tau among the keys in play (all in [kp, kmax], a narrow range
      // near the top of the row): 1024 bins of 2^sh2 keys from kp
      // (barrier 5), each wave picks the pivot bin, its elements are
      // gathered (barrier 6) and ranked by each wave (or refined in LDS when
      // there are many).  Rows kept whole take the score-linear select.
      auto shift_for = [](uint32_t sp) {  // smallest shift fitting sp into the bins
        return sp < (uint32_t)kSelBins ? 0 : 32 - (int)__clz(sp) - kSelBits;
      };
      const int sh2 = shift_for(kmax - kp);
      WavePick p2{0u, 0u, 0u, false};
      if (filter) {
#pragma unroll
        for (int e = 0; e < E2; ++e) {
          const uint32_t k = src.k[e];
          atomicAdd(&L.hist2[k ? (k - kp) >> sh2 : spare], 1u);
        }
        __syncthreads();
        p2 = wave_pick(L.hist2, (uint32_t)bh);
      }
      uint64_t tau = 0;
      if (!filter) {
        tau = adaptive_select<NT, E2>(src, (uint32_t)bh, L.s);
        emit_ordered<E2, NT>(src, tau, (uint32_t)bh, L.s, [&](uint32_t r, int e) {
          const int pos = src.pos(e);
          if (o) o[r] = pos;
          L.sel[r] = pos;
        });
      } else if (!p2.ok) {
        // Fewer in play than bh: never with consistent group maxima.
        if (t == 0) raise_flag(err, FASA_DEVFLAG_SELECT);
        stream = true;
      } else {
        const uint32_t need = (uint32_t)bh - p2.above;
        const uint32_t blo = kp + (p2.bin << sh2);
        const uint32_t bhi = blo + ((1u << sh2) - 1u);  // same bin <=> key in [blo, bhi]
        const uint64_t clo = (uint64_t)blo << 32, chi = ((uint64_t)bhi << 32) | 0xffffffffull;
        if (p2.count <= (uint32_t)kFilterCandCap) {
          const uint32_t M = gather_cand<NT, E2>(src, [&](int e) {
            return src.k[e] >= blo && src.k[e] <= bhi;
          }, L.s);
          tau = M <= (uint32_t)kWave ? wave_rank(L.s.cand, M, need)
                                     : refine<NT, E2>(src, need, clo, chi, true, M, L.s);
        } else {
          // A pivot bin larger than the LDS gather (ties, or short rows kept
          // whole): refinement passes over the registers.
          tau = refine<NT, E2>(src, need, clo, chi, false, 0u, L.s);
        }
        emit_ordered<E2, NT>(src, tau, (uint32_t)bh, L.s, [&](uint32_t r, int e) {
          const int pos = src.pos(e);
          if (o) o[r] = pos;
          L.sel[r] = pos;
        });
      }
    }
    if (stream) {
      // 3. Streaming passes over all of the row's composites.
      __syncthreads();  // LDS of the steps above is reused
      const uint64_t tau =
          stream_select(row_scores, n, (uint32_t)bh, 1ull << 32, ~0ull, L.s, err);
      stream_emit(row_scores, n, tau, (uint32_t)bh, L.s, [&](uint32_t r, int pos) {
        if (o) o[r] = pos;
        L.sel[r] = pos;
      });
    }
    if (o != nullptr)
      for (int j = bh + t; j < budget; j += NT) o[j] = -1;
  }
  __syncthreads();
  float* out_row = out + row * D;
  if (take == 0) {
    if (lead)
      for (int d = t; d < D; d += NT) out_row[d] = 0.0f;
    return;
  }
  const size_t kvbase = ((size_t)b * hkv + h / G) * cap;
  if constexpr (S > 1)
    attend_rows_split<BF16, D, NW, S>(L.sel, take, k_cache, v_cache, qrot, row, kvbase, part,
                                      out_row, L.att);
  else
    attend_rows<BF16, D, NW>(L.sel, take, k_cache, v_cache, qrot, row, kvbase, out_row, L.att);
}

bool filter_path_applies(int max_seq_len, int budget) {
  const long long groups = ((long long)max_seq_len + kGroupTokens - 1) / kGroupTokens;
  // Rows up to 16 scores per thread of one 512-thread select are held whole
  // there (one launch after TIP already).
  return budget >= 1 && budget <= kFusedMaxBudget && max_seq_len > 16 * kFilterThreads &&
         groups <= kFilterMaxGroups;
}

int filter_group_slots(int max_seq_len) {
  const int groups = (max_seq_len + kGroupTokens - 1) / kGroupTokens;
  return groups <= 8 * kFilterThreads ? 8 : 40;
}

// Survivors are about B groups; the slots leave room for those in bin P.
int filter_survivor_slots(int budget) { return budget <= 384 ? 8 : 24; }

// Column parts of the fused FAC when the rows are few (as in select2.hip).
constexpr int kFilterColumnParts = 4;

template <bool BF16, int D, int E1, int E2>
static void launch_filter_t(const fasa_ctx* c, hipStream_t s, const uint32_t* gm,
                            const float* scores, const int32_t* nb, int max_seq_len, int budget,
                            const int32_t* hb, int32_t* idx, const void* k, const void* v,
                            const float* qrot, float* out, int32_t* advance, uint32_t* err) {
  const bool split = (long long)c->batch * c->hq * kFilterColumnParts <= c->cus;
  if (split)
    hipLaunchKernelGGL((filter_select_kernel<BF16, D, E1, E2, kFilterColumnParts>),
                       dim3((unsigned)(c->hq * kFilterColumnParts), (unsigned)c->batch),
                       dim3(kFilterThreads), 0, s, gm, c->ws.gstride, scores, nb, max_seq_len,
                       c->hq, c->cap, budget, hb, idx, k, v, qrot, c->hkv, c->G, out, advance,
                       err);
  else
    hipLaunchKernelGGL((filter_select_kernel<BF16, D, E1, E2, 1>),
                       dim3((unsigned)c->hq, (unsigned)c->batch), dim3(kFilterThreads), 0, s, gm,
                       c->ws.gstride, scores, nb, max_seq_len, c->hq, c->cap, budget, hb, idx,
                       k, v, qrot, c->hkv, c->G, out, advance, err);
}

template <bool BF16, int D>
static void launch_filter_d(const fasa_ctx* c, hipStream_t s, const uint32_t* gm,
                            const float* scores, const int32_t* nb, int max_seq_len, int budget,
                            const int32_t* hb, int32_t* idx, const void* k, const void* v,
                            const float* qrot, float* out, int32_t* advance, uint32_t* err) {
#define FASA_FILTER(E1V, E2V)                                                                 \
  launch_filter_t<BF16, D, E1V, E2V>(c, s, gm, scores, nb, max_seq_len, budget, hb, idx, k, v, \
                                     qrot, out, advance, err)
  const bool short_rows = filter_group_slots(max_seq_len) == 8;
  const bool few = filter_survivor_slots(budget) == 8;
  if (short_rows) {
    if (few) FASA_FILTER(8, 8); else FASA_FILTER(8, 24);
  } else {
    if (few) FASA_FILTER(40, 8); else FASA_FILTER(40, 24);
  }
#undef FASA_FILTER
}

hipError_t launch_filter_select(const fasa_ctx* c, const float* scores, const int32_t* nb,
                                int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                                const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                                hipStream_t s, const int32_t* head_budget) {
  if (!filter_path_applies(max_seq_len, budget) || out == nullptr) return hipErrorInvalidValue;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  const uint32_t* gm = reinterpret_cast<const uint32_t*>(ws + c->ws.gmax);
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf)
      launch_filter_d<true, 128>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                 k_cache, v_cache, qrot, out, advance, err);
    else
      launch_filter_d<false, 128>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                  k_cache, v_cache, qrot, out, advance, err);
  } else {
    if (bf)
      launch_filter_d<true, 64>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                k_cache, v_cache, qrot, out, advance, err);
    else
      launch_filter_d<false, 64>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                 k_cache, v_cache, qrot, out, advance, err);
  }
  return hipGetLastError();
}

}  // namespace fasa
