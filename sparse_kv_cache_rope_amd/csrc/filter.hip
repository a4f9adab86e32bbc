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
// score key of every 16-token group of each row.  Group maxima are scores of
// distinct tokens, so the B-th largest of them is at most tau, and every
// token >= tau lies in a group whose maximum is >= it.  Here:
//   1. one histogram pass over the row's group maxima (bins linear in the
//      score between their min and max) finds the bin P holding the B-th
//      largest; every group whose maximum falls in bin P or above survives
//      (about B groups), and kp, the smallest surviving maximum, is at most
//      tau;
//   2. the survivors' scores (16 each, 64 contiguous bytes) are gathered;
//      those >= kp are "in play" and listed in position order in LDS, and a
//      second histogram (keys from kp) counts them;
//   3. the K and V rows of the in-play tokens are requested right away, so
//      the gather overlaps the rest of the selection: the bin of the B-th
//      largest in-play key gives tau at once when the whole bin is taken,
//      else its few elements are ranked;
//   4. FAC over the list, unselected entries masked: logits of every listed
//      row, then the softmax max and denominator, then the weighted sum of
//      V (two passes over LDS logits instead of an online merge);
//   5. rows this does not fit (fewer groups than B, one score value, more
//      survivors or in-play tokens than the slots hold, a crowded pivot bin)
//      are selected by streaming range refinement over their scores and an
//      ordered streaming emit, then attended the same way.
//
// One 512-thread workgroup per row, or S per row for the FAC's column split
// (each part makes the same selection and writes D / S output columns);
// part 0 writes idx, the advanced length and flags.  No workgroup waits on
// another.

#include "attention_common.hpp"
#include "budget.hpp"
#include "fasa_internal.hpp"
#include "select_common.hpp"
#include "select_src.hpp"

namespace fasa {

constexpr int kFilterThreads = kFilterSelectThreads;
constexpr int kFilterWaves = kFilterThreads / kWave;
// Streaming route: histogram copies and LDS candidates.
constexpr int kFilterHistCopies = 4;
constexpr int kFilterCandCap = 4096;
// In-play tokens listed in LDS, and pivot-bin elements ranked by one wave.
constexpr int kPlayCap = 2048;
constexpr int kPivotCap = kWave;
// Threads per surviving group (a 16-byte score load each).
constexpr int kGroupThreads = kGroupTokens / 4;
// Most surviving groups: 40 survivor slots per thread.
constexpr int kFilterMaxSurvivors = kFilterThreads * 40 / kGroupTokens;
// FAC partial sums: up to 4 row slots per wave of D / S floats each.
constexpr int kFacRedFloats = kFilterWaves * 4 * 128;
static_assert(kPlayCap % kFilterThreads == 0, "emit chunks");

using FilterSelLds = RegSelectLds<kFilterThreads, kFilterHistCopies, kFilterCandCap>;

struct FilterLds {
  union {
    FilterSelLds s;             // streaming route; block_minmax's wave extremes
    float red[kFacRedFloats];   // FAC partial sums (after every select)
  };
  // Histograms of the group maxima and of the in-play keys, cleared at the
  // kernel's start (a spare word per lane past the bins, as in RegSelectLds).
  alignas(16) uint32_t hist1[kSelBins + kWave];
  alignas(16) uint32_t hist2[kSelBins + kWave];
  int32_t grp[kFilterMaxSurvivors];  // surviving groups, ascending
  // The list FAC reads: positions ascending, their keys, their logits.
  int32_t pos[kPlayCap];
  uint32_t key[kPlayCap];
  float z[kPlayCap];
  uint64_t pivot[kPivotCap];
  uint32_t pivot_n;
  uint32_t kpmin[kFilterWaves];  // per-wave smallest surviving group maximum
  uint32_t slab_g[kMaxSlabs * kFilterWaves];
  uint32_t slab_p[kMaxSlabs * kFilterWaves];
  uint32_t emit_cnt[kPlayCap / kWave];
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

// ---- FAC over the in-play list ---------------------------------------------
//
// Rows r < np of the list (L.pos, L.key); a row takes part iff its composite
// is >= tau.  Each of the S parts computes every logit (the softmax needs
// them all) and the weighted V sum of its D / S columns.
//
// K: LPR lanes hold a row (RS rows per wave step); V: VL = LPR / S lanes hold
// a row's column slice (RV rows per wave step).  A round of loads covers RK
// rows of K and RVR rows of V; list slots past np load the list's last row
// (fetched anyway) and count as absent.
template <bool BF16, int D, int S>
struct PlayFac {
  using Geo = RowGeom<BF16, D>;
  static constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS;
  static constexpr int NW = kFilterWaves;
  static_assert(LPR % S == 0, "V slice lanes");
  static constexpr int VL = LPR / S;
  static constexpr int RV = kWave / VL;
  static constexpr int cl(int x) { return x < 1 ? 1 : (x > 10 ? 10 : x); }
  static constexpr int KST = cl(320 / (RS * NW));
  static constexpr int VST = cl((320 + RV * NW - 1) / (RV * NW));
  static constexpr int RK = RS * NW * KST;
  static constexpr int RVR = RV * NW * VST;
  // Row slots of a wave after the in-row V sums, and the floats they hold.
  static constexpr int SLOTS = VL < 16 ? 4 : kWave / VL;
  static constexpr int W = D / S;
  static_assert(NW * SLOTS * W <= kFacRedFloats, "partial sums");
  uint4 k[KST], v[VST];
};

template <class F>
__device__ __forceinline__ void fac_issue_k(F& f, int r0, int np, const int32_t* pos,
                                            const uint4* __restrict__ K, size_t kvbase) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int last = np - 1;
#pragma unroll
  for (int s = 0; s < F::KST; ++s) {
    const int r = r0 + (s * F::NW + wave) * F::RS + lane / F::LPR;
    const int j = pos[r < np ? r : last];
    f.k[s] = K[(kvbase + (size_t)j) * F::LPR + lane % F::LPR];
  }
}

template <class F>
__device__ __forceinline__ void fac_issue_v(F& f, int r0, int np, const int32_t* pos,
                                            const uint4* __restrict__ V, size_t kvbase, int part) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int last = np - 1;
#pragma unroll
  for (int s = 0; s < F::VST; ++s) {
    const int r = r0 + (s * F::NW + wave) * F::RV + lane / F::VL;
    const int j = pos[r < np ? r : last];
    f.v[s] = V[(kvbase + (size_t)j) * F::LPR + part * F::VL + lane % F::VL];
  }
}

// bf16 pair of a float, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 fasa_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(fasa_bf16x2, a),
                                         __builtin_bit_cast(fasa_bf16x2, b), c, false);
}

template <int SH>
__device__ __forceinline__ float row_shr_add(float v) {
  // Lanes with no source SH lanes below in their 16-lane row add 0.
  return v + __int_as_float(
                 __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + SH, 0xf, 0xf, true));
}

// The query's part of a logit: q~ scaled to log2 units; for bf16 rows split
// into a high and a low bf16 pair per two dims (q = hi + lo to about 2^-16),
// so that each 16-byte K load takes EPL dot2 steps and no unpacking.
template <bool BF16, int EPL>
struct FacQuery {
  float q[EPL];
  uint32_t hi[EPL / 2], lo[EPL / 2];
};

template <class F, class Q>
__device__ __forceinline__ void fac_logits(const F& f, const Q& qq, int r0, int np, uint64_t tau,
                                           FilterLds& L) {
  using Geo = typename F::Geo;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int s = 0; s < F::KST; ++s) {
    const uint4 x = f.k[s];
    float dot = 0.0f;
    if constexpr (Geo::ES == 2) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dot = dot2_bf16(w[i], qq.hi[i], dot);
        dot = dot2_bf16(w[i], qq.lo[i], dot);
      }
    } else {
      const float kf[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                           __uint_as_float(x.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = fmaf(qq.q[e], kf[e], dot);
    }
    dot = group_sum<F::LPR>(dot);
    const int r = r0 + (s * F::NW + wave) * F::RS + lane / F::LPR;
    if (lane % F::LPR == 0 && r < np) {
      const bool in = composite(L.key[r], (uint32_t)L.pos[r]) >= tau;
      L.z[r] = in ? dot : -INFINITY;
    }
  }
}

// FAC over the list (loads of the first round already issued in f), this
// part's columns written to out_row.  Two barriers; reads L.pos, L.key.
template <bool BF16, int D, int S>
__device__ __forceinline__ void fac_play(PlayFac<BF16, D, S>& f, int np, uint64_t tau,
                                         const uint4* __restrict__ K, const uint4* __restrict__ V,
                                         size_t kvbase, int part, const float* __restrict__ qrow,
                                         float* __restrict__ out_row, FilterLds& L) {
  using F = PlayFac<BF16, D, S>;
  constexpr int LPR = F::LPR, EPL = F::EPL, VL = F::VL;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  FacQuery<BF16, EPL> qq;
  {
    const float scale = logit_scale<D>();
    const int sub = lane % LPR;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qq.q[e] = qrow[sub * EPL + e] * scale;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        const uint32_t h0 = f32_to_bf16_bits(qq.q[2 * i]), h1 = f32_to_bf16_bits(qq.q[2 * i + 1]);
        const uint32_t l0 = f32_to_bf16_bits(qq.q[2 * i] - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_bits(qq.q[2 * i + 1] - __uint_as_float(h1 << 16));
        qq.hi[i] = h0 | (h1 << 16);
        qq.lo[i] = l0 | (l1 << 16);
      }
    }
  }
  // Logits, round by round (the first round's K is in flight already).
  fac_logits(f, qq, 0, np, tau, L);
  for (int r0 = F::RK; r0 < np; r0 += F::RK) {
    fac_issue_k(f, r0, np, L.pos, K, kvbase);
    fac_logits(f, qq, r0, np, tau, L);
  }
  __syncthreads();
  // Softmax max and denominator over the list, every wave on its own.
  float m = -INFINITY;
  for (int i = lane; i < np; i += kWave) m = fmaxf(m, L.z[i]);
  m = wave_max(m);
  float l = 0.0f;
  for (int i = lane; i < np; i += kWave) l += exp2f(L.z[i] - m);  // -inf gives 0
  l = group_sum<kWave>(l);
  // Weighted V sum of this part's columns.
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int r0 = 0; r0 < np; r0 += F::RVR) {
    if (r0 > 0) fac_issue_v(f, r0, np, L.pos, V, kvbase, part);
#pragma unroll
    for (int s = 0; s < F::VST; ++s) {
      const int r = r0 + (s * F::NW + wave) * F::RV + lane / VL;
      const float p = r < np ? exp2f(L.z[r] - m) : 0.0f;
      float vf[EPL];
      unpack<BF16, EPL>(f.v[s], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
    }
  }
  // Sum over the row slots holding the same slice: within 16-lane rows by
  // DPP, then the waves' rows through LDS.
  if constexpr (VL < 16) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (VL <= 1) acc[e] = row_shr_add<1>(acc[e]);
      if constexpr (VL <= 2) acc[e] = row_shr_add<2>(acc[e]);
      if constexpr (VL <= 4) acc[e] = row_shr_add<4>(acc[e]);
      acc[e] = row_shr_add<8>(acc[e]);
    }
  }
  const bool holder = VL < 16 ? (lane & 15) >= 16 - VL : true;
  const int slot = VL < 16 ? lane >> 4 : lane / VL;
  if (holder) {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      L.red[(wave * F::SLOTS + slot) * F::W + (lane % VL) * EPL + e] = acc[e];
  }
  __syncthreads();
  if (t < F::W) {
    float sum = 0.0f;
#pragma unroll 8
    for (int st = 0; st < F::NW * F::SLOTS; ++st) sum += L.red[st * F::W + t];
    out_row[part * F::W + t] = l > 0.0f ? sum / l : 0.0f;
  }
}

// Smallest shift that fits [0, sp] into the histogram's bins.
__device__ __forceinline__ int bin_shift(uint32_t sp) {
  return sp < (uint32_t)kSelBins ? 0 : 32 - (int)__clz(sp) - kSelBits;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  uint32_t unused = 0u;
  wave_minmax(v, unused);
  return v;
}

// T_t of row (b, h) from the group maxima (see the file comment), written to
// idx (part 0, if given) and attended (FAC) by every part for its columns.
// E1 group maxima per thread (E1 NT >= the row's groups), E2 survivor slots
// per thread (E2 NT / 16 groups).
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
  static_assert(E1 % 4 == 0 && E1 / 4 <= kMaxSlabs && E2 % 4 == 0 && E2 / 4 <= kMaxSlabs,
                "slabs");
  using F = PlayFac<BF16, D, S>;
  __shared__ FilterLds L;
  const int part = S > 1 ? (int)blockIdx.x / hq : 0;
  const int h = S > 1 ? (int)blockIdx.x % hq : (int)blockIdx.x, b = blockIdx.y;
  const bool lead = part == 0;
  const size_t row = (size_t)b * hq + h;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;

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
  // Both histograms and the pivot counter are cleared while the loads fly
  // (the first barrier below orders that before any count).
  {
    uint4* h1 = reinterpret_cast<uint4*>(L.hist1);
    uint4* h2 = reinterpret_cast<uint4*>(L.hist2);
    for (int i = t; i < kSelBins / 4; i += NT) {
      h1[i] = make_uint4(0, 0, 0, 0);
      h2[i] = make_uint4(0, 0, 0, 0);
    }
    if (t == 0) L.pivot_n = 0u;
  }
  const int n = checked_len(nb, b, max_seq_len, cap, err, lead && h == 0 && t == 0);
  if (advance != nullptr && lead && h == 0 && t == 0 && n > 0) advance[b] = n;
  int32_t* o = (idx && lead) ? idx + row * budget : nullptr;
  const int bh = row_budget(head_budget, h, budget, err, lead && b == 0 && t == 0);
  const int take = n < bh ? n : bh;
  const bool whole = n <= bh || bh == 0;  // every position, or none
  const float* row_scores = scores + row * cap;
  const size_t kvbase = ((size_t)b * hkv + h / G) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);

  int np = take;      // entries of the list FAC reads
  uint64_t tau = 0;   // an entry takes part <=> its composite >= tau
  F fac;
  bool issued = false;  // the first round of FAC loads is in flight
  bool cold = false;    // the streaming route selects this row

  if (whole) {
    for (int j = t; j < take; j += NT) {
      L.pos[j] = j;
      L.key[j] = 1u;
    }
    if (o)
      for (int j = t; j < budget; j += NT) o[j] = (j < take) ? j : -1;
  } else {
    const int ng = (n + kGroupTokens - 1) / kGroupTokens;
    cold = ng <= bh;  // every group would survive
    if (!cold) {
      // 1. Bin P of the bh-th largest group maximum (1024 bins linear in the
      // score over the maxima's range); groups at bin P or above survive.
      uint32_t gk[E1];
#pragma unroll
      for (int g = 0; g < E1 / 4; ++g) {
        const uint32_t w4[4] = {graw[g].x, graw[g].y, graw[g].z, graw[g].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) gk[4 * g + e] = (4 * (g * NT + t) + e < ng) ? w4[e] : 0u;
      }
      uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
      for (int e = 0; e < E1; ++e) {
        kmin = min(kmin, gk[e] ? gk[e] : ~0u);
        kmax = max(kmax, gk[e]);
      }
      block_minmax(kmin, kmax, L.s);  // barrier
      const float vmin = key_value(kmin), vmax = key_value(kmax);
      const float span = vmax - vmin;
      const float scale = (float)kSelBins / span;
      cold = !(isfinite(vmin) && isfinite(vmax) && span > 0.0f && isfinite(span) &&
               isfinite(scale));
      WavePick p{0u, 0u, 0u, false};
      uint32_t bn[E1];
      if (!cold) {
#pragma unroll
        for (int e = 0; e < E1; ++e) {
          const uint32_t k = gk[e];
          bn[e] = (uint32_t)min(kSelBins - 1, (int)((key_value(k) - vmin) * scale));
          if (k) atomicAdd(&L.hist1[bn[e]], 1u);
        }
        __syncthreads();
        p = wave_pick(L.hist1, (uint32_t)bh);
        cold = !p.ok || p.above + p.count > (uint32_t)kCapGroups;
      }
      if (!cold) {
        // The surviving groups, ascending, into L.grp; kp, the smallest
        // surviving maximum (its wave minima ride along with the barriers).
        uint32_t m4[E1 / 4], off[E1 / 4];
        uint32_t kmine = ~0u;
#pragma unroll
        for (int g = 0; g < E1 / 4; ++g) {
          m4[g] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = gk[4 * g + e] != 0u && bn[4 * g + e] >= p.bin;
            m4[g] |= (in ? 1u : 0u) << e;
            kmine = in ? min(kmine, gk[4 * g + e]) : kmine;
          }
        }
        kmine = wave_min_u32(kmine);
        if (lane == 0) L.kpmin[wave] = kmine;
        const uint32_t ns = ordered_offsets_tab<NT>(m4, off, L.slab_g);
#pragma unroll
        for (int g = 0; g < E1 / 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((m4[g] >> e) & 1u) L.grp[off[g]++] = 4 * (g * NT + t) + e;
        __syncthreads();
        uint32_t kp = ~0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) kp = min(kp, L.kpmin[w]);

        // 2. The survivors' scores: slab s of thread t holds the quarter
        // t % 4 of list entry (s NT + t) / 4, so (slab, thread, element)
        // order is position order.  Keys below kp are out of play.
        uint32_t kk[E2];
        int p0[E2 / 4];
        {
          const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row_scores, ((n + 3) & ~3) * 4);
          float4 sv[E2 / 4];
#pragma unroll
          for (int s = 0; s < E2 / 4; ++s) {
            const uint32_t li = (uint32_t)(s * NT + t) / kGroupThreads;
            const int g = li < ns ? L.grp[li] : 0;
            p0[s] = g * kGroupTokens + 4 * (t % kGroupThreads);
            const uint32_t at = li < ns ? (uint32_t)p0[s] * 4u : 0xfffffff0u;  // past: zeros
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, at, 0, 0);
            sv[s] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                __uint_as_float(x[2]), __uint_as_float(x[3]));
          }
#pragma unroll
          for (int s = 0; s < E2 / 4; ++s) {
            const bool slab = (uint32_t)(s * NT + t) / kGroupThreads < ns;
            const float fv[4] = {sv[s].x, sv[s].y, sv[s].z, sv[s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t k0 = score_key(fv[e]);
              const uint32_t k = k0 ? k0 : 1u;
              kk[4 * s + e] = (slab && p0[s] + e < n && k >= kp) ? k : 0u;
            }
          }
        }
        // The in-play tokens, in position order, into the list; their keys
        // counted in 1024 bins of 2^sh2 keys from kp.
        const int sh2 = bin_shift(kmax - kp);
        uint32_t mp[E2 / 4], offp[E2 / 4];
#pragma unroll
        for (int s = 0; s < E2 / 4; ++s) {
          mp[s] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t k = kk[4 * s + e];
            mp[s] |= (k ? 1u : 0u) << e;
            if (k) atomicAdd(&L.hist2[(k - kp) >> sh2], 1u);
          }
        }
        np = (int)ordered_offsets_tab<NT>(mp, offp, L.slab_p);  // barrier (hist2 complete)
        cold = np > kPlayCap;
        if (!cold) {
#pragma unroll
          for (int s = 0; s < E2 / 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if ((mp[s] >> e) & 1u) {
                L.pos[offp[s]] = p0[s] + e;
                L.key[offp[s]] = kk[4 * s + e];
                ++offp[s];
              }
          __syncthreads();
          // 3. The rows FAC will read go out now.
          fac_issue_k(fac, 0, np, L.pos, K, kvbase);
          fac_issue_v(fac, 0, np, L.pos, V, kvbase, part);
          issued = true;
          const WavePick p2 = wave_pick(L.hist2, (uint32_t)bh);
          if (!p2.ok) {
            // Fewer in play than bh: never with consistent group maxima.
            if (t == 0) raise_flag(err, FASA_DEVFLAG_SELECT);
            cold = true;
          } else {
            const uint32_t need = (uint32_t)bh - p2.above;
            const uint32_t blo = kp + (p2.bin << sh2);
            const uint64_t bend = (uint64_t)blo + ((1ull << sh2) - 1ull);
            const uint32_t bhi = bend > 0xffffffffull ? 0xffffffffu : (uint32_t)bend;
            if (p2.count == need) {
              tau = (uint64_t)blo << 32;  // the whole pivot bin is taken
            } else {
              // The pivot bin's few elements, ranked by each wave.
              for (int i = t; i < np; i += NT) {
                const uint32_t k = L.key[i];
                if (k >= blo && k <= bhi) {
                  const uint32_t at = atomicAdd(&L.pivot_n, 1u);
                  if (at < (uint32_t)kPivotCap) L.pivot[at] = composite(k, (uint32_t)L.pos[i]);
                }
              }
              __syncthreads();
              const uint32_t M = L.pivot_n;
              if (M > (uint32_t)kPivotCap) cold = true;
              else tau = wave_rank(L.pivot, M, need);
            }
          }
        }
      }
    }
    if (cold) {
      // 5. Streaming passes over all of the row's composites.
      __syncthreads();  // LDS of the steps above is reused
      const uint64_t ts =
          stream_select(row_scores, n, (uint32_t)bh, 1ull << 32, ~0ull, L.s, err);
      stream_emit(row_scores, n, ts, (uint32_t)bh, L.s, [&](uint32_t r, int pos) {
        if (o) o[r] = pos;
        L.pos[r] = pos;
        L.key[r] = 1u;
      });
      np = take;
      tau = 0;
      issued = false;
    } else if (o != nullptr) {
      // idx: each listed entry's rank among the selected ones (the list is
      // in position order); one barrier.
      constexpr int CH = kPlayCap / NT;
      uint32_t pre[CH];
      bool sel[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int i = c * NT + t;
        sel[c] = i < np && composite(L.key[i], (uint32_t)L.pos[i]) >= tau;
        const uint64_t bal = __ballot(sel[c]);
        pre[c] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (lane == 0) L.emit_cnt[c * NW + wave] = (uint32_t)__popcll(bal);
      }
      __syncthreads();
      uint32_t before = 0;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        uint32_t mine = before;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const uint32_t cnt = L.emit_cnt[c * NW + w];
          mine += w < wave ? cnt : 0u;
          before += cnt;
        }
        if (sel[c] && mine + pre[c] < (uint32_t)bh) o[mine + pre[c]] = L.pos[c * NT + t];
      }
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
  // 4. FAC over the list.
  if (!issued) {
    fac_issue_k(fac, 0, np, L.pos, K, kvbase);
    fac_issue_v(fac, 0, np, L.pos, V, kvbase, part);
  }
  fac_play<BF16, D, S>(fac, np, tau, K, V, kvbase, part, qrot + row * D, out_row, L);
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
  return groups <= 4 * kFilterThreads ? 4 : 20;
}

// Survivors are about B groups; the slots leave room for those in bin P.
int filter_survivor_slots(int budget) { return budget <= 320 ? 12 : 40; }

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
  const bool short_rows = filter_group_slots(max_seq_len) == 4;
  const bool few = filter_survivor_slots(budget) == 12;
  if (short_rows) {
    if (few) FASA_FILTER(4, 12); else FASA_FILTER(4, 40);
  } else {
    if (few) FASA_FILTER(20, 12); else FASA_FILTER(20, 40);
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
