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
//   2. each wave reads the scores of the surviving groups it holds (group g
//      belongs to thread g mod 512, so a run of groups spreads over all
//      waves) and lists its tokens >= kp, "in play", in position order in
//      its own part of LDS, with no barrier;
//   3. each wave requests the K and V rows of its listed tokens at once, so
//      the gathers overlap the rest of the selection, and counts the listed
//      keys in a shared histogram (bins of keys from kp): the bin of the
//      B-th largest in-play key gives tau at once when the whole bin is
//      taken, else its few elements are ranked;
//   4. FAC, each wave over its own list (entries below tau masked): logits
//      (on the matrix cores for bf16 at d = 128 when the list's rows are all
//      in flight at once), the wave's softmax max and sum, its weighted V
//      sum, then one merge of the waves' states through LDS; when some wave's list is long (tokens
//      clustered in few waves' groups), T_t is first laid out flat and split
//      evenly over the waves;
//   5. rows this does not fit (fewer groups than B, one score value, more
//      survivors or in-play tokens than the slots hold, a crowded pivot bin)
//      are selected by streaming range refinement over their scores and an
//      ordered streaming emit, then attended the same way (the list split
//      evenly over the waves).
// With idx requested, part 0 also writes T_t in position order: the waves'
// runs of positions interleave in a fixed pattern, so per-(block, wave)
// counts of the selected entries give every entry its rank.
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
// In-play tokens a wave lists, and pivot-bin elements ranked by one wave.
constexpr int kWavePlayCap = 512;
constexpr int kPivotCap = kWave;
// Lanes per surviving group (a 16-byte score load each).
constexpr int kGroupLanes = kGroupTokens / 4;
// Surviving groups a wave holds: 40 survivor slots per lane at most.
constexpr int kWaveMaxSurvivors = kWave * 40 / kGroupTokens;
// FAC partial sums: one state of D / S floats per wave.
constexpr int kFacRedFloats = kFilterWaves * 128;
static_assert(kFusedMaxBudget <= kFilterWaves * kWavePlayCap, "a streamed T_t fits the lists");

using FilterSelLds = RegSelectLds<kFilterThreads, kFilterHistCopies, kFilterCandCap>;

struct FilterLds {
  union {
    FilterSelLds s;           // streaming route; block_minmax's wave extremes
    int32_t emit[kFilterWaves][kWavePlayCap];  // idx: each wave's selected positions
  };
  // Histograms of the group maxima and of the in-play keys, cleared at the
  // kernel's start (a spare word per lane past the bins, as in RegSelectLds).
  alignas(16) uint32_t hist1[kSelBins + kWave];
  alignas(16) uint32_t hist2[kSelBins + kWave];
  // Each wave's surviving groups and in-play list (positions ascending, their
  // keys); a streamed or whole T_t lies flat over pos.
  int32_t grp[kFilterWaves][kWaveMaxSurvivors];
  int32_t pos[kFilterWaves * kWavePlayCap];
  uint32_t key[kFilterWaves * kWavePlayCap];
  float red[kFacRedFloats];  // FAC: the waves' partial sums
  // FAC on the matrix cores (bf16, d = 128): the scaled query's high and low
  // bf16 halves, staged once per workgroup.
  alignas(16) uint16_t qhi[128], qlo[128];
  float zw[kFilterWaves][64];  // FAC: a wave's logits of one round
  float mw[kFilterWaves], lw[kFilterWaves];
  uint64_t pivot[kPivotCap];
  uint32_t pivot_n;
  uint32_t kpmin[kFilterWaves];   // per-wave smallest surviving group maximum
  uint32_t overflow;              // a wave's survivors or list did not fit
  int32_t wcnt[kFilterWaves];     // each wave's list length
  uint32_t selcnt[kFilterWaves];  // each wave's selected entries (FAC rebalance)
  // idx: selected tokens per (block of 512 groups, wave), then each one's
  // first rank.
  alignas(16) uint32_t emit_cnt[kFilterMaxGroups / kFilterThreads][kFilterWaves];
  uint32_t emit_base[kFilterMaxGroups / kFilterThreads][kFilterWaves];
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
  uint32_t q4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) q4[q] = c[4 * q] + c[4 * q + 1] + c[4 * q + 2] + c[4 * q + 3];
  const uint32_t local = q4[0] + q4[1] + q4[2] + q4[3];
  const uint32_t incl = wave_scan_incl(local);
  const uint32_t before = incl - local;
  const uint64_t bal = __ballot(before < need && need <= incl);
  WavePick p{0u, 0u, 0u, bal != 0ull};
  if (!p.ok) return p;
  // The target lane's bin: first the run of 4 (ranks 4 q ..) holding it,
  // then the bin within that run.
  uint32_t qsel = 0, acc = before, qacc = before;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bool hit = acc < need && need <= acc + q4[q];
    qsel = hit ? (uint32_t)q : qsel;
    qacc = hit ? acc : qacc;
    acc += q4[q];
  }
  uint32_t cq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    cq[i] = qsel == 0 ? c[i] : qsel == 1 ? c[4 + i] : qsel == 2 ? c[8 + i] : c[12 + i];
  uint32_t bin = 0, above = 0, count = 0;
  acc = qacc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (acc < need && need <= acc + cq[i]) {
      bin = (uint32_t)(kSelBins - 1 - 16 * l) - (4u * qsel + (uint32_t)i);
      above = acc;
      count = cq[i];
    }
    acc += cq[i];
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

// ---- FAC over a wave's list ------------------------------------------------
//
// A wave attends over its own list entries r < cnt (positions pos[r], keys
// key[r]); an entry takes part iff its composite is >= tau.  K: LPR lanes
// hold a row (RS rows per step); V: VL = LPR / S lanes hold the row's column
// slice of this part (RV rows per step).  A round covers RR entries: their
// logits (through the wave's LDS slot), the round's max, a rescale of the
// wave's running state, and the weighted V sum.  Two register sets hold
// consecutive rounds, so round r + 1's rows fly while round r is computed.
// Entries past cnt load the list's last row (fetched anyway) and count as
// absent.
template <bool BF16, int D, int S, bool MFOK>
struct WaveFac {
  using Geo = RowGeom<BF16, D>;
  static constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS;
  static_assert(LPR % S == 0, "V slice lanes");
  static constexpr int VL = LPR / S;
  static constexpr int RV = kWave / VL;
  static constexpr int KST = (32 / RS) > 8 ? 8 : (32 / RS) < 1 ? 1 : (32 / RS);
  static constexpr int RR = RS * KST;
  static constexpr int VST = (RR + RV - 1) / RV;
  static_assert(2 * RR <= 64, "two rounds' logits fit the wave's LDS slot");
  // Floats of a wave's state (this part's columns).
  static constexpr int W = D / S;
  // bf16 at d = 128, lists whose rounds are all in flight at once (the TRIM
  // issue and round): logits on the matrix cores.  k[4 t + kk] then holds,
  // for 16-row tile t of the round, row 16 t + lane % 16's 16-byte chunk
  // lane / 16 + 4 kk (dims 32 kk + 8 (lane / 16) ..): the A operand of
  // v_mfma_f32_16x16x32_bf16 step kk.
  static constexpr bool MF = MFOK && BF16 && D == 128;
  static_assert(!MF || (KST == 8 && RR == 32), "two 16-row tiles of 4 steps");
  static_assert(VL <= 32 && kFilterWaves * W <= kFacRedFloats, "partial sums");
  uint4 k[KST], v[VST];
};

// Issues round r0's K and V loads (cnt >= 1).  TRIM: a step whose rows all
// lie past cnt loads nothing (fac_round<.., true> skips it); only for rounds
// after which no further loads are issued, since the guards cost the
// compiler its exact load counts.
template <bool TRIM, class F>
__device__ __forceinline__ void fac_issue(F& f, int r0, int cnt, const int32_t* pos,
                                          const uint4* __restrict__ K, const uint4* __restrict__ V,
                                          size_t kvbase, int part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int last = cnt - 1;
  if constexpr (F::MF && TRIM) {
#pragma unroll
    for (int s = 0; s < F::KST; ++s) {
      const int t = s / 4, kk = s % 4;
      if (TRIM && r0 + 16 * t >= cnt) continue;
      const int r = r0 + 16 * t + lane % 16;
      const int j = pos[r < cnt ? r : last];
      f.k[s] = K[(kvbase + (size_t)j) * F::LPR + lane / 16 + 4 * kk];
    }
  } else {
#pragma unroll
    for (int s = 0; s < F::KST; ++s) {
      if (TRIM && r0 + s * F::RS >= cnt) continue;
      const int r = r0 + s * F::RS + lane / F::LPR;
      const int j = pos[r < cnt ? r : last];
      f.k[s] = K[(kvbase + (size_t)j) * F::LPR + lane % F::LPR];
    }
  }
#pragma unroll
  for (int s = 0; s < F::VST; ++s) {
    if (TRIM && r0 + s * F::RV >= cnt) continue;
    const int r = r0 + s * F::RV + lane / F::VL;
    const int j = pos[r < cnt ? r : last];
    f.v[s] = V[(kvbase + (size_t)j) * F::LPR + part * F::VL + lane % F::VL];
  }
}

// bf16 bits of a float, round to nearest even (finite inputs).
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

// The query's part of a logit: q~ scaled to log2 units; for bf16 rows also
// split into a high and a low bf16 pair per two dims (q = hi + lo to about
// 2^-16), so a 16-byte K load takes EPL dot2 steps and no unpacking.
template <int EPL>
struct FacQuery {
  float q[EPL];
  uint32_t hi[EPL / 2], lo[EPL / 2];
};

// This lane's EPL query values (its 16-byte column chunk of a K row), loaded
// at the kernel's start so that FAC never waits for them.
template <bool BF16, int D>
struct QueryRaw {
  float4 v[RowGeom<BF16, D>::EPL / 4];
};

template <bool BF16, int D>
__device__ __forceinline__ QueryRaw<BF16, D> load_query(const float* __restrict__ qrow) {
  constexpr int LPR = RowGeom<BF16, D>::LPR, EPL = RowGeom<BF16, D>::EPL;
  QueryRaw<BF16, D> r;
  const int sub = (threadIdx.x & (kWave - 1)) % LPR;
  const float4* q4 = reinterpret_cast<const float4*>(qrow + sub * EPL);
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) r.v[i] = q4[i];
  return r;
}

template <bool BF16, int D>
__device__ __forceinline__ FacQuery<RowGeom<BF16, D>::EPL> fac_query(const QueryRaw<BF16, D>& raw) {
  constexpr int EPL = RowGeom<BF16, D>::EPL;
  FacQuery<EPL> qq;
  const float scale = logit_scale<D>();
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) {
    qq.q[4 * i] = raw.v[i].x * scale;
    qq.q[4 * i + 1] = raw.v[i].y * scale;
    qq.q[4 * i + 2] = raw.v[i].z * scale;
    qq.q[4 * i + 3] = raw.v[i].w * scale;
  }
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
  return qq;
}

// The B operand of the matrix-core logits: column 0 holds the scaled query's
// high bf16 half, column 1 its low half (so a logit is column 0 plus column
// 1, within about 2^-16 of q~ . k), the other columns zero.  Lane l holds
// column l % 16, dims 32 kk + 8 (l / 16) .. + 7 for step kk.
typedef __bf16 fasa_fbf16x8 __attribute__((ext_vector_type(8)));
typedef float fasa_ff32x4 __attribute__((ext_vector_type(4)));

struct FacQueryM {
  fasa_fbf16x8 b[4];
};

__device__ __forceinline__ FacQueryM fac_query_mfma(const FilterLds& L) {
  const int lane = threadIdx.x & (kWave - 1), c = lane % 16;
  FacQueryM qm;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int d0 = 32 * kk + 8 * (lane / 16);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c < 2) v = *reinterpret_cast<const uint4*>(c == 0 ? &L.qhi[d0] : &L.qlo[d0]);
    qm.b[kk] = __builtin_bit_cast(fasa_fbf16x8, v);
  }
  return qm;
}

// The wave's online-softmax state over its list.
template <int EPL>
struct WaveSoft {
  float m, l, acc[EPL];
};

// One round: logits of the entries r0 .. in the register sets given (one
// set: RR entries; both: 2 RR, f0's then f1's), then their weighted V.  The
// dot products are independent chains (so they interleave), their group sums
// likewise; lane i then masks entry r0 + i (past cnt, or below tau) and the
// masked logits go back through the wave's LDS slot.
template <int NSETS, bool TRIM, class F, class Q>
__device__ __forceinline__ void fac_round(const F& f0, const F& f1, const Q& qq, int r0, int cnt,
                                          const int32_t* pos, const uint32_t* key, uint64_t tau,
                                          float* zw, WaveSoft<F::EPL>& st) {
  constexpr int LPR = F::LPR, EPL = F::EPL, VL = F::VL;
  constexpr int KS = F::KST * NSETS, VS = F::VST * NSETS, RN = F::RR * NSETS;
  static_assert(RN <= kWave, "a round's logits fit the wave's LDS slot");
  const int lane = threadIdx.x & (kWave - 1);
  // Step s's first entry; with TRIM a step whose entries all lie past cnt
  // (its rows were never loaded) is skipped: they are masked below anyway.
  auto kfirst = [&](int s) { return r0 + (s / F::KST) * F::RR + (s % F::KST) * F::RS; };
  auto vfirst = [&](int s) { return r0 + (s / F::VST) * F::RR + (s % F::VST) * F::RV; };
  if constexpr (F::MF && TRIM) {
    // Per 16-row tile, 4 matrix-core steps; the D fragment's lane l holds
    // rows 4 (l / 16) + i of column l % 16, and a row's logit is column 0
    // plus column 1 (lane l + 1).
#pragma unroll
    for (int t = 0; t < 2 * NSETS; ++t) {
      if (TRIM && r0 + 16 * t >= cnt) continue;
      fasa_ff32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 x = t < 2 ? f0.k[4 * (t % 2) + kk] : f1.k[4 * (t % 2) + kk];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fasa_fbf16x8, x),
                                                      qq.b[kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] + __int_as_float(__builtin_amdgcn_update_dpp(
                                     0, __float_as_int(acc[i]), 0x101, 0xf, 0xf, true));
        if (lane % 16 == 0) zw[16 * t + 4 * (lane / 16) + i] = v;
      }
    }
  } else {
  float d[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    d[s] = 0.0f;
    if (TRIM && kfirst(s) >= cnt) continue;
    const uint4 x = s < F::KST ? f0.k[s % F::KST] : f1.k[s % F::KST];
    if constexpr (F::Geo::ES == 2) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      float a = 0.0f, c = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a = dot2_bf16(w[i], qq.hi[i], a);
        c = dot2_bf16(w[i], qq.lo[i], c);
      }
      d[s] = a + c;
    } else {
      d[s] = fmaf(qq.q[0], __uint_as_float(x.x), qq.q[1] * __uint_as_float(x.y)) +
             fmaf(qq.q[2], __uint_as_float(x.z), qq.q[3] * __uint_as_float(x.w));
    }
  }
#pragma unroll
  for (int s = 0; s < KS; ++s)
    if (!TRIM || kfirst(s) < cnt) d[s] = group_sum<LPR>(d[s]);
  if (lane % LPR == 0) {
    // Set k's step s covers round entries k RR + s RS + lane / LPR.
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (!TRIM || kfirst(s) < cnt)
        zw[(s / F::KST) * F::RR + (s % F::KST) * F::RS + lane / LPR] = d[s];
  }
  }
  // The wave reads back what its own lanes wrote (LDS keeps a wave's
  // accesses in order); the barrier only stops the compiler moving them.
  __builtin_amdgcn_wave_barrier();
  float zl = -INFINITY;
  {
    const int r = r0 + lane;
    if (lane < RN && r < cnt && composite(key[r], (uint32_t)pos[r]) >= tau) zl = zw[lane];
  }
  const float mr = wave_max(zl);
  const float mn = fmaxf(st.m, mr);
  if (mn == -INFINITY) return;  // nothing selected yet (wave-uniform)
  __builtin_amdgcn_wave_barrier();
  if (lane < RN) zw[lane] = zl;
  __builtin_amdgcn_wave_barrier();
  const float sc = exp2f(st.m - mn);  // m = -inf gives 0
  st.l *= sc;
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] *= sc;
  st.m = mn;
#pragma unroll
  for (int s = 0; s < VS; ++s) {
    if (TRIM && vfirst(s) >= cnt) continue;
    const int rr = (s / F::VST) * F::RR + (s % F::VST) * F::RV + lane / VL;
    const bool in_set = (s % F::VST) * F::RV + lane / VL < F::RR;
    const float z = in_set ? zw[in_set ? rr : 0] : -INFINITY;
    const float p = exp2f(z - mn);  // -inf gives 0
    float vf[EPL];
    unpack<F::Geo::ES == 2, EPL>(s < F::VST ? f0.v[s % F::VST] : f1.v[s % F::VST], vf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[e] = fmaf(p, vf[e], st.acc[e]);
    if (lane % VL == 0) st.l += p;
  }
  __builtin_amdgcn_wave_barrier();  // zw is rewritten next round
}

// FAC of a wave over its list (rounds 0 and 1 already in flight in f0 / f1
// when `issued` says so), its state left in L.red / L.mw / L.lw for
// fac_merge.
template <bool BF16, int D, int S, bool MFOK>
__device__ __forceinline__ void fac_wave(WaveFac<BF16, D, S, MFOK>& f0,
                                         WaveFac<BF16, D, S, MFOK>& f1,
                                         int issued, int cnt, const int32_t* pos,
                                         const uint32_t* key, uint64_t tau,
                                         const uint4* __restrict__ K, const uint4* __restrict__ V,
                                         size_t kvbase, int part,
                                         const QueryRaw<BF16, D>& qraw, FilterLds& L) {
  using F = WaveFac<BF16, D, S, MFOK>;
  constexpr int EPL = F::EPL, VL = F::VL;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

  WaveSoft<EPL> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] = 0.0f;
  float* zw = L.zw[wave];
  const int nr = (cnt + F::RR - 1) / F::RR;
  if (nr <= 2) {
    // Both sets as one round: one max, one rescale.  The whole list is in
    // flight, so its logits may take the matrix cores (bf16, d = 128).
    const auto qq = [&]() {
      if constexpr (F::MF) return fac_query_mfma(L);
      else return fac_query<BF16, D>(qraw);
    }();
    if (nr > 0 && issued < 1) fac_issue<true>(f0, 0, cnt, pos, K, V, kvbase, part);
    if (nr > 1 && issued < 2) fac_issue<true>(f1, F::RR, cnt, pos, K, V, kvbase, part);
    if (nr == 2) fac_round<2, true>(f0, f1, qq, 0, cnt, pos, key, tau, zw, st);
    else if (nr == 1) fac_round<1, true>(f0, f1, qq, 0, cnt, pos, key, tau, zw, st);
  } else {
    const auto qq = fac_query<BF16, D>(qraw);
    // Longer lists: round r computed while round r + 1 flies.
    if (issued < 1) fac_issue<false>(f0, 0, cnt, pos, K, V, kvbase, part);
    if (issued < 2) fac_issue<false>(f1, F::RR, cnt, pos, K, V, kvbase, part);
    for (int r = 0; r < nr; r += 2) {
      fac_round<1, false>(f0, f0, qq, r * F::RR, cnt, pos, key, tau, zw, st);
      if (r + 2 < nr) fac_issue<false>(f0, (r + 2) * F::RR, cnt, pos, K, V, kvbase, part);
      if (r + 1 < nr) {
        fac_round<1, false>(f1, f1, qq, (r + 1) * F::RR, cnt, pos, key, tau, zw, st);
        if (r + 3 < nr) fac_issue<false>(f1, (r + 3) * F::RR, cnt, pos, K, V, kvbase, part);
      }
    }
  }
  // Sum over the row slots holding the same slice: within 16-lane rows by
  // DPP, the rows and waves through LDS.
  if constexpr (VL < 16) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (VL <= 1) st.acc[e] = row_shr_add<1>(st.acc[e]);
      if constexpr (VL <= 2) st.acc[e] = row_shr_add<2>(st.acc[e]);
      if constexpr (VL <= 4) st.acc[e] = row_shr_add<4>(st.acc[e]);
      st.acc[e] = row_shr_add<8>(st.acc[e]);
    }
  }
  // Then across the wave's rows of 16 lanes (lane l meets l ^ 16, l ^ 32):
  // lanes 48 .. 63 end with the wave's sums, slice l % VL in lane l.
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] += __shfl_xor(st.acc[e], 32);
  if constexpr (VL <= 16) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[e] += __shfl_xor(st.acc[e], 16);
  }
  if (lane >= kWave - VL) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) L.red[wave * F::W + (lane % VL) * EPL + e] = st.acc[e];
  }
  const float l = group_sum<kWave>(st.l);
  if (lane == 0) {
    L.mw[wave] = st.m;
    L.lw[wave] = l;
  }
}

// The waves' states merged (after a barrier): this part's columns.  Thread t
// takes wave t % 8's term of column t / 8 (and of every further column
// 64 apart), and the 8 lanes holding one column's terms sum them.
template <bool BF16, int D, int S>
__device__ __forceinline__ void fac_merge(float* __restrict__ out_row, int part, FilterLds& L) {
  using F = WaveFac<BF16, D, S, false>;
  constexpr int NW = kFilterWaves;
  static_assert(NW == 8, "a column's terms are 8 consecutive lanes");
  const int t = threadIdx.x, w = t % NW;
  if (t / NW >= F::W) return;  // whole waves (W is a multiple of 8)
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) mx = fmaxf(mx, L.mw[i]);
  const float wt = mx == -INFINITY ? 0.0f : exp2f(L.mw[w] - mx);  // m = -inf gives 0
  float lsum = L.lw[w] * wt;
  lsum += __shfl_xor(lsum, 1);
  lsum += __shfl_xor(lsum, 2);
  lsum += __shfl_xor(lsum, 4);
  for (int col = t / NW; col < F::W; col += kFilterThreads / NW) {
    float v = L.red[w * F::W + col] * wt;
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (w == 0) out_row[part * F::W + col] = lsum > 0.0f ? v / lsum : 0.0f;
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

__device__ __forceinline__ uint32_t lanes_below_count(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// T_t of row (b, h) from the group maxima (see the file comment), written to
// idx (part 0, if given) and attended (FAC) by every part for its columns.
// E1 group maxima per thread (E1 NT >= the row's groups), E2 survivor slots
// per lane (a wave holds E2 * 64 / 16 surviving groups).
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
  constexpr int kCapW = E2 * kWave / kGroupTokens;  // surviving groups a wave holds
  static_assert(kCapW <= kWaveMaxSurvivors && E2 % 4 == 0, "survivor slots");
  // Matrix-core logits for the small survivor slots (B <= 320): those lists
  // stay within the two rounds in flight.  Larger budgets run their long
  // lists' pipelined rounds on VALU, and their instances carry no
  // matrix-core code at all.
  using F = WaveFac<BF16, D, S, (E2 <= 16)>;
  __shared__ FilterLds L;
  const int part = S > 1 ? (int)blockIdx.x / hq : 0;
  const int h = S > 1 ? (int)blockIdx.x % hq : (int)blockIdx.x, b = blockIdx.y;
  const bool lead = part == 0;
  const size_t row = (size_t)b * hq + h;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;

  // The row's group maxima (group g at thread g % NT, slot g / NT) go out
  // before n_b arrives (bounded by the launch's longest row); groups past the
  // row's own length are masked once it is known.
  const int groups_max = (min(max_seq_len, cap) + kGroupTokens - 1) / kGroupTokens;
  uint32_t graw[E1];
  {
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(gmax + row * (size_t)gstride, groups_max * 4);
#pragma unroll
    for (int e = 0; e < E1; ++e)
      graw[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(e * NT + t) * 4u, 0, 0);
  }
  // This lane's query values for FAC (written by TIP for this row).
  const QueryRaw<BF16, D> qraw = load_query<BF16, D>(qrot + row * D);
  // Both histograms and the counters are cleared while the loads fly (the
  // first barrier below orders that before any count).
  {
    uint4* h1 = reinterpret_cast<uint4*>(L.hist1);
    uint4* h2 = reinterpret_cast<uint4*>(L.hist2);
    for (int i = t; i < kSelBins / 4; i += NT) {
      h1[i] = make_uint4(0, 0, 0, 0);
      h2[i] = make_uint4(0, 0, 0, 0);
    }
    if (t == 0) {
      L.pivot_n = 0u;
      L.overflow = 0u;
    }
    for (int i = t; i < kFilterMaxGroups / kFilterThreads * kFilterWaves; i += NT)
      (&L.emit_cnt[0][0])[i] = 0u;
  }
  if constexpr (F::MF) {
    // The scaled query's bf16 halves for the matrix-core logits (read after
    // the barriers every route passes before FAC).
    if (t < 16) {
      const float scale = logit_scale<D>();
      const float qv[8] = {qraw.v[0].x, qraw.v[0].y, qraw.v[0].z, qraw.v[0].w,
                           qraw.v[1].x, qraw.v[1].y, qraw.v[1].z, qraw.v[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = qv[i] * scale;
        const uint32_t hb = f32_to_bf16_bits(x);
        L.qhi[8 * t + i] = (uint16_t)hb;
        L.qlo[8 * t + i] = (uint16_t)f32_to_bf16_bits(x - __uint_as_float(hb << 16));
      }
    }
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

  // This wave's list for FAC: cnt entries at lpos / lkey.
  const int32_t* lpos = &L.pos[wave * kWavePlayCap];
  const uint32_t* lkey = &L.key[wave * kWavePlayCap];
  int cnt = 0;
  uint64_t tau = 0;     // an entry takes part <=> its composite >= tau
  F fac0, fac1;
  int issued = 0;       // FAC rounds whose loads are in flight (0, 1 or 2)
  bool listed = false;  // the waves' own lists hold the row's in-play tokens
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
      for (int e = 0; e < E1; ++e) gk[e] = (e * NT + t < ng) ? graw[e] : 0u;
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
        cold = !p.ok || p.above + p.count > (uint32_t)(NW * kCapW);
      }
      if (!cold) {
        // 2. This wave's surviving groups, ascending (slot-major, then
        // lane), and the smallest surviving maximum of the wave.
        uint32_t ns = 0, kmine = ~0u;
#pragma unroll
        for (int e = 0; e < E1; ++e) {
          const bool in = gk[e] != 0u && bn[e] >= p.bin;
          const uint64_t bal = __ballot(in);
          const uint32_t at = ns + lanes_below_count(bal);
          if (in && at < (uint32_t)kCapW) L.grp[wave][at] = e * NT + t;
          ns += (uint32_t)__popcll(bal);
          kmine = in ? min(kmine, gk[e]) : kmine;
        }
        kmine = wave_min_u32(kmine);
        if (lane == 0) L.kpmin[wave] = kmine;
        bool ovf = ns > (uint32_t)kCapW;
        const uint32_t nsw = ovf ? (uint32_t)kCapW : ns;
        __builtin_amdgcn_wave_barrier();  // the wave reads back its own L.grp
        // Their scores: slab s holds the wave's survivors 16 s .. 16 s + 15,
        // 4 lanes each, so (slab, lane, element) order is position order.
        float4 sv[E2 / 4];
        int p0[E2 / 4];
        {
          const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row_scores, ((n + 3) & ~3) * 4);
#pragma unroll
          for (int s = 0; s < E2 / 4; ++s) {
            const uint32_t li = (uint32_t)(s * kWave + lane) / kGroupLanes;
            const int g = li < nsw ? L.grp[wave][li] : 0;
            p0[s] = li < nsw ? g * kGroupTokens + 4 * (lane % kGroupLanes) : -kGroupTokens;
            const uint32_t at = li < nsw ? (uint32_t)p0[s] * 4u : 0xfffffff0u;  // past: zeros
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, at, 0, 0);
            sv[s] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                __uint_as_float(x[2]), __uint_as_float(x[3]));
          }
        }
        __syncthreads();  // every wave's smallest surviving maximum
        uint32_t kp = ~0u;
#pragma unroll
        for (int w = 0; w < NW; ++w) kp = min(kp, L.kpmin[w]);
        // The wave's tokens >= kp into its list, in position order; their
        // keys counted in 1024 bins of 2^sh2 keys from kp.
        const int sh2 = bin_shift(kmax - kp);
        int32_t* wpos = &L.pos[wave * kWavePlayCap];
        uint32_t* wkey = &L.key[wave * kWavePlayCap];
#pragma unroll
        for (int s = 0; s < E2 / 4; ++s) {
          const float fv[4] = {sv[s].x, sv[s].y, sv[s].z, sv[s].w};
          uint32_t kk[4];
          uint64_t bal[4];
          uint32_t below = 0, tot = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t k0 = score_key(fv[e]);
            const uint32_t k = k0 ? k0 : 1u;
            kk[e] = (p0[s] >= 0 && p0[s] + e < n && k >= kp) ? k : 0u;
            bal[e] = __ballot(kk[e] != 0u);
            below += lanes_below_count(bal[e]);  // this slab's entries of lower lanes
            tot += (uint32_t)__popcll(bal[e]);
          }
          // (slab, lane, element) order: lower lanes first, then this lane's
          // elements in order.
          uint32_t at = (uint32_t)cnt + below;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kk[e]) {
              if (at < (uint32_t)kWavePlayCap) {
                wpos[at] = p0[s] + e;
                wkey[at] = kk[e];
              }
              ++at;
            }
          cnt += (int)tot;
        }
        ovf = ovf || cnt > kWavePlayCap;
        if (ovf && lane == 0) L.overflow = 1u;
        // 3. The rows FAC will read go out now; then the list's keys are
        // counted (one atomic per listed token).
        __builtin_amdgcn_wave_barrier();  // the wave reads back its own list
        // A list longer than the two rounds in flight makes FAC lay T_t out
        // flat and re-deal it (below), so its rows would be issued for nothing.
        if (!ovf && cnt > 0 && cnt <= 2 * F::RR) {
          fac_issue<true>(fac0, 0, cnt, wpos, K, V, kvbase, part);
          issued = 1;
          if (cnt > F::RR) {
            fac_issue<true>(fac1, F::RR, cnt, wpos, K, V, kvbase, part);
            issued = 2;
          }
        }
        const int listed_n = min(cnt, kWavePlayCap);
        for (int i = lane; i < listed_n; i += kWave)
          atomicAdd(&L.hist2[(wkey[i] - kp) >> sh2], 1u);
        if (lane == 0) L.wcnt[wave] = cnt;
        __syncthreads();  // the histogram, the overflow flag and the list lengths are complete
        cold = L.overflow != 0u;
        if (!cold) {
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
              for (int i = lane; i < cnt; i += kWave) {
                const uint32_t k = wkey[i];
                if (k >= blo && k <= bhi) {
                  const uint32_t at = atomicAdd(&L.pivot_n, 1u);
                  if (at < (uint32_t)kPivotCap) L.pivot[at] = composite(k, (uint32_t)wpos[i]);
                }
              }
              __syncthreads();
              const uint32_t M = L.pivot_n;
              if (M > (uint32_t)kPivotCap) cold = true;
              else tau = wave_rank(L.pivot, M, need);
            }
          }
        }
        listed = !cold;
      }
    }
    if (cold) {
      // 5. Streaming passes over all of the row's composites; T_t lies flat
      // over L.pos.
      __syncthreads();  // LDS of the steps above is reused
      const uint64_t ts =
          stream_select(row_scores, n, (uint32_t)bh, 1ull << 32, ~0ull, L.s, err);
      stream_emit(row_scores, n, ts, (uint32_t)bh, L.s, [&](uint32_t r, int pos) {
        if (o) o[r] = pos;
        L.pos[r] = pos;
        L.key[r] = 1u;
      });
      tau = 0;
      issued = 0;
    }
    if (o != nullptr)
      for (int j = bh + t; j < budget; j += NT) o[j] = -1;
  }
  float* out_row = out + row * D;
  if (take == 0) {
    if (lead)
      for (int d = t; d < D; d += NT) out_row[d] = 0.0f;
    return;
  }
  if (!listed) {
    // A whole or streamed T_t: wave w takes the w-th share of the flat list.
    __syncthreads();
    const int share = (take + NW - 1) / NW;
    const int lo = wave * share;
    cnt = max(0, min(take - lo, share));
    lpos = &L.pos[lo];
    lkey = &L.key[lo];
  }
  // FAC reads fcnt entries at fpos / fkey (selected <=> composite >= ftau).
  int fcnt = cnt;
  const int32_t* fpos = lpos;
  const uint32_t* fkey = lkey;
  uint64_t ftau = tau;
  if (listed) {
    int maxcnt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) maxcnt = max(maxcnt, L.wcnt[w]);
    if (maxcnt > 2 * F::RR) {
      // Some wave's list runs past the two rounds in flight (clustered
      // tokens land in few waves): T_t is laid out flat, the waves' selected
      // entries one after another, and each wave attends an even share.
      uint32_t mine = 0;
      for (int i0 = 0; i0 < cnt; i0 += kWave) {
        const int i = i0 + lane;
        mine += (uint32_t)__popcll(
            __ballot(i < cnt && composite(lkey[i], (uint32_t)lpos[i]) >= tau));
      }
      if (lane == 0) L.selcnt[wave] = mine;
      __syncthreads();
      uint32_t base = 0, total = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        base += w < wave ? L.selcnt[w] : 0u;
        total += L.selcnt[w];
      }
      int32_t* flat = &L.emit[0][0];
      for (int i0 = 0; i0 < cnt; i0 += kWave) {
        const int i = i0 + lane;
        const bool sel = i < cnt && composite(lkey[i], (uint32_t)lpos[i]) >= tau;
        const uint64_t bal = __ballot(sel);
        if (sel) flat[base + lanes_below_count(bal)] = lpos[i];
        base += (uint32_t)__popcll(bal);
      }
      __syncthreads();
      const int share = ((int)total + NW - 1) / NW;
      const int lo = wave * share;
      fcnt = max(0, min((int)total - lo, share));
      fpos = flat + lo;
      fkey = reinterpret_cast<const uint32_t*>(fpos);  // with ftau = 0 every entry is in
      ftau = 0;
      issued = 0;
    }
  }
  // 4. FAC.
  fac_wave<BF16, D, S>(fac0, fac1, issued, fcnt, fpos, fkey, ftau, K, V, kvbase, part, qraw, L);
  __syncthreads();
  fac_merge<BF16, D, S>(out_row, part, L);

  if (listed && o != nullptr) {
    // idx in position order.  Block k of 512 groups (8192 positions) holds,
    // for wave w, the 1024 positions 8192 k + 1024 w ..: so T_t in position
    // order is by (block, wave, position), and each wave's sorted list holds
    // its blocks' entries one after another.  Count the selected entries per
    // (block, wave), take first ranks from the counts, and rank each entry
    // by its place among its wave's selected ones.
    constexpr int NB = kFilterMaxGroups / kFilterThreads;
    constexpr int kBlockPos = kFilterThreads * kGroupTokens;
    constexpr int kWavePos = kWave * kGroupTokens;
    uint32_t mine = 0;
    for (int i0 = 0; i0 < cnt; i0 += kWave) {
      const int i = i0 + lane;
      const bool sel = i < cnt && composite(lkey[i], (uint32_t)lpos[i]) >= tau;
      const uint64_t bal = __ballot(sel);
      if (sel) {
        L.emit[wave][mine + lanes_below_count(bal)] = lpos[i];
        atomicAdd(&L.emit_cnt[lpos[i] / kBlockPos][wave], 1u);
      }
      mine += (uint32_t)__popcll(bal);
    }
    __syncthreads();
    {
      // This wave's first rank in block k (lane k): the entries of earlier
      // blocks not its own, plus those of lower waves in block k.
      uint32_t x = 0, below = 0;
      if (lane < NB) {
        const uint4* c4 = reinterpret_cast<const uint4*>(L.emit_cnt[lane]);
        const uint4 a = c4[0], c = c4[1];
        const uint32_t cw[kFilterWaves] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        uint32_t tot = 0, own = 0;
#pragma unroll
        for (int w = 0; w < kFilterWaves; ++w) {
          tot += cw[w];
          own = w == wave ? cw[w] : own;
          below += w < wave ? cw[w] : 0u;
        }
        x = tot - own;
      }
      const uint32_t incl = wave_scan_incl(x);
      if (lane < NB) L.emit_base[lane][wave] = incl - x + below;
    }
    __builtin_amdgcn_wave_barrier();  // the wave reads back its own bases
    for (uint32_t i = lane; i < mine; i += kWave) {
      const int32_t v = L.emit[wave][i];
      const uint32_t r = L.emit_base[v / kBlockPos][wave] + i;
      if (r < (uint32_t)bh) o[r] = v;
    }
    static_assert(kBlockPos == kFilterWaves * kWavePos && NB <= kWave && kFilterWaves == 8,
                  "blocks of the waves' runs");
  }
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

// Survivors are about B groups, about B / 8 per wave; the slots leave room for
// those in bin P and for uneven waves.
int filter_survivor_slots(int budget) { return budget <= 320 ? 16 : 40; }

// Column parts of the fused FAC when the rows are few (as in select2.hip).
constexpr int kFilterColumnParts = 8;

template <bool BF16, int D, int E1, int E2>
static void launch_filter_t(const fasa_ctx* c, hipStream_t s, const uint32_t* gm,
                            const float* scores, const int32_t* nb, int max_seq_len, int budget,
                            const int32_t* hb, int32_t* idx, const void* k, const void* v,
                            const float* qrot, float* out, int32_t* advance, uint32_t* err,
                            bool whole_rows) {
  const bool split = !whole_rows && (long long)c->batch * c->hq * kFilterColumnParts <= c->cus;
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
                            const float* qrot, float* out, int32_t* advance, uint32_t* err,
                            bool whole_rows) {
#define FASA_FILTER(E1V, E2V)                                                                 \
  launch_filter_t<BF16, D, E1V, E2V>(c, s, gm, scores, nb, max_seq_len, budget, hb, idx, k, v, \
                                     qrot, out, advance, err, whole_rows)
  const bool short_rows = filter_group_slots(max_seq_len) == 4;
  const bool few = filter_survivor_slots(budget) == 16;
  if (short_rows) {
    if (few) FASA_FILTER(4, 16); else FASA_FILTER(4, 40);
  } else {
    if (few) FASA_FILTER(20, 16); else FASA_FILTER(20, 40);
  }
#undef FASA_FILTER
}

hipError_t launch_filter_select(const fasa_ctx* c, const float* scores, const int32_t* nb,
                                int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                                const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                                hipStream_t s, const int32_t* head_budget, bool whole_rows) {
  if (!filter_path_applies(max_seq_len, budget) || out == nullptr) return hipErrorInvalidValue;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  const uint32_t* gm = reinterpret_cast<const uint32_t*>(ws + c->ws.gmax);
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf)
      launch_filter_d<true, 128>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                 k_cache, v_cache, qrot, out, advance, err, whole_rows);
    else
      launch_filter_d<false, 128>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                  k_cache, v_cache, qrot, out, advance, err, whole_rows);
  } else {
    if (bf)
      launch_filter_d<true, 64>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                k_cache, v_cache, qrot, out, advance, err, whole_rows);
    else
      launch_filter_d<false, 64>(c, s, gm, scores, nb, max_seq_len, budget, head_budget, idx,
                                 k_cache, v_cache, qrot, out, advance, err, whole_rows);
  }
  return hipGetLastError();
}

}  // namespace fasa
