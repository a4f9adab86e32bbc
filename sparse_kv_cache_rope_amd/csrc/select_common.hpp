// Radix-select building blocks shared by the two-stage top-B kernels.
//
// Order: 64-bit composites, the order-preserving 32-bit key of an fp32 score
// in the high half and the inverted position in the low half (higher score
// first, then lower position).  All composites of a row differ, so the B-th
// largest one, tau, splits the row exactly: selected <=> composite >= tau.
// tau is found digit by digit (11 bits at a time) from LDS histograms; once
// the bin holding the B-th largest is small it is gathered into LDS and the
// remaining digits are resolved there.
//
// With one or two waves per SIMD nothing hides latency, so every step here is
// built to keep dependent LDS round trips and barriers few: wave scans use
// DPP and lane reads instead of LDS shuffles, histogram copies are folded
// while picking the bin (vector LDS reads), gathers take one LDS atomic per
// wave, and the ordered emit needs a single barrier.
#pragma once

#include "device_common.hpp"

namespace fasa {

struct BinPick {
  uint32_t bin, above, count;
};

// Scratch of a register-resident select with NT threads.
template <int NT, int COPIES, int CAP>
struct RegSelectLds {
  static constexpr int kWaves = NT / kWave;
  // Each copy has kWave spare words past the bins: lanes that count nothing
  // add 0 there (one word per lane) instead of hammering one bin address.
  uint32_t hist[COPIES][kHistBins + kWave];
  uint64_t cand[CAP];
  uint32_t wsum[kWaves];
  uint32_t slab_cnt[8][kWaves];
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
  constexpr int kRow4 = (kHistBins + kWave) / 4;
  uint4* h = reinterpret_cast<uint4*>(&L.hist[0][0]);
  for (int i = threadIdx.x; i < copies * kRow4; i += NT)
    if (i % kRow4 < kHistBins / 4) h[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
}

// Sums `copies` histogram copies and finds, scanning from the top bin down,
// the bin where the running count reaches `need` (1 <= need <= total).
// Thread t owns the PER bins of ranks [PER t, PER t + PER), read with vector
// LDS loads.  Two barriers.
template <int NT, int COPIES, int CAP>
__device__ __forceinline__ BinPick fold_and_pick(RegSelectLds<NT, COPIES, CAP>& L, int bins,
                                                 int copies, uint32_t need) {
  constexpr int PER = kHistBins / NT;  // 8, 4 or 2 bins per thread
  static_assert(PER == 2 || PER == 4 || PER == 8, "bins per thread");
  const int t = threadIdx.x;
  const int lo = bins - PER * (t + 1);  // lowest bin index of this thread's ranks
  uint32_t c[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) c[r] = 0u;
  if (lo >= 0) {
    for (int k = 0; k < copies; ++k) {
      if constexpr (PER == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(&L.hist[k][lo]);
        c[1] += v.x;
        c[0] += v.y;
      } else {
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(&L.hist[k][lo + 4 * q]);
          // bin lo + i has rank PER t + PER - 1 - i
          c[PER - 1 - 4 * q] += v.x;
          c[PER - 2 - 4 * q] += v.y;
          c[PER - 3 - 4 * q] += v.z;
          c[PER - 4 - 4 * q] += v.w;
        }
      }
    }
  }
  uint32_t local = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) local += c[r];
  const uint32_t incl = wave_scan_incl(local);
  const int wave = t / kWave;
  if (lane_id() == kWave - 1) L.wsum[wave] = incl;
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

__device__ __forceinline__ bool has_prefix64(uint64_t c, uint64_t prefix, int known) {
  return known == 0 || (c >> (64 - known)) == prefix;
}

// tau = the need-th largest of the valid composites held in registers
// (c[e] valid when bit e of vmask is set); need >= 1 and <= the valid count.
template <int NT, int E, int COPIES, int CAP>
__device__ uint64_t reg_select(const uint64_t (&c)[E], uint32_t vmask, uint32_t need,
                               RegSelectLds<NT, COPIES, CAP>& L) {
  static_assert(E <= 32, "validity mask is 32 bits");
  const int tid = threadIdx.x;
  const int copy = (tid / kWave) % COPIES;
  uint64_t prefix = 0;
  int known = 0;
  bool in_lds = false;
  uint32_t M = 0;
  for (;;) {
    const int width = (64 - known < kHistBits) ? (64 - known) : kHistBits;
    const int shift = 64 - known - width;
    const uint32_t mask = (1u << width) - 1u;
    if (!in_lds) {
      zero_hist(L, COPIES);
      const uint32_t spare = (uint32_t)(kHistBins + lane_id());
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool take = ((vmask >> e) & 1u) && has_prefix64(c[e], prefix, known);
        atomicAdd(&L.hist[copy][take ? ((uint32_t)(c[e] >> shift) & mask) : spare], take ? 1u : 0u);
      }
    } else {
      zero_hist(L, 1);
      for (uint32_t i = tid; i < M; i += NT) {
        const uint64_t v = L.cand[i];
        if (has_prefix64(v, prefix, known)) atomicAdd(&L.hist[0][(uint32_t)(v >> shift) & mask], 1u);
      }
    }
    __syncthreads();
    const BinPick p = fold_and_pick(L, 1 << width, in_lds ? 1 : COPIES, need);
    prefix = (prefix << width) | p.bin;
    known += width;
    need -= p.above;
    if (p.count == need || known == 64) break;  // the whole bin is taken
    if (!in_lds && p.count <= (uint32_t)CAP) {
      // Gather the bin: one LDS atomic per wave reserves the wave's slots.
      uint32_t mine = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        mine += (((vmask >> e) & 1u) && has_prefix64(c[e], prefix, known)) ? 1u : 0u;
      if (tid == 0) L.cand_n = 0;
      __syncthreads();
      const uint32_t incl = wave_scan_incl(mine);
      uint32_t base = 0;
      if (lane_id() == kWave - 1 && incl) base = atomicAdd(&L.cand_n, incl);
      base = (uint32_t)__builtin_amdgcn_readlane((int)base, kWave - 1);
      uint32_t slot = base + incl - mine;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (((vmask >> e) & 1u) && has_prefix64(c[e], prefix, known)) {
          if (slot < (uint32_t)CAP) L.cand[slot] = c[e];
          ++slot;
        }
      __syncthreads();
      M = min(L.cand_n, (uint32_t)CAP);
      in_lds = true;
    }
  }
  return (known >= 64) ? prefix : (prefix << (64 - known));
}

// Output offsets for an ordered compaction over S slabs: element e of slab s
// of thread t has order (s, t, e); sel[s] is the thread's 4-bit mask of
// selected elements in slab s.  off[s] receives the output index of the
// thread's first selected element of slab s; the return value is the total.
// One barrier.
template <int NT, int S, int COPIES, int CAP>
__device__ __forceinline__ uint32_t ordered_offsets(const uint32_t (&sel)[S], uint32_t (&off)[S],
                                                    RegSelectLds<NT, COPIES, CAP>& L) {
  static_assert(S <= 8, "slab table holds 8 slabs");
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  const uint64_t below = lanes_below();
  uint32_t pre[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint32_t p = 0, tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot((sel[s] >> e) & 1u);
      p += (uint32_t)__popcll(bal & below);
      tot += (uint32_t)__popcll(bal);
    }
    pre[s] = p;
    if (lane_id() == 0) L.slab_cnt[s][wave] = tot;
  }
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t v = L.slab_cnt[s][w];
      before += (w < wave) ? v : 0u;
      all += v;
    }
    off[s] = base + before + pre[s];
    base += all;
  }
  return base;
}

}  // namespace fasa
