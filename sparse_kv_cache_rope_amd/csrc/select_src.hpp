// Register-resident sources for the top-B selects: a row segment's scores or
// a row's candidate composites held in slab layout, the range-limited buffer
// loads that fill them, and the ordered emit of the selected elements.
// Shared by the row selects (select2.hip) and the tile-filter select
// (filter.hip).
#pragma once

#include "select_common.hpp"

namespace fasa {

// Scores of one row segment held in registers: element e of thread t is
// position first + 4 * NT * (e / 4) + (e % 4), first = segment + 4 t
// (coalesced float4 slabs).  Only keys are kept (0 for a position past the
// segment, at least 1 otherwise); positions follow from the indexes.
template <int E, int NT>
struct ScoreSrc {
  uint32_t k[E];
  int first;  // position of element 0 of this thread
  __device__ __forceinline__ int pos(int e) const {
    return first + (e / 4) * 4 * NT + (e & 3);
  }
  __device__ __forceinline__ uint32_t key(int e) const { return k[e]; }
  __device__ __forceinline__ uint32_t low(int e) const { return 0xffffffffu - (uint32_t)pos(e); }
};

// Candidate composites held in registers as their two halves (key 0 where
// there is none); same slab layout as ScoreSrc.
template <int E, int NT>
struct CandSrc {
  uint32_t hi[E], lo[E];
  __device__ __forceinline__ uint32_t key(int e) const { return hi[e]; }
  __device__ __forceinline__ uint32_t low(int e) const { return lo[e]; }
};

// A wave-uniform raw buffer resource over `bytes` bytes from `base`:
// out-of-range lanes of a load read zeros and fetch nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                           kBufferRsrcWord3);
}

// Scores of a row segment as loaded, before the row's length is known.
template <int E>
struct RawScores {
  float4 v[E / 4];
};

// Issues the loads of positions [seg, seg + cn_max) of a row's scores (slab
// layout of ScoreSrc) with range-limited buffer loads: quads past cn_max read
// zeros, so no load waits behind a branch.  Nothing here needs the row's own
// length, so callers issue it before that length arrives.
template <int E, int NT>
__device__ __forceinline__ void issue_scores(RawScores<E>& raw, const float* row_scores, int seg,
                                             int cn_max) {
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row_scores + seg, ((cn_max + 3) & ~3) * 4);
#pragma unroll
  for (int g = 0; g < E / 4; ++g) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(
        rs, (uint32_t)(4 * (g * NT + t)) * 4u, 0, 0);
    raw.v[g] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                           __uint_as_float(x[3]));
  }
}

// Keys of positions [seg, seg + cn) from issued loads (cn <= their cn_max):
// positions past cn get key 0, and keys of real positions are raised to at
// least 1, which only merges the two lowest keys (NaN patterns below every
// number).
template <int E, int NT>
__device__ __forceinline__ void scores_to_keys(ScoreSrc<E, NT>& src, const RawScores<E>& raw,
                                               int seg, int cn) {
  const int t = threadIdx.x;
  src.first = seg + 4 * t;
  const int lim = cn - 4 * t;  // element e is valid when (e / 4) * 4 NT + e % 4 < lim
#pragma unroll
  for (int g = 0; g < E / 4; ++g) {
    const float f[4] = {raw.v[g].x, raw.v[g].y, raw.v[g].z, raw.v[g].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = score_key(f[e]);
      src.k[4 * g + e] = (g * 4 * NT + e < lim) ? (k ? k : 1u) : 0u;
    }
  }
}

// Candidate composites of a row as loaded, before the row's length is known.
template <int E>
struct RawCands {
  ulonglong2 v[E / 2];
};

// Issues the loads of a row's candidate slots (slab layout of CandSrc, 4 per
// thread per slab) with range-limited buffer loads over the row's `stride`
// slots: slots past it read zeros.
template <int E, int NT>
__device__ __forceinline__ void issue_cands(RawCands<E>& raw, const uint64_t* row_cand,
                                            int stride) {
  const int t = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(row_cand, stride * 8);
#pragma unroll
  for (int g = 0; g < E / 4; ++g) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(
          rs, (uint32_t)(4 * (g * NT + t) + 2 * half) * 8u, 0, 0);
      raw.v[2 * g + half] = make_ulonglong2(((uint64_t)x[1] << 32) | x[0],
                                            ((uint64_t)x[3] << 32) | x[2]);
    }
  }
}

// Candidates [0, M) from issued loads; slots past M get key 0.
template <int E, int NT>
__device__ __forceinline__ void cands_to_src(CandSrc<E, NT>& src, const RawCands<E>& raw,
                                             int M) {
  const int t = threadIdx.x;
#pragma unroll
  for (int g = 0; g < E / 4; ++g) {
    const int k0 = 4 * (g * NT + t);
    const uint64_t c[4] = {raw.v[2 * g].x, raw.v[2 * g].y, raw.v[2 * g + 1].x,
                           raw.v[2 * g + 1].y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = k0 + e < M;
      src.hi[4 * g + e] = in ? (uint32_t)(c[e] >> 32) : 0u;
      src.lo[4 * g + e] = in ? (uint32_t)c[e] : 0u;
    }
  }
}

// Selected elements (composite >= tau, tau >= 2^32) in ascending position
// order: calls f(rank, element) for the first `limit` of them.  One barrier.
template <int E, int NT, class Src, class LdsT, class F>
__device__ __forceinline__ void emit_ordered(const Src& src, uint64_t tau, uint32_t limit,
                                             LdsT& L, F f) {
  uint32_t m4[E / 4], off[E / 4];
#pragma unroll
  for (int g = 0; g < E / 4; ++g) {
    m4[g] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) m4[g] |= (is_selected(src, 4 * g + e, tau) ? 1u : 0u) << e;
  }
  ordered_offsets<NT>(m4, off, L);
#pragma unroll
  for (int g = 0; g < E / 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((m4[g] >> e) & 1u) {
        if (off[g] < limit) f(off[g], 4 * g + e);
        ++off[g];
      }
}

}  // namespace fasa
