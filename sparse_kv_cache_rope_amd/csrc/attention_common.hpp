// Attention building blocks shared by the FAC, fused select+FAC and dense
// kernels: row geometry, unpacking, per-lane online softmax and its merges.
//
// Row layout: a K or V row is d * sizeof(dtype) bytes (256 B for bf16 d=128);
// LPR = row_bytes / 16 lanes each load 16 bytes of it, so a wave holds
// RS = 64 / LPR rows at once.  A lane owns EPL = 16 / sizeof(dtype) dims of
// q~ (pre-scaled by log2(e)/sqrt(d), so logits are in log2 units and every
// softmax weight is one exp2) and of the output accumulator.  Dot products
// are summed across the LPR lanes of a row with DPP, each lane keeps a running
// (max, sum, acc) over the rows it saw, and those are merged across row
// slots and waves in LDS.
#pragma once

#include <math.h>

#include "device_common.hpp"

namespace fasa {

// Factor applied to q~: 1/sqrt(d) of the attention scale times log2(e), so
// that exp2 of a logit difference is the softmax weight.
template <int D>
__device__ __forceinline__ float logit_scale() {
  return 1.44269504088896340736f / sqrtf((float)D);
}

template <bool BF16, int D>
struct RowGeom {
  static constexpr int ES = BF16 ? 2 : 4;
  static constexpr int LPR = D * ES / 16;
  static constexpr int EPL = 16 / ES;
  static constexpr int RS = kWave / LPR;
  static_assert(LPR >= 4 && LPR <= 32, "row must span 4..32 lanes");
};

template <bool BF16, int EPL>
__device__ __forceinline__ void unpack(const uint4& x, float (&f)[EPL]) {
  if constexpr (BF16) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z);
    f[3] = __uint_as_float(x.w);
  }
}

// Online-softmax state of one lane (logits in log2 units).
template <int EPL>
struct Soft {
  float m, l, a[EPL];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = 0.0f;
  }
  // Adds R rows with logits z (-inf = absent) and values v: one rescale of the
  // running state per batch, and the rows' weights independent of each other.
  template <int R>
  __device__ __forceinline__ void add_batch(const float (&z)[R], const float (&v)[R][EPL]) {
    float mn = m;
#pragma unroll
    for (int r = 0; r < R; ++r) mn = fmaxf(mn, z[r]);
    if (mn == -INFINITY) return;
    const float sc = exp2f(m - mn);  // m = -inf gives 0
    l *= sc;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] *= sc;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float p = exp2f(z[r] - mn);  // z = -inf gives 0
      l += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] = fmaf(p, v[r][e], a[e]);
    }
    m = mn;
  }
  __device__ __forceinline__ void merge(float m2, float l2, const float (&a2)[EPL]) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float s1 = exp2f(m - mn), s2 = exp2f(m2 - mn);
    l = l * s1 + l2 * s2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = a[e] * s1 + a2[e] * s2;
    m = mn;
  }
  __device__ __forceinline__ void merge_xor(int off) {
    float a2[EPL];
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(a[e], off);
    merge(m2, l2, a2);
  }
};

// Merges the row slots of each wave, then the NW waves through LDS; on return
// wave 0 lanes 0..LPR-1 hold the workgroup's state.  `lds` needs
// NW * (D + 2 * LPR) floats.  Ends with the LDS free for reuse.
template <int D, int LPR, int EPL, int NW>
__device__ __forceinline__ void merge_block(Soft<EPL>& st, float* lds) {
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) st.merge_xor(off);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  float* mine = lds + wave * (D + 2 * LPR);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) mine[lane * EPL + e] = st.a[e];
    mine[D + lane] = st.m;
    mine[D + LPR + lane] = st.l;
  }
  __syncthreads();
  if (wave == 0 && lane < LPR) {
    // All NW states at once (independent LDS reads, one max, NW weights)
    // rather than folding them in one after another.
    float ms[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) ms[w] = lds[w * (D + 2 * LPR) + D + lane];
    float mx = ms[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, ms[w]);
    float l = 0.0f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float* o = lds + w * (D + 2 * LPR);
        const float wt = exp2f(ms[w] - mx);  // m = -inf gives 0
        l = fmaf(o[D + LPR + lane], wt, l);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(o[lane * EPL + e], wt, acc[e]);
      }
    }
    st.m = mx;
    st.l = l;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.a[e] = acc[e];
  }
  __syncthreads();
}

// Wave 0 lanes < LPR write the workgroup's result: the normalised output when
// it is the only split, else the partial (m, l, acc[D]).
template <int D, int LPR, int EPL>
__device__ __forceinline__ void write_state(const Soft<EPL>& st, bool only, float* out_row,
                                            float* part) {
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x >= kWave || lane >= LPR) return;
  if (only) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out_row[lane * EPL + e] = (st.l > 0.0f) ? st.a[e] / st.l : 0.0f;
  } else {
    if (lane == 0) {
      part[0] = st.m;
      part[1] = st.l;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) part[2 + lane * EPL + e] = st.a[e];
  }
}

}  // namespace fasa

namespace fasa {

// Final merge of NS per-lane-group softmax states through LDS in one parallel
// step (no sequential state-by-state merging): every (wave, row slot) state
// is written out, wave 0 forms the global max and the per-state weights, and
// each output dim is a weighted sum over the states.  `scratch` needs
// NS * (D + 3) + 1 + (blockDim.x / D) * D floats.  Writes out_row[0 .. D).
template <int D, int LPR, int EPL, int NS>
__device__ __forceinline__ void merge_states_lds(const Soft<EPL>& st, int state, float* scratch,
                                                 float* __restrict__ out_row) {
  float* A = scratch;          // [NS][D]
  float* Mv = A + NS * D;      // [NS]
  float* Lv = Mv + NS;         // [NS]
  float* W = Lv + NS;          // [NS]
  float* tot = W + NS;         // [1]
  const int lane = threadIdx.x & (kWave - 1);
  const int sub = lane % LPR;
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[state * D + sub * EPL + e] = st.a[e];
  if (sub == 0) {
    Mv[state] = st.m;
    Lv[state] = st.l;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    float m = -INFINITY;
    for (int s = lane; s < NS; s += kWave) m = fmaxf(m, Mv[s]);
    m = wave_max(m);
    float l = 0.0f;
    for (int s = lane; s < NS; s += kWave) {
      const float w = (m == -INFINITY) ? 0.0f : exp2f(Mv[s] - m);
      W[s] = w;
      l = fmaf(Lv[s], w, l);
    }
    l = group_sum<kWave>(l);
    if (lane == 0) tot[0] = l;
  }
  __syncthreads();
  // Each dim's weighted sum over the NS states, split over all threads: part
  // p of dim d covers states p, p + P, ...; the parts meet in LDS.
  const float L = tot[0];
  const int nthreads = blockDim.x;
  const int parts = nthreads >= 2 * D ? nthreads / D : 1;
  float* part_sum = W + NS + 1;  // [parts][D]
  if (threadIdx.x < parts * D) {
    const int d = threadIdx.x % D, p = threadIdx.x / D;
    float acc = 0.0f;
    for (int s = p; s < NS; s += parts) acc = fmaf(A[s * D + d], W[s], acc);
    part_sum[p * D + d] = acc;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += nthreads) {
    float acc = 0.0f;
    for (int p = 0; p < parts; ++p) acc += part_sum[p * D + d];
    out_row[d] = (L > 0.0f) ? acc / L : 0.0f;
  }
}

}  // namespace fasa

namespace fasa {

// FAC of query head `row` over the cache rows sel[0 .. take) (sel in LDS,
// take >= 1), NW waves: softmax(q~ . K[j] / sqrt(d)) weighted sum of V[j].
// `scratch` is LDS for the state merge (NW * RS * (D + 3) + 1 + NW * 64
// floats).
//
// Rows go in batches of PER_BATCH (BATCH per row slot); a 256-row selection
// is one round of loads.  Slots past the selection load row sel[take - 1]
// (fetched by another slot, so no new HBM traffic) and count as absent, so
// every load is issued unconditionally.
template <bool BF16, int D, int NW>
__device__ __forceinline__ void attend_rows(const int32_t* sel, int take, const void* __restrict__ k_cache,
                            const void* __restrict__ v_cache, const float* __restrict__ qrot,
                            size_t row, size_t kvbase, float* __restrict__ out_row,
                            float* scratch) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS;
  // Rows per row slot in a batch: enough that a 256-row selection is one
  // round of loads.
  constexpr int BATCH = (256 / (RS * NW)) < 4 ? 4 : (256 / (RS * NW)) > 8 ? 8 : (256 / (RS * NW));
  constexpr int PER_BATCH = BATCH * RS * NW;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = logit_scale<D>();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int last = sel[take - 1];

  struct Batch {
    int jr[BATCH];
    uint4 kc[BATCH], vc[BATCH];
  };
  auto load = [&](int r0, Batch& x) {
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      const int r = r0 + it * RS * NW + wave * RS + slot;
      const bool in = r < take;
      const int j = in ? sel[r] : last;
      x.jr[it] = in ? j : -1;
      const size_t off = (kvbase + j) * LPR + sub;
      x.kc[it] = K[off];
      x.vc[it] = V[off];
    }
  };
  Soft<EPL> st;
  st.init();
  auto fold = [&](const Batch& x) {
    float z[BATCH], vf[BATCH][EPL];
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      float kf[EPL];
      unpack<BF16, EPL>(x.kc[it], kf);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[e], s);
      s = group_sum<LPR>(s);
      z[it] = x.jr[it] >= 0 ? s : -INFINITY;
      unpack<BF16, EPL>(x.vc[it], vf[it]);
    }
    st.template add_batch<BATCH>(z, vf);
  };
  for (int r0 = 0; r0 < take; r0 += PER_BATCH) {
    Batch a;
    load(r0, a);
    fold(a);
  }
  __syncthreads();  // scratch may alias LDS the caller read above
  merge_states_lds<D, LPR, EPL, NW * RS>(st, wave * RS + slot, scratch, out_row);
}

// FAC of query head `row` over sel[0 .. take) (sel in LDS, take >= 1), split
// by output columns over S workgroups; this one (`part`) writes columns
// [part * D / S, (part + 1) * D / S).  Each of the S workgroups reads every
// selected row's K (it needs every logit) but only its share of V, so there
// are no partial states to merge across workgroups and the per-row work of a
// workgroup drops by about a third at S = 4.
//
// A wave step covers S * RS rows.  For K, LPR lanes hold a row, and lane
// group g (lanes g * LPR ..) scores rows g * S .. g * S + S - 1 in S loads.
// For V, VL = LPR / S lanes hold a row's slice, and lane L takes row L / VL,
// which its own K group scored in load (L % LPR) / VL: the logit is already
// in the lane after the group sum.
template <bool BF16, int D, int NW, int S>
__device__ __forceinline__ void attend_rows_split(const int32_t* sel, int take,
                                                  const void* __restrict__ k_cache,
                                                  const void* __restrict__ v_cache,
                                                  const float* __restrict__ qrot, size_t row,
                                                  size_t kvbase, int part,
                                                  float* __restrict__ out_row, float* scratch) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL;
  static_assert(S > 1 && LPR % S == 0, "V slice lanes");
  constexpr int VL = LPR / S;           // lanes per V slice
  constexpr int RPS = kWave / VL;       // rows per wave step
  constexpr int STEPS = 2;              // steps per round of loads
  constexpr int PER_ROUND = RPS * NW * STEPS;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int kg = lane / LPR, sub = lane % LPR;
  const int vrow = lane / VL, vsub = lane % VL, mine = (lane % LPR) / VL;
  const float scale = logit_scale<D>();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int last = sel[take - 1];
  Soft<EPL> st;
  st.init();
  for (int r0 = 0; r0 < take; r0 += PER_ROUND) {
    uint4 kc[STEPS][S], vc[STEPS];
    int jv[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const int base = r0 + (t * NW + wave) * RPS;
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const int r = base + kg * S + i;
        const int j = r < take ? sel[r] : last;
        kc[t][i] = K[(kvbase + j) * LPR + sub];
      }
      const int rv = base + vrow;
      const bool in = rv < take;
      const int j = in ? sel[rv] : last;
      jv[t] = in ? j : -1;
      vc[t] = V[(kvbase + j) * LPR + part * VL + vsub];
    }
    float z[STEPS], vf[STEPS][EPL];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      float zi = 0.0f;
#pragma unroll
      for (int i = 0; i < S; ++i) {
        float kf[EPL];
        unpack<BF16, EPL>(kc[t][i], kf);
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[e], s);
        s = group_sum<LPR>(s);
        zi = (i == mine) ? s : zi;
      }
      z[t] = jv[t] >= 0 ? zi : -INFINITY;
      unpack<BF16, EPL>(vc[t], vf[t]);
    }
    st.template add_batch<STEPS>(z, vf);
  }
  __syncthreads();  // scratch may alias LDS the caller read above
  merge_block<D / S, VL, EPL, NW>(st, scratch);
  write_state<D / S, VL, EPL>(st, true, out_row + part * (D / S), nullptr);
}

}  // namespace fasa

