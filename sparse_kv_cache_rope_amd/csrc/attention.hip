// FAC (sparse attention over the selected rows) and the dense full-KV decode
// comparator, both split-K with an online-softmax merge.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC second and third bullets: full attention is executed only
// over the selected tokens, whose keys keep their original absolute
// positions (the cache already holds them rotated).  The dense kernel is the
// full-KV baseline the pages compare against (same page, section 4).
//
// Row layout: a K or V row is d * sizeof(dtype) bytes (256 B for bf16 d=128);
// LPR = row_bytes / 16 lanes each load 16 bytes of it, so a wave holds
// RS = 64 / LPR rows at once.  A lane owns EPL = 16 / sizeof(dtype) dims of
// q~ (pre-scaled by 1/sqrt(d)) and of the output accumulator.  Dot products
// are summed across the LPR lanes of a row with DPP, each lane keeps a running
// (max, sum, acc) over the rows it saw, and those are merged across row
// slots, waves and then splits.  The selection is per query head, so a
// workgroup's rows form a gather, not a dense tile: this stays on VALU and is
// bound by the bytes moved, not by MFMA.

#include <math.h>

#include "device_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

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

// Online-softmax state of one lane.
template <int EPL>
struct Soft {
  float m, l, a[EPL];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = 0.0f;
  }
  // Adds one row with logit z (-inf = absent) and values v.
  __device__ __forceinline__ void add(float z, const float (&v)[EPL]) {
    if (z == -INFINITY) return;
    const float mn = fmaxf(m, z);
    const float sc = expf(m - mn);  // m = -inf gives 0
    const float p = expf(z - mn);
    l = l * sc + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = fmaf(p, v[e], a[e] * sc);
    m = mn;
  }
  __device__ __forceinline__ void merge(float m2, float l2, const float (&a2)[EPL]) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float s1 = expf(m - mn), s2 = expf(m2 - mn);
    l = l * s1 + l2 * s2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] = a[e] * s1 + a2[e] * s2;
    m = mn;
  }
  // Merge with the lane `off` away (xor).
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
// NW * (D + 2 * LPR) floats.
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
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float* o = lds + w * (D + 2 * LPR);
      float a2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) a2[e] = o[lane * EPL + e];
      st.merge(o[D + lane], o[D + LPR + lane], a2);
    }
  }
}

// Merges the per-split partials [nsplit][D + 2] (m, l, acc) of one row into
// out[D]; called by one workgroup.
template <int D>
__device__ __forceinline__ void merge_splits(const float* __restrict__ part, int nsplit,
                                             float* __restrict__ out) {
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part[(size_t)s * (D + 2)]);
    float L = 0.0f, A = 0.0f;
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float* p = part + (size_t)s * (D + 2);
        const float w = expf(p[0] - M);
        L = fmaf(p[1], w, L);
        A = fmaf(p[2 + d], w, A);
      }
    }
    out[d] = (L > 0.0f) ? A / L : 0.0f;
  }
}

// ---------------------------------------------------------------- FAC ----

// grid (splits, Hq, b), 256 threads; split s covers idx entries
// [s * kFacSplitRows, ...) of the first min(budget, n_b).
template <bool BF16, int D>
__global__ void __launch_bounds__(256)
fac_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
           const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
           const int32_t* __restrict__ idx, int budget, int hq, int hkv, int G, int cap,
           float* __restrict__ partial, int max_splits, uint32_t* __restrict__ tickets,
           float* __restrict__ out, uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = 4;
  constexpr int ITERS = kFacSplitRows / (RS * NW);
  static_assert(ITERS >= 1, "split smaller than one pass");
  __shared__ float lds[NW * (D + 2 * LPR)];
  __shared__ uint32_t flag;

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  const int g = h / G;
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int take = n < budget ? n : budget;
  const int nsplit = (take + kFacSplitRows - 1) / kFacSplitRows;
  float* o = out + row * D;
  if (nsplit == 0) {
    if (split == 0)
      for (int d = threadIdx.x; d < D; d += 256) o[d] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = 1.0f / sqrtf((float)D);
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int32_t* ids = idx + row * budget + (size_t)split * kFacSplitRows;
  const int rows_here = min(kFacSplitRows, take - split * kFacSplitRows);

  int jr[ITERS];
  uint4 kc[ITERS], vc[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * RS * NW + wave * RS + slot;
    int j = (r < rows_here) ? ids[r] : -1;
    if (j >= n) {
      if (sub == 0) raise_flag(err, FASA_DEVFLAG_INDEX);
      j = -1;
    }
    jr[it] = j;
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    if (jr[it] >= 0) {
      const size_t off = (kvbase + jr[it]) * LPR + sub;
      kc[it] = K[off];
      vc[it] = V[off];
    } else {
      kc[it] = make_uint4(0, 0, 0, 0);
      vc[it] = make_uint4(0, 0, 0, 0);
    }
  }
  Soft<EPL> st;
  st.init();
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float kf[EPL], vf[EPL];
    unpack<BF16, EPL>(kc[it], kf);
    float z = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) z = fmaf(qv[e], kf[e], z);
    z = group_sum<LPR>(z);
    unpack<BF16, EPL>(vc[it], vf);
    st.add(jr[it] >= 0 ? z : -INFINITY, vf);
  }
  merge_block<D, LPR, EPL, NW>(st, lds);

  if (nsplit == 1) {
    if (wave == 0 && lane < LPR) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[lane * EPL + e] = (st.l > 0.0f) ? st.a[e] / st.l : 0.0f;
    }
    return;
  }
  float* part = partial + row * max_splits * (D + 2);
  if (wave == 0 && lane < LPR) {
    float* p = part + (size_t)split * (D + 2);
    if (lane == 0) {
      p[0] = st.m;
      p[1] = st.l;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) p[2 + lane * EPL + e] = st.a[e];
  }
  if (!last_block_arrives(&tickets[row * kTicketsPerRow + 2], (uint32_t)nsplit, &flag)) return;
  merge_splits<D>(part, nsplit, o);
}

// -------------------------------------------------------------- dense ----

// grid (splits, Hkv, b), 256 threads; split s covers tokens
// [s * kDenseSplitTokens, ...) for all G query heads of KV head g.
template <bool BF16, int D, int G>
__global__ void __launch_bounds__(256)
dense_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
             const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
             int hq, int hkv, int cap, float* __restrict__ partial, int max_splits,
             uint32_t* __restrict__ tickets, float* __restrict__ out, uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = 4;
  constexpr int ITERS = kDenseSplitTokens / (RS * NW);
  constexpr int BATCH = 4;
  static_assert(ITERS % BATCH == 0, "token split must be a multiple of one batch");
  __shared__ float lds[NW * (D + 2 * LPR)];
  __shared__ uint32_t flag;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int nsplit = (n + kDenseSplitTokens - 1) / kDenseSplitTokens;
  const size_t row0 = (size_t)b * hq + (size_t)g * G;
  if (nsplit == 0) {
    if (split == 0)
      for (int i = threadIdx.x; i < G * D; i += 256) out[row0 * D + i] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = 1.0f / sqrtf((float)D);
  float qv[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = qrot[(row0 + hh) * D + sub * EPL + e] * scale;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int t0 = split * kDenseSplitTokens;

  Soft<EPL> st[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) st[hh].init();
  for (int it0 = 0; it0 < ITERS; it0 += BATCH) {
    uint4 kc[BATCH], vc[BATCH];
    bool ok[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int j = t0 + (it0 + i) * RS * NW + wave * RS + slot;
      ok[i] = j < n;
      const size_t off = (kvbase + (ok[i] ? j : 0)) * LPR + sub;
      kc[i] = K[off];
      vc[i] = V[off];
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      float kf[EPL], vf[EPL];
      unpack<BF16, EPL>(kc[i], kf);
      unpack<BF16, EPL>(vc[i], vf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float z = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) z = fmaf(qv[hh][e], kf[e], z);
        z = group_sum<LPR>(z);
        st[hh].add(ok[i] ? z : -INFINITY, vf);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    merge_block<D, LPR, EPL, NW>(st[hh], lds);
    if (wave == 0 && lane < LPR) {
      if (nsplit == 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          out[(row0 + hh) * D + lane * EPL + e] = (st[hh].l > 0.0f) ? st[hh].a[e] / st[hh].l : 0.0f;
      } else {
        float* p = partial + ((row0 + hh) * max_splits + split) * (D + 2);
        if (lane == 0) {
          p[0] = st[hh].m;
          p[1] = st[hh].l;
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) p[2 + lane * EPL + e] = st[hh].a[e];
      }
    }
    __syncthreads();
  }
  if (nsplit == 1) return;
  if (!last_block_arrives(&tickets[((size_t)b * hkv + g) * kTicketsPerRow + 3], (uint32_t)nsplit,
                          &flag))
    return;
#pragma unroll 1
  for (int hh = 0; hh < G; ++hh)
    merge_splits<D>(partial + (row0 + hh) * max_splits * (D + 2), nsplit, out + (row0 + hh) * D);
}

// ------------------------------------------------------------ launchers --

hipError_t launch_fac(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                      const int32_t* nb, int max_seq_len, const int32_t* idx, int budget,
                      float* out, uint8_t* ws, hipStream_t s) {
  int take = budget < max_seq_len ? budget : max_seq_len;
  int splits = (take + kFacSplitRows - 1) / kFacSplitRows;
  if (splits < 1) splits = 1;
  dim3 grid((unsigned)splits, (unsigned)c->hq, (unsigned)c->batch);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.fac);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws + c->ws.ticket);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
#define FASA_FAC(BF, DD)                                                                     \
  hipLaunchKernelGGL((fac_kernel<BF, DD>), grid, dim3(256), 0, s, k_cache, v_cache, qrot, nb, \
                     max_seq_len, idx, budget, c->hq, c->hkv, c->G, c->cap, part,             \
                     c->ws.fac_splits, tickets, out, err)
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) FASA_FAC(true, 128); else FASA_FAC(false, 128);
  } else {
    if (bf) FASA_FAC(true, 64); else FASA_FAC(false, 64);
  }
#undef FASA_FAC
  return hipGetLastError();
}

template <bool BF, int DD>
static void launch_dense_g(const fasa_ctx* c, dim3 grid, hipStream_t s, const void* k_cache,
                           const void* v_cache, const float* qrot, const int32_t* nb,
                           int max_seq_len, float* part, uint32_t* tickets, float* out,
                           uint32_t* err) {
#define FASA_DENSE(GG)                                                                         \
  hipLaunchKernelGGL((dense_kernel<BF, DD, GG>), grid, dim3(256), 0, s, k_cache, v_cache, qrot, \
                     nb, max_seq_len, c->hq, c->hkv, c->cap, part, c->ws.dense_splits, tickets, \
                     out, err)
  switch (c->G) {
    case 1: FASA_DENSE(1); break;
    case 2: FASA_DENSE(2); break;
    case 4: FASA_DENSE(4); break;
    default: FASA_DENSE(8); break;
  }
#undef FASA_DENSE
}

hipError_t launch_dense(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                        const int32_t* nb, int max_seq_len, float* out, uint8_t* ws,
                        hipStream_t s) {
  int splits = (max_seq_len + kDenseSplitTokens - 1) / kDenseSplitTokens;
  if (splits < 1) splits = 1;
  dim3 grid((unsigned)splits, (unsigned)c->hkv, (unsigned)c->batch);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.dense);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws + c->ws.ticket);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_dense_g<true, 128>(c, grid, s, k_cache, v_cache, qrot, nb, max_seq_len, part, tickets, out, err);
    else launch_dense_g<false, 128>(c, grid, s, k_cache, v_cache, qrot, nb, max_seq_len, part, tickets, out, err);
  } else {
    if (bf) launch_dense_g<true, 64>(c, grid, s, k_cache, v_cache, qrot, nb, max_seq_len, part, tickets, out, err);
    else launch_dense_g<false, 64>(c, grid, s, k_cache, v_cache, qrot, nb, max_seq_len, part, tickets, out, err);
  }
  return hipGetLastError();
}

}  // namespace fasa
