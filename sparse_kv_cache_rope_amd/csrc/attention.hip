// FAC (sparse attention over the selected rows) and the dense full-KV decode
// comparator, both split-K with an online-softmax merge.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC second and third bullets: full attention is executed only
// over the selected tokens, whose keys keep their original absolute
// positions (the cache already holds them rotated).  The dense kernel is the
// full-KV baseline the pages compare against (same page, section 4).
//
// Rows are gathered 16 bytes per lane (attention_common.hpp).  A head whose
// work spans several workgroups writes
// per-split partials that a separate small kernel merges: no workgroup waits
// on another.  Selection is per query head, so a workgroup's rows form a
// gather, not a dense tile: this stays on VALU and is bound by bytes moved.

#include "attention_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

// ---------------------------------------------------------------- FAC ----

// One workgroup per (b, query head h, split); split s covers idx entries
// [s * kFacSplitRows, ...) of the first min(budget, n_b).
//
// The grid is 1-D.  Workgroups are dealt to the 8 XCDs by linear id mod 8 and
// each XCD has its own L2.  The G query heads of one KV group gather, at the
// same split, rows from the same stretch of positions (each head's indices are
// ascending), and some of the same rows.  So the tuple t = (b, g, split) and
// its G heads take the ids ((t / 8) * G + h % G) * 8 + t % 8: one XCD, back to
// back in dispatch order.  Ids whose t is past the last tuple exit.
template <bool BF16, int D>
__global__ void __launch_bounds__(kFacThreads)
fac_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
           const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
           const int32_t* __restrict__ idx, int budget, int splits, int batch, int hq, int hkv,
           int G, int cap, float* __restrict__ partial, int max_splits, float* __restrict__ out,
           uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = kFacThreads / kWave;
  constexpr int ITERS = kFacSplitRows / (RS * NW);
  static_assert(ITERS >= 1 && ITERS * RS * NW == kFacSplitRows, "split geometry");
  __shared__ float lds[NW * (D + 2 * LPR)];

  const int id = blockIdx.x, round = id >> 3;
  const int t = (round / G) * 8 + (id & 7);
  if (t >= splits * hkv * batch) return;
  const int split = t % splits, g = (t / splits) % hkv, b = t / (splits * hkv);
  const int h = g * G + round % G;
  const size_t row = (size_t)b * hq + h;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;

  // The split's indices and the query are loaded before n_b is known (an idx
  // row is `budget` wide whatever n_b is), so their round trip overlaps the
  // length's instead of following it.
  const int32_t* ids = idx + row * budget + (size_t)split * kFacSplitRows;
  const int in_row = min(kFacSplitRows, budget - split * kFacSplitRows);
  int jr[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * RS * NW + wave * RS + slot;
    jr[it] = (r < in_row) ? ids[r] : -1;
  }
  const float scale = logit_scale<D>();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;

  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int take = n < budget ? n : budget;
  const int nsplit = (take + kFacSplitRows - 1) / kFacSplitRows;
  float* o = out + row * D;
  if (nsplit == 0) {
    if (split == 0)
      for (int d = threadIdx.x; d < D; d += kFacThreads) o[d] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int rows_here = min(kFacSplitRows, take - split * kFacSplitRows);

  uint4 kc[ITERS], vc[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * RS * NW + wave * RS + slot;
    int j = (r < rows_here) ? jr[it] : -1;
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
  float z[ITERS], vf[ITERS][EPL];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float kf[EPL];
    unpack<BF16, EPL>(kc[it], kf);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[e], s);
    s = group_sum<LPR>(s);
    z[it] = jr[it] >= 0 ? s : -INFINITY;
    unpack<BF16, EPL>(vc[it], vf[it]);
  }
  st.template add_batch<ITERS>(z, vf);
  merge_block<D, LPR, EPL, NW>(st, lds);
  write_state<D, LPR, EPL>(st, nsplit == 1, o,
                           partial + (row * max_splits + split) * (D + 2));
}

// -------------------------------------------------------------- dense ----

constexpr int kDenseThreads = 512;
// Query heads a dense workgroup holds softmax states for.
constexpr int kDenseHeads = 2;

// One workgroup per (b, KV head g, split, group of HPW of g's query heads);
// split s covers tokens [s * kDenseSplitTokens, ...).  Fewer heads per
// workgroup than G keep the per-lane softmax states few enough for two
// workgroups per CU; the NG = G / HPW workgroups of one (b, g, split) read
// the same K/V rows, so they take ids on one XCD back to back (the FAC
// kernel's order: ((t / 8) * NG + head group) * 8 + t % 8 for tuple t) and
// all but the first find the rows in that XCD's L2.
template <bool BF16, int D, int HPW>
__global__ void __launch_bounds__(kDenseThreads)
dense_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
             const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
             int hq, int hkv, int cap, int splits, int batch, int groups,
             float* __restrict__ partial, int max_splits, float* __restrict__ out,
             uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = kDenseThreads / kWave;
  constexpr int ITERS = kDenseSplitTokens / (RS * NW);
  constexpr int BATCH = 4;
  static_assert(ITERS % BATCH == 0 && ITERS * RS * NW == kDenseSplitTokens, "split geometry");
  __shared__ float lds[NW * (D + 2 * LPR)];

  const int id = blockIdx.x, round = id >> 3;
  const int tt = (round / groups) * 8 + (id & 7);
  if (tt >= splits * hkv * batch) return;
  const int split = tt % splits, g = (tt / splits) % hkv, b = tt / (splits * hkv);
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int nsplit = (n + kDenseSplitTokens - 1) / kDenseSplitTokens;
  const size_t row0 = (size_t)b * hq + (size_t)g * (HPW * groups) + (size_t)(round % groups) * HPW;
  if (nsplit == 0) {
    if (split == 0)
      for (int i = threadIdx.x; i < HPW * D; i += kDenseThreads) out[row0 * D + i] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = logit_scale<D>();
  float qv[HPW][EPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = qrot[(row0 + hh) * D + sub * EPL + e] * scale;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int t0 = split * kDenseSplitTokens;

  Soft<EPL> st[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) st[hh].init();
  // Batches of BATCH rows per row slot, double-buffered: the next batch's
  // loads are issued before the current batch is used, so every workgroup
  // keeps loads in flight while it computes.  Rows past n read row 0 and are
  // masked.
  auto load = [&](int i0, uint4 (&kc)[BATCH], uint4 (&vc)[BATCH]) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int j = t0 + (i0 + i) * RS * NW + wave * RS + slot;
      const size_t off = (kvbase + (j < n ? j : 0)) * LPR + sub;
      kc[i] = K[off];
      vc[i] = V[off];
    }
  };
  uint4 kb[2][BATCH], vb[2][BATCH];
  load(0, kb[0], vb[0]);
#pragma unroll
  for (int i0 = 0; i0 < ITERS; i0 += BATCH) {
    const int cur = (i0 / BATCH) & 1;
    if (i0 + BATCH < ITERS) load(i0 + BATCH, kb[cur ^ 1], vb[cur ^ 1]);
    float z[HPW][BATCH], vf[BATCH][EPL];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const bool ok = t0 + (i0 + i) * RS * NW + wave * RS + slot < n;
      float kf[EPL];
      unpack<BF16, EPL>(kb[cur][i], kf);
      unpack<BF16, EPL>(vb[cur][i], vf[i]);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[hh][e], kf[e], s);
        s = group_sum<LPR>(s);
        z[hh][i] = ok ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) st[hh].template add_batch<BATCH>(z[hh], vf);
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    merge_block<D, LPR, EPL, NW>(st[hh], lds);
    write_state<D, LPR, EPL>(st[hh], nsplit == 1, out + (row0 + hh) * D,
                             partial + ((row0 + hh) * max_splits + split) * (D + 2));
  }
}

// -------------------------------------------------------------- merge ----

// One 1024-thread workgroup per (h, b) combines the per-split partials
// (m, l, acc) of a row whose work spanned more than one split.  `unit` is the
// rows (FAC: of min(budget, n)) or tokens (dense: of n) per split.  Every
// split's partial is loaded at once (thread = split x 16 dims) and summed
// through LDS, so the merge costs one memory round trip per 1024/(D/16)
// splits instead of one per split.
constexpr int kMergeThreads = 1024;

template <int D>
__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ partial, int max_splits, const int32_t* __restrict__ nb,
             int max_seq_len, int cap, int budget, int unit, int hq, float* __restrict__ out) {
  constexpr int DPT = 16;                      // dims per thread
  constexpr int TPS = D / DPT;                 // threads per split
  constexpr int SPB = kMergeThreads / TPS;     // splits per pass
  __shared__ float red[SPB][D + 1];
  __shared__ float lred[SPB];
  __shared__ float wmax[kMergeThreads / kWave];
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * hq + h;
  int n = nb[b];
  if (n < 0 || n > max_seq_len || n > cap) n = 0;
  const int work = (budget > 0 && budget < n) ? budget : n;
  const int nsplit = (work + unit - 1) / unit;
  if (nsplit <= 1) return;  // written directly by the split kernel
  const float* p = partial + row * max_splits * (D + 2);
  const int t = threadIdx.x;

  float m = -INFINITY;
  for (int s = t; s < nsplit; s += kMergeThreads) m = fmaxf(m, p[(size_t)s * (D + 2)]);
  m = wave_max(m);
  if ((t & (kWave - 1)) == 0) wmax[t / kWave] = m;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeThreads / kWave; ++w) M = fmaxf(M, wmax[w]);

  float A = 0.0f, L = 0.0f;
  const int sl = t / TPS, dd = (t % TPS) * DPT;
  for (int c0 = 0; c0 < nsplit; c0 += SPB) {
    const int s = c0 + sl;
    float v[DPT];
    float l = 0.0f;
    if (s < nsplit && M != -INFINITY) {
      const float* q = p + (size_t)s * (D + 2);
      const float w = exp2f(q[0] - M);
      l = q[1] * w;
#pragma unroll
      for (int i = 0; i < DPT; ++i) v[i] = q[2 + dd + i] * w;
    } else {
#pragma unroll
      for (int i = 0; i < DPT; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) red[sl][dd + i] = v[i];
    if (dd == 0) lred[sl] = l;
    __syncthreads();
    if (t < D) {
      const int lim = min(SPB, nsplit - c0);
      for (int r = 0; r < lim; ++r) {
        A += red[r][t];
        L += lred[r];
      }
    }
    __syncthreads();
  }
  if (t < D) out[row * D + t] = (L > 0.0f) ? A / L : 0.0f;
}

// ------------------------------------------------------------ launchers --

static void launch_merge(const fasa_ctx* c, const float* part, int max_splits, const int32_t* nb,
                         int max_seq_len, int budget, int unit, float* out, hipStream_t s) {
  dim3 grid((unsigned)c->hq, (unsigned)c->batch);
  if (c->d == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, s, part, max_splits, nb,
                       max_seq_len, c->cap, budget, unit, c->hq, out);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, s, part, max_splits, nb,
                       max_seq_len, c->cap, budget, unit, c->hq, out);
}

hipError_t launch_fac(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                      const int32_t* nb, int max_seq_len, const int32_t* idx, int budget,
                      float* out, uint8_t* ws, hipStream_t s) {
  const int take = budget < max_seq_len ? budget : max_seq_len;
  int splits = (take + kFacSplitRows - 1) / kFacSplitRows;
  if (splits < 1) splits = 1;
  // (b, g, split) tuples rounded up to whole rounds of 8 XCDs, G heads each.
  const long tuples = (long)splits * c->hkv * c->batch;
  const dim3 grid((unsigned)((tuples + 7) / 8 * 8 * c->G));
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.fac);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
#define FASA_FAC(BF, DD)                                                                      \
  hipLaunchKernelGGL((fac_kernel<BF, DD>), grid, dim3(kFacThreads), 0, s, k_cache, v_cache, qrot, \
                     nb, max_seq_len, idx, budget, splits, c->batch, c->hq, c->hkv, c->G,      \
                     c->cap, part, c->ws.fac_splits, out, err)
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) FASA_FAC(true, 128); else FASA_FAC(false, 128);
  } else {
    if (bf) FASA_FAC(true, 64); else FASA_FAC(false, 64);
  }
#undef FASA_FAC
  if (splits > 1)
    launch_merge(c, part, c->ws.fac_splits, nb, max_seq_len, budget, kFacSplitRows, out, s);
  return hipGetLastError();
}

template <bool BF, int DD>
static bool launch_dense_g(const fasa_ctx* c, int splits, hipStream_t s, const void* k_cache,
                           const void* v_cache, const float* qrot, const int32_t* nb,
                           int max_seq_len, float* part, float* out, uint32_t* err) {
  // Query heads per workgroup: at most kDenseHeads.
  const int hpw = c->G < kDenseHeads ? c->G : kDenseHeads;
  const int groups = c->G / hpw;
  const long tuples = (long)splits * c->hkv * c->batch;
  const long ids = (tuples + 7) / 8 * 8 * groups;
  if (ids * kDenseThreads > 0xffffffffL) {
    (void)hipGetLastError();
    return false;
  }
  const dim3 grid((unsigned)ids);
#define FASA_DENSE(GG)                                                                          \
  hipLaunchKernelGGL((dense_kernel<BF, DD, GG>), grid, dim3(kDenseThreads), 0, s, k_cache,       \
                     v_cache, qrot, nb, max_seq_len, c->hq, c->hkv, c->cap, splits, c->batch,    \
                     groups, part, c->ws.dense_splits, out, err)
  if (hpw == 1) FASA_DENSE(1);
  else if (hpw == 2) FASA_DENSE(2);
  else FASA_DENSE(4);
#undef FASA_DENSE
  return true;
}

hipError_t launch_dense(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                        const int32_t* nb, int max_seq_len, float* out, uint8_t* ws,
                        hipStream_t s) {
  int splits = (max_seq_len + kDenseSplitTokens - 1) / kDenseSplitTokens;
  if (splits < 1) splits = 1;
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.dense);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const bool bf = (c->dtype == FASA_BF16);
  bool launched;
  if (c->d == 128) {
    launched = bf ? launch_dense_g<true, 128>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err)
                  : launch_dense_g<false, 128>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err);
  } else {
    launched = bf ? launch_dense_g<true, 64>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err)
                  : launch_dense_g<false, 64>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err);
  }
  // A grid past one 1-D launch (2^32 work items) is refused before launching.
  if (!launched) return hipErrorInvalidConfiguration;
  if (splits > 1)
    launch_merge(c, part, c->ws.dense_splits, nb, max_seq_len, 0, kDenseSplitTokens, out, s);
  return hipGetLastError();
}

}  // namespace fasa
