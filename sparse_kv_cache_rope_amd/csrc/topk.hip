// Per-head top-B selection of the critical token set T_t, optionally fused
// with FAC over the selected rows.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC bullets: from the TIP scores a critical subset of tokens T_t
// is selected, then full attention runs over T_t only.  Selection here: the
// min(B, n) highest scores of each (sequence, query head) row, equal scores
// going to the lower position, listed ascending.
//
// Exact radix select.  A row's order is that of 64-bit composites (the
// order-preserving 32-bit key of the fp32 score, then the inverted position),
// all distinct, so the B-th largest composite tau splits the row: selected <=>
// composite >= tau.  The hot passes work on the 32-bit keys alone (a shift and
// an LDS atomic per element); positions only enter among the few candidates
// that share the threshold's key bin, or when ties are massive.
//
// One 512-thread workgroup owns a whole row, so no workgroup ever waits on
// another (on a multi-die GPU a device-wide hand-off costs far more than the
// selection).  Keys are read with coalesced 16-byte loads and, for rows up to
// 32768 positions, kept in registers.
//   1. Histogram the top 11 key bits (LDS, 8 copies against atomic
//      contention) and find the bin holding the B-th largest.
//   2. A small bin is gathered into LDS and the select finishes there; a big
//      one is refined with the next 11 key bits (then 10, then positions).
//   3. Selected positions are compacted slab by slab (a scan over per-wave
//      counts) and written in ascending order, to global memory and/or to LDS.
//   4. With FAC fused, the workgroup then gathers the selected K/V rows and
//      computes softmax(q~ K^T / sqrt(d)) V over them (attention_common.hpp).
// Rows with n <= B take every position and are padded with -1.

#include "attention_common.hpp"
#include "budget.hpp"
#include "fasa_internal.hpp"

namespace fasa {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kHistCopies = 8;
constexpr int kCandCap = 4096;
constexpr int kCacheVec = 16;  // float4 slabs per thread kept in registers
constexpr int kCachedRow = kCacheVec * 4 * kSelThreads;
constexpr bool kUseCachedKeys = false;

struct BinPick {
  uint32_t bin, above, count;
};

struct SelectLds {
  uint32_t hist[kHistCopies][kHistBins];  // reused as float scratch by the FAC merge
  uint64_t cand[kCandCap];
  int32_t sel[kFusedMaxBudget];
  uint32_t scan[kSelWaves];
  uint32_t slab_cnt[kSelWaves];
  uint32_t pick[4];
  uint32_t cand_n;
};

// Finds, scanning `hist[bins]` from the top bin down, the bin where the running
// count reaches `need` (1 <= need <= total).  All kSelThreads threads call it.
__device__ __forceinline__ BinPick pick_from_top(const uint32_t* hist, int bins, uint32_t need,
                                                 SelectLds& L) {
  const int per = (bins + kSelThreads - 1) / kSelThreads;
  uint32_t local = 0;
  for (int e = 0; e < per; ++e) {
    const int rank = threadIdx.x * per + e;  // rank 0 = top bin
    if (rank < bins) local += hist[bins - 1 - rank];
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan<kSelThreads>(local, L.scan, &total);
  if (before < need && need <= before + local) {
    uint32_t acc = before;
    for (int e = 0; e < per; ++e) {
      const int rank = threadIdx.x * per + e;
      if (rank >= bins) break;
      const uint32_t c = hist[bins - 1 - rank];
      if (acc < need && need <= acc + c) {
        L.pick[0] = (uint32_t)(bins - 1 - rank);
        L.pick[1] = acc;
        L.pick[2] = c;
      }
      acc += c;
    }
  }
  __syncthreads();
  BinPick p{L.pick[0], L.pick[1], L.pick[2]};
  __syncthreads();
  return p;
}

// The keys of one row.  Thread t owns the float4 slabs v = i * kSelThreads + t
// (positions 4v .. 4v+3), i < nvec; positions >= n read as key 0 and are
// masked by the callers.
template <bool CACHED>
struct RowKeys {
  const float* __restrict__ row;
  int n, nvec;
  uint32_t kk[CACHED ? kCacheVec * 4 : 1];

  __device__ __forceinline__ void load4(int i, uint32_t (&k)[4]) const {
    const int j = 4 * (i * kSelThreads + (int)threadIdx.x);
    if (j + 4 <= n) {
      const float4 x = *reinterpret_cast<const float4*>(row + j);
      k[0] = score_key(x.x);
      k[1] = score_key(x.y);
      k[2] = score_key(x.z);
      k[3] = score_key(x.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k[e] = (j + e < n) ? score_key(row[j + e]) : 0u;
    }
  }

  __device__ __forceinline__ void init(const float* r, int n_) {
    row = r;
    n = n_;
    nvec = (n + 4 * kSelThreads - 1) / (4 * kSelThreads);
    if constexpr (CACHED) {
#pragma unroll
      for (int i = 0; i < kCacheVec; ++i) {
        uint32_t k[4] = {0u, 0u, 0u, 0u};
        if (i < nvec) load4(i, k);
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[4 * i + e] = k[e];
      }
    }
  }

  // fn(k[4], j0) for the slabs i = 0 .. nvec-1 in order; j0 = first position.
  template <typename F>
  __device__ __forceinline__ void slabs(F fn) const {
    if constexpr (CACHED) {
#pragma unroll
      for (int i = 0; i < kCacheVec; ++i) {
        if (i < nvec) {  // constant trip count: kk stays in registers
          const uint32_t k[4] = {kk[4 * i], kk[4 * i + 1], kk[4 * i + 2], kk[4 * i + 3]};
          fn(k, 4 * (i * kSelThreads + (int)threadIdx.x));
        }
      }
    } else {
#pragma unroll 2
      for (int i = 0; i < nvec; ++i) {
        uint32_t k[4];
        load4(i, k);
        fn(k, 4 * (i * kSelThreads + (int)threadIdx.x));
      }
    }
  }
};

__device__ __forceinline__ bool has_prefix64(uint64_t c, uint64_t prefix, int known) {
  return known == 0 || (c >> (64 - known)) == prefix;
}

// Radix select over the M composites in LDS, continuing from (prefix, known,
// need); returns tau.
__device__ uint64_t resolve_in_lds(SelectLds& L, uint32_t M, uint64_t prefix, int known,
                                   uint32_t need) {
  const int tid = threadIdx.x;
  while (known < 64) {
    const int w = (64 - known < kHistBits) ? (64 - known) : kHistBits;
    const int sh = 64 - known - w;
    const int bins = 1 << w;
    for (int i = tid; i < bins; i += kSelThreads) L.hist[0][i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < M; i += kSelThreads) {
      const uint64_t c = L.cand[i];
      if (has_prefix64(c, prefix, known))
        atomicAdd(&L.hist[0][(uint32_t)(c >> sh) & (uint32_t)(bins - 1)], 1u);
    }
    __syncthreads();
    const BinPick q = pick_from_top(L.hist[0], bins, need, L);
    prefix = (prefix << w) | q.bin;
    known += w;
    need -= q.above;
    if (q.count == need) break;
  }
  return (known >= 64) ? prefix : (prefix << (64 - known));
}

// Sums the histogram copies into copy 0.
__device__ __forceinline__ void fold_copies(SelectLds& L, int bins) {
  __syncthreads();
  for (int i = threadIdx.x; i < bins; i += kSelThreads) {
    uint32_t s = 0;
#pragma unroll
    for (int k = 0; k < kHistCopies; ++k) s += L.hist[k][i];
    L.hist[0][i] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ void zero_copies(SelectLds& L) {
  for (int i = threadIdx.x; i < kHistCopies * kHistBins; i += kSelThreads) (&L.hist[0][0])[i] = 0u;
  __syncthreads();
}

// tau for a row with n > budget.
template <bool CACHED>
__device__ uint64_t select_threshold(const RowKeys<CACHED>& rk, int budget, SelectLds& L) {
  const int copy = (threadIdx.x / kWave) % kHistCopies;
  const int n = rk.n;
  uint32_t need = (uint32_t)budget;
  // Key bits: levels of 11, 11 and 10 bits.
  uint32_t kpre = 0;
  int kknown = 0;
  while (kknown < 32) {
    const int width = (32 - kknown < kHistBits) ? (32 - kknown) : kHistBits;
    const int shift = 32 - kknown - width;
    const uint32_t mask = (1u << width) - 1u;
    zero_copies(L);
    rk.slabs([&](const uint32_t (&k)[4], int j0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < n && (kknown == 0 || (k[e] >> (32 - kknown)) == kpre))
          atomicAdd(&L.hist[copy][(k[e] >> shift) & mask], 1u);
    });
    fold_copies(L, 1 << width);
    const BinPick p = pick_from_top(L.hist[0], 1 << width, need, L);
    kpre = (kpre << width) | p.bin;
    kknown += width;
    need -= p.above;
    if (p.count == need) {  // the whole bin is taken
      const uint64_t low = (kknown == 32) ? (uint64_t)kpre : ((uint64_t)kpre << (32 - kknown));
      return low << 32;
    }
    if (p.count <= (uint32_t)kCandCap) {
      // Gather the bin into LDS as composites and finish there.
      if (threadIdx.x == 0) L.cand_n = 0;
      __syncthreads();
      rk.slabs([&](const uint32_t (&k)[4], int j0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < n && (k[e] >> (32 - kknown)) == kpre) {
            const uint32_t slot = atomicAdd(&L.cand_n, 1u);
            if (slot < (uint32_t)kCandCap) L.cand[slot] = composite(k[e], (uint32_t)(j0 + e));
          }
      });
      __syncthreads();
      return resolve_in_lds(L, min(L.cand_n, (uint32_t)kCandCap), kpre, kknown, need);
    }
  }
  // More than kCandCap positions share the threshold key: split them by
  // position bits over the row until the bin fits in LDS.
  uint64_t prefix = kpre;
  int known = 32;
  for (;;) {
    const int width = (64 - known < kHistBits) ? (64 - known) : kHistBits;
    const int shift = 64 - known - width;
    const uint32_t mask = (1u << width) - 1u;
    zero_copies(L);
    rk.slabs([&](const uint32_t (&k)[4], int j0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + e < n && k[e] == kpre) {
          const uint64_t c = composite(k[e], (uint32_t)(j0 + e));
          if (has_prefix64(c, prefix, known))
            atomicAdd(&L.hist[copy][(uint32_t)(c >> shift) & mask], 1u);
        }
    });
    fold_copies(L, 1 << width);
    const BinPick p = pick_from_top(L.hist[0], 1 << width, need, L);
    prefix = (prefix << width) | p.bin;
    known += width;
    need -= p.above;
    if (p.count == need || known == 64) return (known == 64) ? prefix : (prefix << (64 - known));
    if (p.count <= (uint32_t)kCandCap) {
      if (threadIdx.x == 0) L.cand_n = 0;
      __syncthreads();
      rk.slabs([&](const uint32_t (&k)[4], int j0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < n && k[e] == kpre) {
            const uint64_t c = composite(k[e], (uint32_t)(j0 + e));
            if (has_prefix64(c, prefix, known)) {
              const uint32_t slot = atomicAdd(&L.cand_n, 1u);
              if (slot < (uint32_t)kCandCap) L.cand[slot] = c;
            }
          }
      });
      __syncthreads();
      return resolve_in_lds(L, min(L.cand_n, (uint32_t)kCandCap), prefix, known, need);
    }
  }
}

// Compacts the positions with composite >= tau, in ascending order, to
// out[0 .. budget) (if out) and L.sel (if to_lds).  Position order is slab
// major, so each slab's offsets come from a scan over its per-wave counts.
template <bool CACHED>
__device__ void emit_selected(const RowKeys<CACHED>& rk, uint64_t tau, int budget, int32_t* out,
                              bool to_lds, SelectLds& L) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const uint32_t tk = (uint32_t)(tau >> 32);
  const uint32_t tpos = 0xffffffffu - (uint32_t)(tau & 0xffffffffu);  // last position taken at key tk
  const int n = rk.n;
  uint32_t base = 0;
  rk.slabs([&](const uint32_t (&k)[4], int j0) {
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t j = (uint32_t)(j0 + e);
      const bool s = (j0 + e < n) && (k[e] > tk || (k[e] == tk && j <= tpos));
      mine |= (s ? 1u : 0u) << e;
    }
    const uint32_t cnt = __popc(mine);
    const uint32_t inc = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) L.slab_cnt[wave] = inc;
    __syncthreads();
    uint32_t before = base, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t t = L.slab_cnt[w];
      before += (w < wave) ? t : 0u;
      all += t;
    }
    __syncthreads();
    uint32_t pos = before + inc - cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((mine >> e) & 1u) {
        if (pos < (uint32_t)budget) {
          if (out) out[pos] = j0 + e;
          if (to_lds && pos < (uint32_t)kFusedMaxBudget) L.sel[pos] = j0 + e;
        }
        ++pos;
      }
    base += all;
  });
}

// FAC over the rows L.sel[0 .. take) for query head h (see attention_common.hpp).
template <bool BF16, int D>
__device__ void attend_selected(SelectLds& L, int take, const void* __restrict__ k_cache,
                                const void* __restrict__ v_cache, const float* __restrict__ qrot,
                                size_t row, size_t kvbase, float* __restrict__ out_row) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = kSelWaves;
  constexpr int BATCH = 4;
  constexpr int PER_BATCH = BATCH * RS * NW;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = logit_scale<D>();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  Soft<EPL> st;
  st.init();
  for (int r0 = 0; r0 < take; r0 += PER_BATCH) {
    int jr[BATCH];
    uint4 kc[BATCH], vc[BATCH];
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      const int r = r0 + it * RS * NW + wave * RS + slot;
      jr[it] = (r < take) ? L.sel[r] : -1;
      if (jr[it] >= 0) {
        const size_t off = (kvbase + jr[it]) * LPR + sub;
        kc[it] = K[off];
        vc[it] = V[off];
      } else {
        kc[it] = make_uint4(0, 0, 0, 0);
        vc[it] = make_uint4(0, 0, 0, 0);
      }
    }
    float z[BATCH], vf[BATCH][EPL];
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      float kf[EPL];
      unpack<BF16, EPL>(kc[it], kf);
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[e], s);
      s = group_sum<LPR>(s);
      z[it] = jr[it] >= 0 ? s : -INFINITY;
      unpack<BF16, EPL>(vc[it], vf[it]);
    }
    st.template add_batch<BATCH>(z, vf);
  }
  __syncthreads();  // the histogram LDS becomes merge scratch
  merge_block<D, LPR, EPL, NW>(st, reinterpret_cast<float*>(&L.hist[0][0]));
  write_state<D, LPR, EPL>(st, true, out_row, nullptr);
}

template <bool CACHED, bool ATTEND, bool BF16, int D>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb, int max_seq_len,
              int hq, int cap, int budget, const int32_t* __restrict__ head_budget,
              int32_t* __restrict__ idx,
              const void* __restrict__ k_cache, const void* __restrict__ v_cache,
              const float* __restrict__ qrot, int hkv, int G, float* __restrict__ out,
              int32_t* __restrict__ advance, uint32_t* err) {
  __shared__ SelectLds L;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * hq + h;
  const int n = checked_len(nb, b, max_seq_len, cap, err, h == 0 && threadIdx.x == 0);
  if (advance != nullptr && h == 0 && threadIdx.x == 0 && n > 0) advance[b] = n;
  int32_t* o = idx ? idx + row * budget : nullptr;
  const int bh = row_budget(head_budget, h, budget, err, b == 0 && threadIdx.x == 0);
  const int take = n < bh ? n : bh;
  if (n <= bh || bh == 0) {
    for (int j = threadIdx.x; j < budget; j += kSelThreads) {
      if (o) o[j] = (j < take) ? j : -1;
      if (ATTEND && j < kFusedMaxBudget) L.sel[j] = j;
    }
  } else {
    RowKeys<CACHED> rk;
    rk.init(scores + row * cap, n);
    const uint64_t tau = select_threshold<CACHED>(rk, bh, L);
    emit_selected<CACHED>(rk, tau, bh, o, ATTEND, L);
    if (o != nullptr)
      for (int j = bh + threadIdx.x; j < budget; j += kSelThreads) o[j] = -1;
  }
  if constexpr (ATTEND) {
    __syncthreads();
    float* out_row = out + row * D;
    if (take == 0) {
      for (int d = threadIdx.x; d < D; d += kSelThreads) out_row[d] = 0.0f;
      return;
    }
    const size_t kvbase = ((size_t)b * hkv + h / G) * cap;
    attend_selected<BF16, D>(L, take, k_cache, v_cache, qrot, row, kvbase, out_row);
  }
}

hipError_t launch_topk(const fasa_ctx* c, const float* scores, const int32_t* nb,
                       int max_seq_len, int budget, int32_t* idx, int32_t* advance, uint8_t* ws,
                       hipStream_t s, const int32_t* head_budget) {
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  dim3 grid((unsigned)c->hq, (unsigned)c->batch);
  if (kUseCachedKeys && max_seq_len <= kCachedRow)
    hipLaunchKernelGGL((select_kernel<true, false, true, 128>), grid, dim3(kSelThreads), 0, s,
                       scores, nb, max_seq_len, c->hq, c->cap, budget, head_budget, idx, nullptr,
                       nullptr, nullptr, c->hkv, c->G, nullptr, advance, err);
  else
    hipLaunchKernelGGL((select_kernel<false, false, true, 128>), grid, dim3(kSelThreads), 0, s,
                       scores, nb, max_seq_len, c->hq, c->cap, budget, head_budget, idx, nullptr,
                       nullptr, nullptr, c->hkv, c->G, nullptr, advance, err);
  return hipGetLastError();
}

template <bool BF, int DD>
static void launch_sel_att(const fasa_ctx* c, dim3 grid, hipStream_t s, bool cached,
                           const float* scores, const int32_t* nb, int max_seq_len, int budget,
                           const int32_t* hb, int32_t* idx, const void* k, const void* v,
                           const float* qrot, float* out, int32_t* advance, uint32_t* err) {
  if (cached)
    hipLaunchKernelGGL((select_kernel<true, true, BF, DD>), grid, dim3(kSelThreads), 0, s, scores,
                       nb, max_seq_len, c->hq, c->cap, budget, hb, idx, k, v, qrot, c->hkv, c->G,
                       out, advance, err);
  else
    hipLaunchKernelGGL((select_kernel<false, true, BF, DD>), grid, dim3(kSelThreads), 0, s, scores,
                       nb, max_seq_len, c->hq, c->cap, budget, hb, idx, k, v, qrot, c->hkv, c->G,
                       out, advance, err);
}

hipError_t launch_select_attend(const fasa_ctx* c, const float* scores, const int32_t* nb,
                                int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                                const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                                hipStream_t s, const int32_t* head_budget) {
  if (budget > kFusedMaxBudget) return hipErrorInvalidValue;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  dim3 grid((unsigned)c->hq, (unsigned)c->batch);
  const bool cached = kUseCachedKeys && max_seq_len <= kCachedRow;
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_sel_att<true, 128>(c, grid, s, cached, scores, nb, max_seq_len, budget, head_budget, idx, k_cache, v_cache, qrot, out, advance, err);
    else launch_sel_att<false, 128>(c, grid, s, cached, scores, nb, max_seq_len, budget, head_budget, idx, k_cache, v_cache, qrot, out, advance, err);
  } else {
    if (bf) launch_sel_att<true, 64>(c, grid, s, cached, scores, nb, max_seq_len, budget, head_budget, idx, k_cache, v_cache, qrot, out, advance, err);
    else launch_sel_att<false, 64>(c, grid, s, cached, scores, nb, max_seq_len, budget, head_budget, idx, k_cache, v_cache, qrot, out, advance, err);
  }
  return hipGetLastError();
}

}  // namespace fasa
