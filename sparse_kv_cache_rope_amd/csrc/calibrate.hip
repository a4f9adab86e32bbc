// Offline calibration of the dominant FCs: per-FC scores, their top-k and the
// agreement of each FC's top-k with the full head's.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, TIP "Calibracao Offline": I_dom of each head is found once from
// a contextual agreement between the attention scores of a single FC and of
// the full head on a small calibration set.  Agreement here: the overlap of
// the two top-k position sets (the selection rule of the decode path),
// divided by k; the caller averages it over calibration queries and keeps the
// FCs of highest agreement.
//
// Rows of the score matrix, per sequence: row h (C + 1) + c holds FC c's
// scores s_c[j] = q~_c K[j][c] + q~_{c+C} K[j][c+C] of query head h (under
// partial RoPE the FC's dims are fc_lo / fc_hi), row h (C + 1) + C the full
// head's s[j] = sum_c s_c[j] (fp32, c ascending).
// Selection over those rows reuses the decode path's top-B kernels.

#include "device_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

constexpr int kCalTokens = 64;  // tokens per workgroup

// grid (ceil(max_seq_len / 64), Hkv, b), 64 * G threads: thread (hh, t) owns
// token tile0 + t of query head g G + hh.  The K tile is staged in LDS as
// fp32 with rows padded by one word, so a wave reading one column of 64 rows
// touches 64 different banks.
template <bool BF16, int D, int G>
__global__ void __launch_bounds__(kCalTokens * G)
calib_scores_kernel(const void* __restrict__ k_cache, const float* __restrict__ qrot,
                    const int32_t* __restrict__ nb, int max_seq_len, int hq, int hkv, int cap,
                    int R, float* __restrict__ scores, uint32_t* err) {
  constexpr int C = D / 2;
  constexpr int RW = D + 1;  // padded LDS row
  __shared__ float kt[kCalTokens * RW];
  __shared__ float qs[G * D];
  const int tile0 = blockIdx.x * kCalTokens, g = blockIdx.y, b = blockIdx.z;
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  if (tile0 >= n) return;
  const int tid = threadIdx.x;

  for (int i = tid; i < G * D; i += kCalTokens * G)
    qs[i] = qrot[((size_t)b * hq + (size_t)g * G) * D + i];
  // K tile: 64 rows of D elements, read row-major (coalesced).
  const size_t kbase = (((size_t)b * hkv + g) * cap + tile0) * D;
  for (int i = tid; i < kCalTokens * D; i += kCalTokens * G) {
    const int r = i / D, col = i % D;
    float v = 0.0f;
    if (tile0 + r < n) {
      if constexpr (BF16)
        v = bf16_bits_to_f32(static_cast<const uint16_t*>(k_cache)[kbase + i]);
      else
        v = static_cast<const float*>(k_cache)[kbase + i];
    }
    kt[r * RW + col] = v;
  }
  __syncthreads();

  const int t = tid % kCalTokens, hh = tid / kCalTokens;
  const int j = tile0 + t;
  if (j >= n) return;
  const float* q = qs + hh * D;
  const float* k = kt + t * RW;
  float* row = scores + ((size_t)b * hq * (C + 1) + (size_t)(g * G + hh) * (C + 1)) * cap + j;
  float full = 0.0f;
#pragma unroll 8
  for (int c = 0; c < C; ++c) {
    const int lo = fc_lo(c, R), hi = fc_hi(c, R, C);
    const float s = fmaf(q[hi], k[hi], q[lo] * k[lo]);
    row[(size_t)c * cap] = s;
    full += s;
  }
  row[(size_t)C * cap] = full;
}

// grid (Hq, b), C threads: thread c counts the positions FC c's top-k shares
// with the full head's (both lists ascending, -1 padded) and writes
// count / min(k, n_b) to ca[b][h][c].
template <int C>
__global__ void __launch_bounds__(64)
ca_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ nb, int max_seq_len,
          int cap, int hq, int topk, float* __restrict__ ca) {
  extern __shared__ int32_t full[];
  const int h = blockIdx.x, b = blockIdx.y;
  int n = nb[b];
  if (n < 0 || n > max_seq_len || n > cap) n = 0;
  const int take = n < topk ? n : topk;
  const int32_t* base = idx + ((size_t)b * hq * (C + 1) + (size_t)h * (C + 1)) * topk;
  for (int i = threadIdx.x; i < take; i += blockDim.x) full[i] = base[(size_t)C * topk + i];
  __syncthreads();
  const int c = threadIdx.x;
  if (c >= C) return;
  float* o = ca + ((size_t)b * hq + h) * C + c;
  if (take == 0) {
    *o = 0.0f;
    return;
  }
  const int32_t* mine = base + (size_t)c * topk;
  int i = 0, f = 0, count = 0;
  while (i < take && f < take) {
    const int a = mine[i], w = full[f];
    count += (a == w) ? 1 : 0;
    i += (a <= w) ? 1 : 0;
    f += (w <= a) ? 1 : 0;
  }
  *o = (float)count / (float)take;
}

template <bool BF16, int D>
static void launch_scores_d(const fasa_ctx* c, dim3 grid, hipStream_t s, const void* k_cache,
                            const float* qrot, const int32_t* nb, int max_seq_len, float* scores,
                            uint32_t* err) {
#define FASA_CAL(GG)                                                                          \
  hipLaunchKernelGGL((calib_scores_kernel<BF16, D, GG>), grid, dim3(kCalTokens * GG), 0, s,   \
                     k_cache, qrot, nb, max_seq_len, c->hq, c->hkv, c->cap, c->R, scores, err)
  switch (c->G) {
    case 1: FASA_CAL(1); break;
    case 2: FASA_CAL(2); break;
    case 4: FASA_CAL(4); break;
    default: FASA_CAL(8); break;
  }
#undef FASA_CAL
}

CalLayout calib_layout(const fasa_ctx* c, int topk) {
  CalLayout w;
  const size_t rows = (size_t)c->batch * c->hq * (c->C + 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  w.ws.err = take(16);
  w.ws.nb = take(sizeof(int32_t) * c->batch);
  w.ws.qrot = take(sizeof(float) * c->batch * (size_t)c->hq * c->d);
  w.ws.scores = take(sizeof(float) * rows * c->cap);
  w.ws.idx = take(sizeof(int32_t) * rows * (size_t)topk);
  const long long nch = (c->cap + 4095) / 4096;
  const long long all = nch * topk;
  const int need = all < kTwoStageMaxCand ? (int)all : kTwoStageMaxCand;
  w.ws.cand_stride = (need + 3) & ~3;
  w.ws.cand = take(sizeof(uint64_t) * rows * w.ws.cand_stride);
  w.ws.total = off;
  return w;
}

hipError_t launch_calibrate(const fasa_ctx* c, const void* k_cache, const void* q,
                            const int32_t* seq_lens, int max_seq_len, int topk, float* ca,
                            uint8_t* ws, hipStream_t s) {
  // A view of the context whose rows are the score matrix's rows and whose
  // workspace is the calibration workspace.
  fasa_ctx view = *c;
  view.ws = calib_layout(c, topk).ws;
  view.max_budget = topk;
  hipError_t e = launch_prologue(&view, q, seq_lens, max_seq_len, ws, s);
  if (e != hipSuccess) return e;
  const int32_t* nb = reinterpret_cast<const int32_t*>(ws + view.ws.nb);
  const float* qrot = reinterpret_cast<const float*>(ws + view.ws.qrot);
  float* scores = reinterpret_cast<float*>(ws + view.ws.scores);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + view.ws.idx);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + view.ws.err);
  dim3 grid((unsigned)((max_seq_len + kCalTokens - 1) / kCalTokens), (unsigned)c->hkv,
            (unsigned)c->batch);
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_scores_d<true, 128>(c, grid, s, k_cache, qrot, nb, max_seq_len, scores, err);
    else launch_scores_d<false, 128>(c, grid, s, k_cache, qrot, nb, max_seq_len, scores, err);
  } else {
    if (bf) launch_scores_d<true, 64>(c, grid, s, k_cache, qrot, nb, max_seq_len, scores, err);
    else launch_scores_d<false, 64>(c, grid, s, k_cache, qrot, nb, max_seq_len, scores, err);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  view.hq = c->hq * (c->C + 1);
  if (select_path_applies(max_seq_len, topk))
    e = launch_select(&view, scores, nb, max_seq_len, topk, idx, nullptr, nullptr, nullptr,
                      nullptr, ws, s);
  else
    e = launch_topk(&view, scores, nb, max_seq_len, topk, idx, nullptr, ws, s);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(int32_t) * (size_t)topk;
  dim3 g2((unsigned)c->hq, (unsigned)c->batch);
  if (c->C == 64)
    hipLaunchKernelGGL(ca_kernel<64>, g2, dim3(64), lds, s, idx, nb, max_seq_len, c->cap, c->hq,
                       topk, ca);
  else
    hipLaunchKernelGGL(ca_kernel<32>, g2, dim3(64), lds, s, idx, nb, max_seq_len, c->cap, c->hq,
                       topk, ca);
  return hipGetLastError();
}

}  // namespace fasa
