// TIP: Token Importance Prediction over the FC-packed sidecar.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, TIP "Previsao Online": while decoding, each cached token's
// importance is estimated from the contributions of the pre-calibrated
// dominant FCs only.  For query head h and token j:
//   s[h][j] = sum_{c in I_dom(h)} q~_c K[j][c] + q~_{c+C} K[j][c+C].
//
// One workgroup (4 waves) covers 256 consecutive tokens of one (sequence, KV
// head) and all G query heads of that KV head.  The KV head's sidecar planes
// (one per FC of the union U_g of the group's dominant FCs) are dealt out to
// the 4 waves; a lane loads 4 consecutive token pairs of a plane with one
// 16-byte load (bf16), so a wave reads 1 KiB contiguous per plane, and every
// wave keeps all its loads in flight at once.  The per-plane weights
// (q~_c, q~_{c+C}) of each head, zero where the FC is not dominant for that
// head, are uniform across the wave (scalar loads).  The waves' partial sums
// meet in LDS.  HBM-bound: 4 bytes per token and plane against 4 G FMAs.

#include "device_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

constexpr int kTipWaves = 4;
constexpr int kTipTokens = kWave * 4;  // tokens per workgroup
constexpr int kMaxPlanes = 64;         // d/2 FCs at d = 128

template <bool BF16, int G>
__global__ void __launch_bounds__(kTipWaves * kWave)
tip_kernel(const void* __restrict__ sidecar, const float* __restrict__ tipw,
           const int32_t* __restrict__ nb, int max_seq_len, int hq, int cap, int P,
           const int32_t* __restrict__ plane_off, float* __restrict__ scores,
           int32_t* __restrict__ advance, uint32_t* err) {
  __shared__ float4 red[kTipWaves][G][kWave];
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const bool lead = (tile == 0 && g == 0 && threadIdx.x == 0);
  const int n = checked_len(nb, b, max_seq_len, cap, err, lead);
  if (lead && advance != nullptr && n > 0) advance[b] = n;
  const int tile0 = tile * kTipTokens;
  if (tile0 >= n) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int j0 = tile0 + lane * 4;

  const int p0 = plane_off[g];
  const int U = plane_off[g + 1] - p0;
  const size_t plane0 = (size_t)b * P + p0;

  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[hh][t] = 0.0f;

  if (j0 < n) {
    const float* __restrict__ w0 = tipw + plane0 * (G * 2);
    if constexpr (BF16) {
      // All of this wave's planes (at most kMaxPlanes / kTipWaves) in flight at once.
      const uint32_t* __restrict__ src = static_cast<const uint32_t*>(sidecar) + plane0 * cap + j0;
      constexpr int PW = kMaxPlanes / kTipWaves;
      uint4 x[PW];
#pragma unroll
      for (int k = 0; k < PW; ++k) {
        const int u = wave + k * kTipWaves;
        if (u < U) x[k] = *reinterpret_cast<const uint4*>(src + (size_t)u * cap);
      }
#pragma unroll
      for (int k = 0; k < PW; ++k) {
        const int u = wave + k * kTipWaves;
        if (u >= U) break;
        const float* w = w0 + u * (G * 2);
        const uint32_t wd[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float lo = bf16_lo(wd[t]), hi = bf16_hi(wd[t]);
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            acc[hh][t] = fmaf(w[2 * hh + 1], hi, fmaf(w[2 * hh], lo, acc[hh][t]));
        }
      }
    } else {
      const float2* __restrict__ src = static_cast<const float2*>(sidecar) + plane0 * cap + j0;
      for (int u = wave; u < U; u += kTipWaves) {
        const float4 a = *reinterpret_cast<const float4*>(src + (size_t)u * cap);
        const float4 c = *reinterpret_cast<const float4*>(src + (size_t)u * cap + 2);
        const float* w = w0 + u * (G * 2);
        const float lo[4] = {a.x, a.z, c.x, c.z};
        const float hi[4] = {a.y, a.w, c.y, c.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            acc[hh][t] = fmaf(w[2 * hh + 1], hi[t], fmaf(w[2 * hh], lo[t], acc[hh][t]));
      }
    }
  }

#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    red[wave][hh][lane] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
  __syncthreads();
  // Thread (hh, quad) sums the waves' partials for 4 tokens of head hh.
  for (int i = threadIdx.x; i < G * kWave; i += kTipWaves * kWave) {
    const int hh = i / kWave, q = i % kWave;
    float4 s = red[0][hh][q];
#pragma unroll
    for (int w = 1; w < kTipWaves; ++w) {
      const float4 o = red[w][hh][q];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    const int j = tile0 + q * 4;
    float* dst = scores + ((size_t)b * hq + (size_t)g * G + hh) * cap + j;
    if (j + 4 <= n) {
      *reinterpret_cast<float4*>(dst) = s;
    } else {
      const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (j + t < n) dst[t] = v[t];
    }
  }
}

template <bool BF16, int G>
static void launch_tip_t(dim3 grid, hipStream_t s, const void* sidecar, const float* tipw,
                         const int32_t* nb, int max_seq_len, int hq, int cap, int P,
                         const int32_t* plane_off, float* scores, int32_t* advance,
                         uint32_t* err) {
  hipLaunchKernelGGL((tip_kernel<BF16, G>), grid, dim3(kTipWaves * kWave), 0, s, sidecar, tipw,
                     nb, max_seq_len, hq, cap, P, plane_off, scores, advance, err);
}

hipError_t launch_tip(const fasa_ctx* c, const void* sidecar, const int32_t* nb,
                      int max_seq_len, float* scores, int32_t* advance_seq_lens, uint8_t* ws,
                      hipStream_t s) {
  dim3 grid((unsigned)((max_seq_len + kTipTokens - 1) / kTipTokens), (unsigned)c->hkv,
            (unsigned)c->batch);
  if (grid.x == 0) grid.x = 1;  // still validates lengths and advances
  const float* tipw = reinterpret_cast<const float*>(ws + c->ws.tipw);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
#define FASA_TIP_CASE(BF, GG)                                                              \
  launch_tip_t<BF, GG>(grid, s, sidecar, tipw, nb, max_seq_len, c->hq, c->cap, c->P,       \
                       c->tab.plane_off, scores, advance_seq_lens, err)
  const bool bf = (c->dtype == FASA_BF16);
  switch (c->G) {
    case 1: if (bf) FASA_TIP_CASE(true, 1); else FASA_TIP_CASE(false, 1); break;
    case 2: if (bf) FASA_TIP_CASE(true, 2); else FASA_TIP_CASE(false, 2); break;
    case 4: if (bf) FASA_TIP_CASE(true, 4); else FASA_TIP_CASE(false, 4); break;
    case 8: if (bf) FASA_TIP_CASE(true, 8); else FASA_TIP_CASE(false, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef FASA_TIP_CASE
  return hipGetLastError();
}

}  // namespace fasa
