// TIP: Token Importance Prediction over the FC-packed sidecar.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, TIP "Previsao Online": while decoding, each cached token's
// importance is estimated from the contributions of the pre-calibrated
// dominant FCs only.  For query head h and token j:
//   s[h][j] = sum_{c in I_dom(h)} q~_c K[j][c] + q~_{c+C} K[j][c+C].
//
// One workgroup covers 256 * TPT consecutive tokens of one (sequence, KV head)
// and all G query heads of that KV head.  It walks the KV head's sidecar
// planes (one per FC of the union U_g of the group's dominant FCs); each
// thread loads TPT consecutive token pairs of a plane with one 16-byte load
// (bf16), so a wave reads 1 KiB contiguous per plane.  The per-plane weights
// (q~_c, q~_{c+C}) for each head, zero where the FC is not dominant for that
// head, are uniform across the workgroup and come in through scalar loads.
// The pass is HBM-bound: 4 bytes per token per plane against 4 * G FMAs.

#include "device_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

template <bool BF16, int G, int TPT>
__global__ void __launch_bounds__(256)
tip_kernel(const void* __restrict__ sidecar, const float* __restrict__ tipw,
           const int32_t* __restrict__ nb, int max_seq_len, int hq, int cap, int P,
           const int32_t* __restrict__ plane_off, float* __restrict__ scores,
           int32_t* __restrict__ advance, uint32_t* err) {
  static_assert(TPT == 4, "one 16-byte bf16 load (two for fp32) per plane");
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const bool lead = (tile == 0 && g == 0 && threadIdx.x == 0);
  const int n = checked_len(nb, b, max_seq_len, cap, err, lead);
  if (lead && advance != nullptr && n > 0) advance[b] = n;
  const int tile0 = tile * 256 * TPT;
  if (tile0 >= n) return;
  const int j0 = tile0 + threadIdx.x * TPT;
  if (j0 >= n) return;

  const int p0 = plane_off[g];
  const int U = plane_off[g + 1] - p0;
  const size_t plane0 = (size_t)b * P + p0;

  float acc[G][TPT];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int t = 0; t < TPT; ++t) acc[hh][t] = 0.0f;

  const float* __restrict__ w0 = tipw + plane0 * (G * 2);

  if constexpr (BF16) {
    const uint32_t* __restrict__ src = static_cast<const uint32_t*>(sidecar) + plane0 * cap + j0;
    constexpr int UNR = 8;
    int u = 0;
    for (; u + UNR <= U; u += UNR) {
      uint4 x[UNR];
#pragma unroll
      for (int k = 0; k < UNR; ++k)
        x[k] = *reinterpret_cast<const uint4*>(src + (size_t)(u + k) * cap);
#pragma unroll
      for (int k = 0; k < UNR; ++k) {
        const float* w = w0 + (u + k) * (G * 2);
        const uint32_t wd[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
        for (int t = 0; t < TPT; ++t) {
          const float lo = bf16_lo(wd[t]), hi = bf16_hi(wd[t]);
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            acc[hh][t] = fmaf(w[2 * hh + 1], hi, fmaf(w[2 * hh], lo, acc[hh][t]));
        }
      }
    }
    for (; u < U; ++u) {
      const uint4 x = *reinterpret_cast<const uint4*>(src + (size_t)u * cap);
      const float* w = w0 + u * (G * 2);
      const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const float lo = bf16_lo(wd[t]), hi = bf16_hi(wd[t]);
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          acc[hh][t] = fmaf(w[2 * hh + 1], hi, fmaf(w[2 * hh], lo, acc[hh][t]));
      }
    }
  } else {
    const float2* __restrict__ src = static_cast<const float2*>(sidecar) + plane0 * cap + j0;
    for (int u = 0; u < U; ++u) {
      const float4 a = *reinterpret_cast<const float4*>(src + (size_t)u * cap);
      const float4 c = *reinterpret_cast<const float4*>(src + (size_t)u * cap + 2);
      const float* w = w0 + u * (G * 2);
      const float lo[4] = {a.x, a.z, c.x, c.z};
      const float hi[4] = {a.y, a.w, c.y, c.w};
#pragma unroll
      for (int t = 0; t < TPT; ++t)
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
          acc[hh][t] = fmaf(w[2 * hh + 1], hi[t], fmaf(w[2 * hh], lo[t], acc[hh][t]));
    }
  }

#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float* dst = scores + ((size_t)b * hq + (size_t)g * G + hh) * cap + j0;
    if (j0 + TPT <= n) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
    } else {
#pragma unroll
      for (int t = 0; t < TPT; ++t)
        if (j0 + t < n) dst[t] = acc[hh][t];
    }
  }
}

template <bool BF16, int G>
static void launch_tip_t(dim3 grid, hipStream_t s, const void* sidecar, const float* tipw,
                         const int32_t* nb, int max_seq_len, int hq, int cap, int P,
                         const int32_t* plane_off, float* scores, int32_t* advance,
                         uint32_t* err) {
  hipLaunchKernelGGL((tip_kernel<BF16, G, 4>), grid, dim3(256), 0, s, sidecar, tipw, nb,
                     max_seq_len, hq, cap, P, plane_off, scores, advance, err);
}

hipError_t launch_tip(const fasa_ctx* c, const void* sidecar, const int32_t* nb,
                      int max_seq_len, float* scores, int32_t* advance_seq_lens, uint8_t* ws,
                      hipStream_t s) {
  const int per_block = 256 * 4;
  dim3 grid((unsigned)((max_seq_len + per_block - 1) / per_block), (unsigned)c->hkv,
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
