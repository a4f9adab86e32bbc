// RoPE helpers shared by the append, prologue and fused TIP kernels.
//
// FC c is the dimension pair (c, c + d/2), its angle at absolute position m is
// m * theta^(-2c/d) ("FASA: Frequency-aware Sparse Attention", gist.science/pt,
// "Resumo Tecnico" section 2, "A Descoberta": 2-D subspaces with one angular
// frequency each).  Angles and the rotation are taken in fp64 and the rotated
// key is rounded once (nearest-even) to the cache dtype.
#pragma once

#include "device_common.hpp"

namespace fasa {

template <bool BF16>
struct CacheT;
template <>
struct CacheT<true> {
  using T = uint16_t;
};
template <>
struct CacheT<false> {
  using T = float;
};

__device__ __forceinline__ double load_elem(const uint16_t* p, size_t i) {
  return (double)bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ double load_elem(const float* p, size_t i) { return (double)p[i]; }

// Rotates FC c of one key row at `pos`, stores K (and V) columns c, c + C and,
// when FC c is in the KV head's union, its sidecar pair.
template <bool BF16>
__device__ __forceinline__ void append_fc(const typename CacheT<BF16>::T* __restrict__ ksrc,
                                          const typename CacheT<BF16>::T* __restrict__ vsrc,
                                          typename CacheT<BF16>::T* __restrict__ kdst,
                                          typename CacheT<BF16>::T* __restrict__ vdst,
                                          void* __restrict__ sidecar, size_t plane_base,
                                          int slot, int c, int C, int cap, long pos,
                                          double omega) {
  const double x0 = load_elem(ksrc, c), x1 = load_elem(ksrc, c + C);
  double sn, cs;
  sincos((double)pos * omega, &sn, &cs);
  const double y0 = x0 * cs - x1 * sn;
  const double y1 = x1 * cs + x0 * sn;
  vdst[c] = vsrc[c];
  vdst[c + C] = vsrc[c + C];
  if constexpr (BF16) {
    const uint16_t k0 = f64_to_bf16_rne(y0), k1 = f64_to_bf16_rne(y1);
    kdst[c] = k0;
    kdst[c + C] = k1;
    if (slot >= 0)
      static_cast<uint32_t*>(sidecar)[(plane_base + slot) * cap + pos] =
          (uint32_t)k0 | ((uint32_t)k1 << 16);
  } else {
    const float k0 = (float)y0, k1 = (float)y1;
    kdst[c] = k0;
    kdst[c + C] = k1;
    if (slot >= 0) static_cast<float2*>(sidecar)[(plane_base + slot) * cap + pos] = make_float2(k0, k1);
  }
}

}  // namespace fasa
