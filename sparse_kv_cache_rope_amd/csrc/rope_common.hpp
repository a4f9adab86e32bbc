// RoPE helpers shared by the append, prologue and fused TIP kernels.
//
// FC c is the dimension pair (c, c + d/2), its angle at absolute position m is
// m * theta^(-2c/d) ("FASA: Frequency-aware Sparse Attention", gist.science/pt,
// "Resumo Tecnico" section 2, "A Descoberta": 2-D subspaces with one angular
// frequency each).  Under partial RoPE (same page, "Contribuicoes": the
// sparsity holds for Partial-RoPE too) only the first r dims rotate, at
// theta^(-2c/r); FC c is then the pair fc_lo / fc_hi gives, and pass-through
// pairs have frequency 0 and are stored as given.  Angles and the rotation
// are taken in fp64 and the rotated key is rounded once (nearest-even) to the
// cache dtype.
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
__device__ __forceinline__ double to_f64(uint16_t bits) { return (double)bf16_bits_to_f32(bits); }
__device__ __forceinline__ double to_f64(float x) { return (double)x; }

// FC pair (x0, x1) rotated by the angle whose sine and cosine are given
// (pass: a pass-through FC, kept as given) and rounded once to the cache
// dtype: the bit patterns stored (bf16: one packed word in .x, low half the
// lower dim; fp32: the two floats).
template <bool BF16>
__device__ __forceinline__ uint2 rotate_pair(double x0, double x1, double sn, double cs,
                                             bool pass) {
  const double y0 = pass ? x0 : x0 * cs - x1 * sn;
  const double y1 = pass ? x1 : x1 * cs + x0 * sn;
  if constexpr (BF16)
    return make_uint2((uint32_t)f64_to_bf16_rne(y0) | ((uint32_t)f64_to_bf16_rne(y1) << 16), 0u);
  else
    return make_uint2(__float_as_uint((float)y0), __float_as_uint((float)y1));
}

// Stores one FC's rotated key pair (rotate_pair's bits) at dims lo, hi of a K
// row, the V pair as given, and, when the FC is in the KV head's union
// (slot >= 0), the sidecar pair.
template <bool BF16>
__device__ __forceinline__ void store_fc_pair(uint2 kbits, typename CacheT<BF16>::T v0,
                                              typename CacheT<BF16>::T v1,
                                              typename CacheT<BF16>::T* __restrict__ kdst,
                                              typename CacheT<BF16>::T* __restrict__ vdst,
                                              void* __restrict__ sidecar, size_t plane_base,
                                              int slot, int lo, int hi, int cap, long pos) {
  vdst[lo] = v0;
  vdst[hi] = v1;
  if constexpr (BF16) {
    kdst[lo] = (uint16_t)(kbits.x & 0xffffu);
    kdst[hi] = (uint16_t)(kbits.x >> 16);
    if (slot >= 0) static_cast<uint32_t*>(sidecar)[(plane_base + slot) * cap + pos] = kbits.x;
  } else {
    const float k0 = __uint_as_float(kbits.x), k1 = __uint_as_float(kbits.y);
    kdst[lo] = k0;
    kdst[hi] = k1;
    if (slot >= 0) static_cast<float2*>(sidecar)[(plane_base + slot) * cap + pos] = make_float2(k0, k1);
  }
}

// Rotates FC c = (x0, x1) of one key row by the angle whose sine and cosine
// are given (pass: a pass-through FC, kept as given), stores K (and V)
// columns lo, hi (the FC's dims) and, when FC c is in the KV head's union
// (slot >= 0), its sidecar pair.  Returns the bit patterns of the stored pair
// (bf16: one packed word in .x; fp32: the two floats).
template <bool BF16>
__device__ __forceinline__ uint2 store_rotated_fc(double x0, double x1,
                                                  const typename CacheT<BF16>::T* __restrict__ vsrc,
                                                  typename CacheT<BF16>::T* __restrict__ kdst,
                                                  typename CacheT<BF16>::T* __restrict__ vdst,
                                                  void* __restrict__ sidecar, size_t plane_base,
                                                  int slot, int lo, int hi, int cap, long pos,
                                                  double sn, double cs, bool pass) {
  const uint2 bits = rotate_pair<BF16>(x0, x1, sn, cs, pass);
  store_fc_pair<BF16>(bits, vsrc[lo], vsrc[hi], kdst, vdst, sidecar, plane_base, slot, lo, hi,
                      cap, pos);
  return bits;
}

// store_rotated_fc at the RoPE angle of FC c (dims lo, hi) at position pos
// (fp64); omega = 0 marks a pass-through FC.
template <bool BF16>
__device__ __forceinline__ void append_fc(const typename CacheT<BF16>::T* __restrict__ ksrc,
                                          const typename CacheT<BF16>::T* __restrict__ vsrc,
                                          typename CacheT<BF16>::T* __restrict__ kdst,
                                          typename CacheT<BF16>::T* __restrict__ vdst,
                                          void* __restrict__ sidecar, size_t plane_base,
                                          int slot, int lo, int hi, int cap, long pos,
                                          double omega) {
  double sn, cs;
  sincos((double)pos * omega, &sn, &cs);
  store_rotated_fc<BF16>(load_elem(ksrc, lo), load_elem(ksrc, hi), vsrc, kdst, vdst, sidecar,
                         plane_base, slot, lo, hi, cap, pos, sn, cs, omega == 0.0);
}

}  // namespace fasa
