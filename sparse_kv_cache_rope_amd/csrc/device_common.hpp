// Device-side helpers shared by the FASA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fasa {

// Word 3 of a raw buffer resource on gfx950 (32-bit dwords, no swizzle):
// out-of-range lanes of a buffer load read zero and fetch nothing.
constexpr int kBufferRsrcWord3 = 0x00020000;

// A pointer into global memory (address space 1): loads through it are
// global_load, never flat_load.
template <typename T>
using global_ptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ global_ptr<T> to_global(T* p) {
  return (global_ptr<T>)p;
}

constexpr int kWave = 64;

// First radix digit of the top-B select: the top kHistBits of the key.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;

// Largest cache capacity (positions must fit the composite's 32-bit field and
// the grids' int arithmetic with room to spare).
constexpr int kMaxCapacity = 1 << 24;

// ---- bf16 <-> fp32 / fp64 ------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp64 -> bf16, rounded once to nearest-even.  The fp32 intermediate is made
// round-to-odd (exact result, or the truncated value with its last bit set),
// which has 16 spare bits over bf16, so the second rounding is exact.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  float f = (float)x;
  uint32_t u = __float_as_uint(f);
  double back = (double)f;
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1u;  // step the magnitude back toward zero
    u |= 1u;
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- ordering keys for the top-B radix select --------------------------

// Order-preserving map float -> uint32 (larger float -> larger key); -0 is
// folded onto +0 so equal scores compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Composite (key, position): higher key first, then lower position.  All
// composites of a row are distinct, so one threshold splits selected from
// unselected exactly.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - pos);
}
__device__ __forceinline__ uint32_t composite_pos(uint64_t c) {
  return 0xffffffffu - (uint32_t)(c & 0xffffffffu);
}

// ---- cross-lane sums -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// Lanes 0, 16, 32 and 48 of v: one value of each 16-lane row (wave-uniform).
// Every lane of the wave must be active.
struct RowVals {
  uint32_t r0, r1, r2, r3;
};
__device__ __forceinline__ RowVals row_vals(uint32_t v) {
  return RowVals{(uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 16),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                 (uint32_t)__builtin_amdgcn_readlane((int)v, 48)};
}

// Sum over aligned groups of N consecutive lanes (N = 4, 8, 16, 32, 64);
// every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_mov<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
  if constexpr (N == 16 || N == 32 || N == 64) {
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x128>(v);  // row_ror:8
  } else if constexpr (N == 8) {
    v += __shfl_xor(v, 4);
  }
  if constexpr (N >= 32) {
    // Every lane of a row holds the row's sum; the rows meet through lane
    // reads (scalar registers), in the order a lane-xor butterfly adds them.
    const RowVals r = row_vals(__float_as_uint(v));
    const float h0 = __uint_as_float(r.r0) + __uint_as_float(r.r1);
    const float h1 = __uint_as_float(r.r2) + __uint_as_float(r.r3);
    if constexpr (N == 32) v = (threadIdx.x & 32) ? h1 : h0;
    else v = h0 + h1;
  }
  return v;
}

// Wave-wide max (every lane gets it).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
  const RowVals r = row_vals(__float_as_uint(v));
  return fmaxf(fmaxf(__uint_as_float(r.r0), __uint_as_float(r.r1)),
               fmaxf(__uint_as_float(r.r2), __uint_as_float(r.r3)));
}

// Wave-wide min of lo and max of hi (wave-uniform results).
__device__ __forceinline__ void wave_minmax(uint32_t& lo, uint32_t& hi) {
  lo = min(lo, dpp_u32<0xB1>(lo));
  hi = max(hi, dpp_u32<0xB1>(hi));
  lo = min(lo, dpp_u32<0x4E>(lo));
  hi = max(hi, dpp_u32<0x4E>(hi));
  lo = min(lo, dpp_u32<0x124>(lo));
  hi = max(hi, dpp_u32<0x124>(hi));
  lo = min(lo, dpp_u32<0x128>(lo));
  hi = max(hi, dpp_u32<0x128>(hi));
  const RowVals a = row_vals(lo), b = row_vals(hi);
  lo = min(min(a.r0, a.r1), min(a.r2, a.r3));
  hi = max(max(b.r0, b.r1), max(b.r2, b.r3));
}

// Inclusive prefix sum of a uint32 over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64).
// `lds` needs NT / 64 words.  Returns the exclusive prefix; *total gets the
// block total.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds,
                                                         uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) lds[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    uint32_t t = lds[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

__device__ __forceinline__ void raise_flag(uint32_t* err, uint32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// n_b of sequence b, or 0 (and the SEQ_LEN flag when `report`) when it lies
// outside [0, min(max_seq_len, cap)].
__device__ __forceinline__ int checked_len(const int32_t* nb, int b, int max_seq_len, int cap,
                                           uint32_t* err, bool report) {
  const int n = nb[b];
  if (n < 0 || n > max_seq_len || n > cap) {
    if (report) raise_flag(err, 1u);
    return 0;
  }
  return n;
}

// Dimension pair (fc_lo, fc_hi) of FC c of a head of C = d/2 FCs whose first
// 2R dims are rotated (rotate-half within them) and whose other dims pass
// through, paired the same way: (c, c + R) for c < R, (c + R, c + C) for
// c >= R.  R = C is full RoPE, (c, c + C).
__device__ __forceinline__ int fc_lo(int c, int R) { return c < R ? c : c + R; }
__device__ __forceinline__ int fc_hi(int c, int R, int C) { return c < R ? c + R : c + C; }

}  // namespace fasa
