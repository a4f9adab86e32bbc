// KV append with RoPE + FC-packed key sidecar, and the query-only prologue.
//
// RoPE splits a head vector into 2-D frequency chunks (FCs), one angular
// frequency each ("FASA: Frequency-aware Sparse Attention", gist.science/pt,
// "Resumo Tecnico" section 2, "A Descoberta"); keys keep their original
// absolute positions (same section, FAC third bullet).  FC c is the pair
// (c, c + d/2), its angle at position m is m * theta^(-2c/d).  Angles and the
// rotation are taken in fp64 so positions up to ~10^6 lose nothing, and the
// rotated key is rounded once (nearest-even) to the cache dtype.
//
// The sidecar keeps, per KV head, a copy of the rotated K columns of the union
// of its query heads' dominant FCs, one plane per FC ([b][P][cap] pairs), so
// the TIP pass streams only those columns with coalesced 16-byte loads.
// Storing dominant key parts apart from the rest is what FASA-M does with GPU
// memory (same page, "Variantes de Implementacao").

#include "fasa_internal.hpp"
#include "rope_common.hpp"

namespace fasa {

// Bulk append: thread = (row, FC).  grid (ceil(n_new / rows), Hkv, b).
template <bool BF16>
__global__ void __launch_bounds__(256)
append_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
              void* __restrict__ k_cache, void* __restrict__ v_cache, void* __restrict__ sidecar,
              const int32_t* __restrict__ start_pos, int n_new, int hkv, int cap, int d, int P,
              const int32_t* __restrict__ plane_off, const int32_t* __restrict__ fc_slot,
              const double* __restrict__ omega, int R, uint32_t* err) {
  using T = typename CacheT<BF16>::T;
  const int C = d / 2;
  const int rows = blockDim.x / C;
  const int c = threadIdx.x % C;
  const int t = blockIdx.x * rows + threadIdx.x / C;
  const int g = blockIdx.y, b = blockIdx.z;
  if (t >= n_new) return;
  const int p0 = start_pos[b];
  const long pos = (long)p0 + t;
  if (p0 < 0 || pos >= cap) {
    if (c == 0) raise_flag(err, FASA_DEVFLAG_APPEND);
    return;
  }
  const size_t src = (((size_t)b * hkv + g) * n_new + t) * d;
  const size_t dst = (((size_t)b * hkv + g) * cap + pos) * d;
  append_fc<BF16>(static_cast<const T*>(k_new) + src, static_cast<const T*>(v_new) + src,
                  static_cast<T*>(k_cache) + dst, static_cast<T*>(v_cache) + dst, sidecar,
                  (size_t)b * P + plane_off[g], fc_slot[g * C + c], fc_lo(c, R), fc_hi(c, R, C),
                  cap, pos, omega[c]);
}

// Query prologue of the entry points that take no TIP pass, one workgroup per
// (KV head g, sequence b), G * C threads: validate n_b = seq_lens[b] and
// rotate the group's queries to position n_b - 1 (fp64 angle, kept in fp32;
// pass-through FCs copied).
template <bool BF16>
__global__ void __launch_bounds__(512)
prologue_kernel(const void* __restrict__ q, const int32_t* __restrict__ seq_lens,
                int max_seq_len, int hq, int G, int cap, int d,
                const double* __restrict__ omega, int R, int32_t* __restrict__ nb_out,
                float* __restrict__ qrot, uint32_t* err) {
  using T = typename CacheT<BF16>::T;
  const int C = d / 2;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = seq_lens[b];
  const bool ok = n >= 1 && n <= max_seq_len && n <= cap;
  if (!ok) {
    if (g == 0 && tid == 0) {
      nb_out[b] = 0;
      if (n != 0) raise_flag(err, FASA_DEVFLAG_SEQ_LEN);
    }
    return;
  }
  if (g == 0 && tid == 0) nb_out[b] = n;
  const long pos = n - 1;
  const int hh = tid / C, c = tid % C;
  const int h = g * G + hh;
  const T* qs = static_cast<const T*>(q) + ((size_t)b * hq + h) * d;
  const int lo = fc_lo(c, R), hi = fc_hi(c, R, C);
  const double x0 = load_elem(qs, lo), x1 = load_elem(qs, hi);
  const double w = omega[c];
  double sn, cs;
  sincos((double)pos * w, &sn, &cs);
  float* qr = qrot + ((size_t)b * hq + h) * d;
  qr[lo] = (float)(w == 0.0 ? x0 : x0 * cs - x1 * sn);
  qr[hi] = (float)(w == 0.0 ? x1 : x1 * cs + x0 * sn);
}

__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                 size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint4*>(p), n16, static_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

__global__ void copy_u32_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst) {
  *dst = *src;
}

hipError_t launch_copy_u32(const uint32_t* src, uint32_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(copy_u32_kernel, dim3(1), dim3(1), 0, s, src, dst);
  return hipGetLastError();
}

hipError_t launch_append(const fasa_ctx* c, void* k_cache, void* v_cache, void* sidecar,
                         const void* k_new, const void* v_new, const int32_t* start_pos,
                         int n_new, uint8_t* ws, hipStream_t s) {
  if (n_new <= 0) return hipSuccess;
  const int rows = 256 / c->C;
  dim3 grid((unsigned)((n_new + rows - 1) / rows), (unsigned)c->hkv, (unsigned)c->batch);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  if (c->dtype == FASA_BF16)
    hipLaunchKernelGGL(append_kernel<true>, grid, dim3(rows * c->C), 0, s, k_new, v_new, k_cache,
                       v_cache, sidecar, start_pos, n_new, c->hkv, c->cap, c->d, c->P,
                       c->tab.plane_off, c->tab.fc_slot, c->tab.omega, c->R, err);
  else
    hipLaunchKernelGGL(append_kernel<false>, grid, dim3(rows * c->C), 0, s, k_new, v_new, k_cache,
                       v_cache, sidecar, start_pos, n_new, c->hkv, c->cap, c->d, c->P,
                       c->tab.plane_off, c->tab.fc_slot, c->tab.omega, c->R, err);
  return hipGetLastError();
}

hipError_t launch_prologue(const fasa_ctx* c, const void* q, const int32_t* seq_lens,
                           int max_seq_len, uint8_t* ws, hipStream_t s) {
  dim3 grid((unsigned)c->hkv, (unsigned)c->batch);
  dim3 block((unsigned)(c->G * c->C));
  int32_t* nb = reinterpret_cast<int32_t*>(ws + c->ws.nb);
  float* qrot = reinterpret_cast<float*>(ws + c->ws.qrot);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  if (c->dtype == FASA_BF16)
    hipLaunchKernelGGL(prologue_kernel<true>, grid, block, 0, s, q, seq_lens, max_seq_len, c->hq,
                       c->G, c->cap, c->d, c->tab.omega, c->R, nb, qrot, err);
  else
    hipLaunchKernelGGL(prologue_kernel<false>, grid, block, 0, s, q, seq_lens, max_seq_len, c->hq,
                       c->G, c->cap, c->d, c->tab.omega, c->R, nb, qrot, err);
  return hipGetLastError();
}

}  // namespace fasa
