// TIP: Token Importance Prediction over the FC-packed sidecar, fused with the
// step's query rotation and (decode) the append of the step's token.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, TIP "Previsao Online": while decoding, each cached token's
// importance is estimated from the contributions of the pre-calibrated
// dominant FCs only.  For query head h and token j:
//   s[h][j] = sum_{c in I_dom(h)} q~_c K[j][c] + q~_{c+C} K[j][c+C],
// with q~ the query rotated to the current position n - 1 (the query is the
// newest token).  Under partial RoPE FC c is the dim pair fc_lo / fc_hi name
// (R rotated FCs; R = C is full RoPE).
//
// One workgroup (4 waves) covers 256 consecutive tokens of one (sequence, KV
// head) and all G query heads of that KV head.  The KV head's sidecar planes
// (one per FC of the union U_g of the group's dominant FCs) are dealt out to
// the 4 waves; a lane loads 4 consecutive token pairs of a plane with one
// 16-byte load (bf16), so a wave reads 1 KiB contiguous per plane, and every
// wave keeps all its loads in flight at once.
//
// Per-step work that used to be a kernel of its own runs while those loads
// are in flight: every workgroup rotates its group's queries (fp64 angle, kept
// in fp32) into LDS weights (q~_c, q~_{c+C}) per plane and head, zero where
// the FC is not dominant for the head; the tile-0 workgroup also writes the
// rotated queries for FAC; in decode mode the workgroup whose tile holds the
// new position n - 1 rotates and stores the step's key (K, V and sidecar) and
// substitutes the new sidecar pairs into the values its lanes loaded for that
// position.  Sequence lengths are read, never written, here: another
// workgroup of the same launch may still be reading them.
//
// HBM-bound: 4 bytes per token and plane (bf16) against 4 G FMAs.

#include "fasa_internal.hpp"
#include "rope_common.hpp"

namespace fasa {

constexpr int kTipWaves = 4;
constexpr int kTipThreads = kTipWaves * kWave;
constexpr int kTipTokens = kWave * 4;  // tokens per workgroup
constexpr int kMaxPlanes = 64;         // d/2 FCs at d = 128

// The arguments needed first lead the list: the build preloads the first 16
// dwords of kernel arguments into registers, which saves a dependent load
// before the stream starts.
template <bool BF16, int G, int D>
__global__ void __launch_bounds__(kTipThreads)
tip_kernel(const int32_t* __restrict__ seq_lens, void* sidecar, int mode, int max_seq_len,
           int cap, int P, int R, int hkv, const void* __restrict__ q,
           const double* __restrict__ omega, const int32_t* __restrict__ fc_slot,
           const uint64_t* __restrict__ dom_mask, const void* __restrict__ k_new,
           const void* __restrict__ v_new, void* __restrict__ k_cache,
           void* __restrict__ v_cache, int32_t* __restrict__ nb_out, float* __restrict__ qrot,
           float* __restrict__ scores, uint32_t* err, PlaneOffsets po) {
  using T = typename CacheT<BF16>::T;
  constexpr int C = D / 2;
  constexpr int PW = kMaxPlanes / kTipWaves;  // planes per wave, at most
  const int hq = hkv * G;
  __shared__ float4 red[kTipWaves][G][kWave];
  __shared__ float2 wts[kMaxPlanes][G];
  __shared__ uint2 patch[kMaxPlanes];

  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile0 = tile * kTipTokens;
  const int j0 = tile0 + lane * 4;

  // The length, the plane offsets and the argument pointers used before the
  // stream are independent scalar loads: joining them in one (empty) asm
  // makes all of them issue before any is waited on.
  int v = seq_lens[b];
  int p0 = po.off[g];
  int p1 = po.off[g + 1];
  asm volatile("" : "+s"(v), "+s"(p0), "+s"(p1), "+s"(fc_slot), "+s"(dom_mask), "+s"(k_new),
               "+s"(nb_out));
  // The asm hides that these point to global memory; say it again so that
  // loads through them stay global (not flat) loads.
  const global_ptr<const int32_t> fc_slot_g = to_global(fc_slot);
  const global_ptr<const uint64_t> dom_mask_g = to_global(dom_mask);
  const global_ptr<const T> k_new_g = to_global(static_cast<const T*>(k_new));
  const int U = p1 - p0;
  const size_t plane0 = (size_t)b * P + p0;

  // Query elements and tables of this thread's (head, FC) pairs, and the
  // step's key row: loaded unconditionally (clamped indexes) and before the
  // sidecar, so that the exact count of loads in flight lets their first use
  // wait for them alone, not for the stream.
  constexpr int QP = (G * C + kTipThreads - 1) / kTipThreads;
  T qr0[QP], qr1[QP];
  double om[QP];
  int slot[QP];
  uint64_t dmask[QP];
#pragma unroll
  for (int r = 0; r < QP; ++r) {
    const int i = min(tid + r * kTipThreads, G * C - 1);
    const int hh = i / C, c = i % C;
    const T* qs = static_cast<const T*>(q) + ((size_t)b * hq + g * G + hh) * D;
    qr0[r] = qs[fc_lo(c, R)];
    qr1[r] = qs[fc_hi(c, R, C)];
    om[r] = omega[c];
    slot[r] = fc_slot_g[g * C + c];
    dmask[r] = dom_mask_g[g * G + hh];
  }
  // Query-only launches have no key row (k_new may be null): they read the
  // same (unused) indexes of q instead, which holds b * Hq * d >= b * Hkv * d
  // elements.
  const size_t kv_src = ((size_t)b * hkv + g) * D;
  const global_ptr<const T> ksrc =
      (mode == kPrologueDecode) ? k_new_g : to_global(static_cast<const T*>(q));
  const T kr0 = ksrc[kv_src + fc_lo(tid % C, R)];
  const T kr1 = ksrc[kv_src + fc_hi(tid % C, R, C)];

  const int n = (mode == kPrologueDecode) ? v + 1 : v;
  const bool ok = v >= 0 && n >= 1 && n <= max_seq_len && n <= cap;
  const bool lead = (tile == 0 && g == 0 && tid == 0);
  if (!ok) {
    if (lead) {
      nb_out[b] = 0;
      if (!(mode == kPrologueQueryOnly && v == 0)) raise_flag(err, FASA_DEVFLAG_SEQ_LEN);
    }
    return;
  }
  if (lead) nb_out[b] = n;
  if (tile0 >= n) return;
  const long pos = n - 1;
  const bool owner = (mode == kPrologueDecode) && (pos - tile0 < kTipTokens);

  // This wave's sidecar planes, all in flight at once, as buffer loads whose
  // range ends at the plane's first 4 * ceil(n / 4) tokens: planes past U and
  // quads past n read zeros without touching memory, so no load is skipped by
  // a branch.  Each plane gets its own resource (base = the plane).
  constexpr int kPairBytes = BF16 ? 4 : 8;
  const int n4 = (n + 3) & ~3;
  const uint32_t range = (uint32_t)n4 * kPairBytes;
  const uint32_t voff = (uint32_t)j0 * kPairBytes;
  const bool live = j0 < n;
  uint4 xa[PW], xb[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    const int u = wave + k * kTipWaves;
    const char* base = static_cast<const char*>(sidecar) + (plane0 + u) * (size_t)cap * kPairBytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, (u < U) ? (int)range : 0, kBufferRsrcWord3);
    const auto va = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    xa[k] = make_uint4(va[0], va[1], va[2], va[3]);
    if constexpr (!BF16) {
      const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, 0, 0);
      xb[k] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
    }
  }

  // Rotations at position n - 1 while the sidecar streams in.
#pragma unroll
  for (int r = 0; r < QP; ++r) {
    const int i = tid + r * kTipThreads;
    if (i < G * C) {
      const int hh = i / C, c = i % C;
      const bool dom = (dmask[r] >> c) & 1ull;
      const int lo = fc_lo(c, R), hi = fc_hi(c, R, C);
      const bool pass = om[r] == 0.0;  // pass-through FC
      const double qx0 = to_f64(qr0[r]), qx1 = to_f64(qr1[r]);
      double sn, cs;
      sincos((double)pos * om[r], &sn, &cs);
      const float y0 = (float)(pass ? qx0 : qx0 * cs - qx1 * sn);
      const float y1 = (float)(pass ? qx1 : qx1 * cs + qx0 * sn);
      if (tile == 0) {
        float* qr = qrot + ((size_t)b * hq + g * G + hh) * D;
        qr[lo] = y0;
        qr[hi] = y1;
      }
      if (slot[r] >= 0) wts[slot[r]][hh] = dom ? make_float2(y0, y1) : make_float2(0.0f, 0.0f);
      if (owner && i < C) {
        const size_t dst = (((size_t)b * hkv + g) * cap + pos) * D;
        const uint2 pair = store_rotated_fc<BF16>(
            to_f64(kr0), to_f64(kr1), static_cast<const T*>(v_new) + kv_src, static_cast<T*>(k_cache) + dst,
            static_cast<T*>(v_cache) + dst, sidecar, plane0, slot[r], lo, hi, cap, pos, sn, cs,
            pass);
        if (slot[r] >= 0) patch[slot[r]] = pair;
      }
    }
  }
  __syncthreads();

  // The new position's loaded values may predate its store: use the pairs
  // just computed instead.
  if (owner && lane == (int)((pos - tile0) >> 2)) {
    const int t = (int)(pos & 3);
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int u = wave + k * kTipWaves;
      if (u < U) {
        const uint2 p = patch[u];
        if constexpr (BF16) {
          xa[k].x = (t == 0) ? p.x : xa[k].x;
          xa[k].y = (t == 1) ? p.x : xa[k].y;
          xa[k].z = (t == 2) ? p.x : xa[k].z;
          xa[k].w = (t == 3) ? p.x : xa[k].w;
        } else {
          if (t == 0) { xa[k].x = p.x; xa[k].y = p.y; }
          if (t == 1) { xa[k].z = p.x; xa[k].w = p.y; }
          if (t == 2) { xb[k].x = p.x; xb[k].y = p.y; }
          if (t == 3) { xb[k].z = p.x; xb[k].w = p.y; }
        }
      }
    }
  }

  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[hh][t] = 0.0f;
  if (live) {
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int u = wave + k * kTipWaves;
      if (u >= U) break;
      float lo[4], hi[4];
      if constexpr (BF16) {
        const uint32_t wd[4] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          lo[t] = bf16_lo(wd[t]);
          hi[t] = bf16_hi(wd[t]);
        }
      } else {
        lo[0] = __uint_as_float(xa[k].x);
        hi[0] = __uint_as_float(xa[k].y);
        lo[1] = __uint_as_float(xa[k].z);
        hi[1] = __uint_as_float(xa[k].w);
        lo[2] = __uint_as_float(xb[k].x);
        hi[2] = __uint_as_float(xb[k].y);
        lo[3] = __uint_as_float(xb[k].z);
        hi[3] = __uint_as_float(xb[k].w);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float2 w = wts[u][hh];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[hh][t] = fmaf(w.y, hi[t], fmaf(w.x, lo[t], acc[hh][t]));
      }
    }
  }

#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    red[wave][hh][lane] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
  __syncthreads();
  // Thread (hh, quad) sums the waves' partials for 4 tokens of head hh.
  for (int i = tid; i < G * kWave; i += kTipThreads) {
    const int hh = i / kWave, qd = i % kWave;
    float4 s = red[0][hh][qd];
#pragma unroll
    for (int w = 1; w < kTipWaves; ++w) {
      const float4 o = red[w][hh][qd];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    const int j = tile0 + qd * 4;
    float* dst = scores + ((size_t)b * hq + (size_t)g * G + hh) * cap + j;
    if (j + 4 <= n) {
      *reinterpret_cast<float4*>(dst) = s;
    } else {
      const float vv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (j + t < n) dst[t] = vv[t];
    }
  }
}

template <bool BF16, int G, int D>
static void launch_tip_t(dim3 grid, hipStream_t s, int mode, const PlaneOffsets& po,
                         const TipArgs& a, const fasa_ctx* c, int32_t* nb, float* qrot,
                         float* scores, uint32_t* err) {
  hipLaunchKernelGGL((tip_kernel<BF16, G, D>), grid, dim3(kTipThreads), 0, s, a.seq_lens,
                     a.sidecar, mode, a.max_seq_len, c->cap, c->P, c->R, c->hkv, a.q,
                     c->tab.omega, c->tab.fc_slot, c->tab.dom_mask, a.k_new, a.v_new, a.k_cache,
                     a.v_cache, nb, qrot, scores, err, po);
}

template <int G>
static void launch_tip_g(dim3 grid, hipStream_t s, int mode, const PlaneOffsets& po,
                         const TipArgs& a, const fasa_ctx* c, int32_t* nb, float* qrot,
                         float* scores, uint32_t* err) {
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_tip_t<true, G, 128>(grid, s, mode, po, a, c, nb, qrot, scores, err);
    else launch_tip_t<false, G, 128>(grid, s, mode, po, a, c, nb, qrot, scores, err);
  } else {
    if (bf) launch_tip_t<true, G, 64>(grid, s, mode, po, a, c, nb, qrot, scores, err);
    else launch_tip_t<false, G, 64>(grid, s, mode, po, a, c, nb, qrot, scores, err);
  }
}

hipError_t launch_tip(const fasa_ctx* c, PrologueMode mode, const TipArgs& a, float* scores,
                      uint8_t* ws, hipStream_t s) {
  if (c->hkv > kArgKvHeads || c->d / 2 > kMaxPlanes) return hipErrorInvalidValue;
  PlaneOffsets po;
  for (int g = 0; g <= c->hkv; ++g) po.off[g] = c->plane_off[g];
  dim3 grid((unsigned)((a.max_seq_len + kTipTokens - 1) / kTipTokens), (unsigned)c->hkv,
            (unsigned)c->batch);
  if (grid.x == 0) grid.x = 1;  // still validates lengths
  int32_t* nb = reinterpret_cast<int32_t*>(ws + c->ws.nb);
  float* qrot = reinterpret_cast<float*>(ws + c->ws.qrot);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  switch (c->G) {
    case 1: launch_tip_g<1>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err); break;
    case 2: launch_tip_g<2>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err); break;
    case 4: launch_tip_g<4>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err); break;
    case 8: launch_tip_g<8>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fasa
