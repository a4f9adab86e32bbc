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
// Two kernels share the layout below.  tip_kernel: one workgroup (4 waves)
// covers 256 consecutive tokens of one (sequence, KV head) and all G query
// heads of that KV head.  tip_head_kernel (G = 4 or 8, at most 16 dominant FCs
// per head): the same tile, one wave per query head over that head's own
// planes (its comment has the details).  In tip_kernel the KV head's sidecar
// planes (one per FC of the union U_g of the group's dominant FCs) are dealt
// out to the 4 waves.  In both, a lane loads 4 consecutive token pairs of a
// plane with one 16-byte load (bf16), so a wave reads 1 KiB contiguous per
// plane, and every wave keeps all its loads in flight at once.
//
// The step's other per-token work is fused here and runs while those loads
// are in flight: every workgroup rotates its group's queries (in fp64, kept
// in fp32) into LDS weights (q~_c, q~_{c+C}) per plane and head, zero where
// the FC is not dominant for the head; in decode mode the workgroup whose tile
// holds the new position n - 1 also rotates the step's key.
//
// Order of work, so that every wait counts exactly the loads it needs:
//   1. the length (scalar), then the query pairs, the tables and the step's
//      K/V pair (vector) are issued;
//   2. once the length is in, the sidecar stream is issued, a wave's planes
//      in order (a workgroup with nothing to read gets empty ranges);
//   3. the rotations run as soon as the step-1 loads are in (issued before
//      the stream, with no branch between: the wait is for them alone);
//      results kept in registers and LDS; only then may a workgroup leave;
//      one barrier;
//   4. plane k's FMAs wait for plane k's load only (the compiler counts the
//      loads issued after it), so the sums proceed as the data arrives;
//   5. every global store of the launch comes last: scores, the rotated
//      queries (tile 0), the step's K, V and sidecar pairs (the owner tile),
//      the length.  A store pending among the loads would make the compiler
//      wait for all of them.
// The owner tile's loaded values at n - 1 may predate the step's own pairs:
// its FMA loop (a copy of the others', under one uniform branch) selects the
// new pairs into that position's lane instead.
//
// In a decode step whose selection is filtered, the launch also writes the
// largest score key of every 16-token group, after the scores: the B-th
// largest group maximum bounds the row's threshold from below (filter.hip).
//
// HBM-bound: 4 bytes per token and plane (bf16) against 4 G FMAs.

#include <type_traits>

#include "fasa_internal.hpp"
#include "rope_common.hpp"

namespace fasa {

constexpr int kTipWaves = 4;
constexpr int kTipThreads = kTipWaves * kWave;
constexpr int kTipTokens = kWave * 4;  // tokens per workgroup
constexpr int kMaxPlanes = 64;         // d/2 FCs at d = 128
static_assert(kGroupTokens == 16, "a group is the 4 tokens of each lane of a quad");

typedef __bf16 tip_bf16x2 __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c over bf16 pairs, accumulated in fp32.
__device__ __forceinline__ float tip_dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(tip_bf16x2, a),
                                         __builtin_bit_cast(tip_bf16x2, b), c, false);
}

// bf16 bits of a finite float, rounded to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The arguments needed first lead the list: the build preloads the first 16
// dwords of kernel arguments into registers, which saves a dependent load
// before the stream starts.  PW: sidecar loads per wave, enough for the
// context's largest union (4 PW >= max_g |U_g|).
template <bool BF16, int G, int D, int PW>
__global__ void __launch_bounds__(kTipThreads)
tip_kernel(const int32_t* __restrict__ seq_lens, void* sidecar, int mode, int max_seq_len,
           int cap, int P, int R, int hkv, const void* __restrict__ q,
           const double* __restrict__ omega, const int32_t* __restrict__ fc_slot,
           const uint64_t* __restrict__ dom_mask, const void* __restrict__ k_new,
           const void* __restrict__ v_new, void* __restrict__ k_cache,
           void* __restrict__ v_cache, int32_t* __restrict__ nb_out, float* __restrict__ qrot,
           float* __restrict__ scores, uint32_t* err, PlaneOffsets po,
           uint32_t* __restrict__ gmax, int gstride) {
  using T = typename CacheT<BF16>::T;
  constexpr int C = D / 2;
  constexpr int kPairBytes = BF16 ? 4 : 8;
  static_assert(PW * kTipWaves <= kMaxPlanes, "planes per wave");
  const int hq = hkv * G;
  __shared__ float4 red[kTipWaves][G][kWave];
  __shared__ float2 wts[kMaxPlanes][G];
  __shared__ uint2 patch[kMaxPlanes];

  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile0 = tile * kTipTokens;

  // The length, the plane offsets and the argument pointers used before the
  // stream are independent scalar loads: joining them in one (empty) asm
  // makes all of them issue before any is waited on.
  int v = seq_lens[b];
  int p0 = po.off[g];
  int p1 = po.off[g + 1];
  asm volatile("" : "+s"(v), "+s"(p0), "+s"(p1), "+s"(fc_slot), "+s"(dom_mask), "+s"(k_new),
               "+s"(v_new));
  // The asm hides that these point to global memory; say it again so that
  // loads through them stay global (not flat) loads.
  const global_ptr<const int32_t> fc_slot_g = to_global(fc_slot);
  const global_ptr<const uint64_t> dom_mask_g = to_global(dom_mask);
  const global_ptr<const T> k_new_g = to_global(static_cast<const T*>(k_new));
  const global_ptr<const T> v_new_g = to_global(static_cast<const T*>(v_new));
  const int U = p1 - p0;
  const size_t plane0 = (size_t)b * P + p0;

  // This thread's (head, FC) pairs: query elements and tables; loaded with
  // clamped indexes so that every thread issues the same loads.
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
  // The step's key and value pair of FC tid % C.  Query-only launches have no
  // such row (k_new, v_new may be null): they read the same (unused) indexes
  // of q instead, which holds b * Hq * d >= b * Hkv * d elements.
  const bool decode = (mode == kPrologueDecode);
  const size_t kv_src = ((size_t)b * hkv + g) * D;
  const global_ptr<const T> ksrc = decode ? k_new_g : to_global(static_cast<const T*>(q));
  const global_ptr<const T> vsrc = decode ? v_new_g : to_global(static_cast<const T*>(q));
  const int c_own = tid % C;
  const T kr0 = ksrc[kv_src + fc_lo(c_own, R)];
  const T kr1 = ksrc[kv_src + fc_hi(c_own, R, C)];
  const T vr0 = vsrc[kv_src + fc_lo(c_own, R)];
  const T vr1 = vsrc[kv_src + fc_hi(c_own, R, C)];

  // Keep the loads above ahead of the stream.
  __builtin_amdgcn_sched_barrier(0);

  const int n = decode ? v + 1 : v;
  const bool ok = v >= 0 && n >= 1 && n <= max_seq_len && n <= cap;
  const bool lead = (tile == 0 && g == 0 && tid == 0);
  const bool live = ok && tile0 < n;  // this workgroup has tokens to score
  const long pos = n - 1;
  const bool owner = live && decode && (pos - tile0 < kTipTokens);

  // 2. This wave's sidecar planes, all in flight at once, as buffer loads
  // whose resource starts at the tile's first pair and ends at the plane's
  // first 4 * ceil(n / 4) tokens: planes past U, quads past n and workgroups
  // with nothing to score read zeros without touching memory, so no load is
  // skipped by a branch, and the per-lane offset is the only vector operand.
  const int left = live ? ((n + 3) & ~3) - tile0 : 0;
  const int range = left * kPairBytes;
  const uint32_t voff = (uint32_t)lane * 4 * kPairBytes;
  uint4 xa[PW], xb[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    const int u = wave + k * kTipWaves;
    const char* base = static_cast<const char*>(sidecar) +
                       ((plane0 + u) * (size_t)cap + (size_t)tile0) * kPairBytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, (u < U) ? range : 0, kBufferRsrcWord3);
    const auto va = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    xa[k] = make_uint4(va[0], va[1], va[2], va[3]);
    if constexpr (!BF16) {
      const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, 0, 0);
      xb[k] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
    }
  }

  // Every stream load issues before the rotations below wait for anything.
  __builtin_amdgcn_sched_barrier(0);

  // 3. Rotations at position n - 1 while the stream is in flight.
  float qy0[QP], qy1[QP];
  uint2 own_bits = make_uint2(0u, 0u);
#pragma unroll
  for (int r = 0; r < QP; ++r) {
    const int i = min(tid + r * kTipThreads, G * C - 1);
    const int hh = i / C, c = i % C;
    const bool dom = (dmask[r] >> c) & 1ull;
    const bool pass = om[r] == 0.0;  // pass-through FC
    const double qx0 = to_f64(qr0[r]), qx1 = to_f64(qr1[r]);
    // The query's rotation in fp64, kept in fp32.
    const double ang = (double)pos * om[r];
    double sn, cs;
    sincos(ang, &sn, &cs);
    qy0[r] = (float)(pass ? qx0 : qx0 * cs - qx1 * sn);
    qy1[r] = (float)(pass ? qx1 : qx1 * cs + qx0 * sn);
    if (tid + r * kTipThreads < G * C && slot[r] >= 0)
      wts[slot[r]][hh] = dom ? make_float2(qy0[r], qy1[r]) : make_float2(0.0f, 0.0f);
    if (r == 0 && owner) {
      // The tile holding the step's position also rotates the step's key, in
      // fp64 like the bulk append (the cache keeps its bf16 rounding of the
      // exact rotation).  Thread tid < C holds FC tid here (head 0), the FC
      // of its key pair.
      own_bits = rotate_pair<BF16>(to_f64(kr0), to_f64(kr1), sn, cs, pass);
      if (tid < C && slot[0] >= 0) patch[slot[0]] = own_bits;
    }
  }
  if (!live) {
    if (lead) {
      nb_out[b] = ok ? n : 0;
      if (!ok && !(mode == kPrologueQueryOnly && v == 0)) raise_flag(err, FASA_DEVFLAG_SEQ_LEN);
    }
    return;
  }
  __syncthreads();

  // 4. Sums over this wave's planes for its 4 tokens and the G heads.
  float acc[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[hh][t] = 0.0f;
  const bool pos_lane = lane == (int)((pos - tile0) >> 2);
  const int pos_t = (int)(pos & 3);
  auto sums = [&](auto own) {
    constexpr bool OWN = decltype(own)::value;
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int u = wave + k * kTipWaves;
      if (u >= U) break;
      uint4 da = xa[k], db = xb[k];
      if constexpr (OWN) {
        const uint2 p = patch[u];
        if constexpr (BF16) {
          da.x = (pos_lane && pos_t == 0) ? p.x : da.x;
          da.y = (pos_lane && pos_t == 1) ? p.x : da.y;
          da.z = (pos_lane && pos_t == 2) ? p.x : da.z;
          da.w = (pos_lane && pos_t == 3) ? p.x : da.w;
        } else {
          da.x = (pos_lane && pos_t == 0) ? p.x : da.x;
          da.y = (pos_lane && pos_t == 0) ? p.y : da.y;
          da.z = (pos_lane && pos_t == 1) ? p.x : da.z;
          da.w = (pos_lane && pos_t == 1) ? p.y : da.w;
          db.x = (pos_lane && pos_t == 2) ? p.x : db.x;
          db.y = (pos_lane && pos_t == 2) ? p.y : db.y;
          db.z = (pos_lane && pos_t == 3) ? p.x : db.z;
          db.w = (pos_lane && pos_t == 3) ? p.y : db.w;
        }
      }
      float lo[4], hi[4];
      if constexpr (BF16) {
        const uint32_t wd[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          lo[t] = bf16_lo(wd[t]);
          hi[t] = bf16_hi(wd[t]);
        }
      } else {
        lo[0] = __uint_as_float(da.x);
        hi[0] = __uint_as_float(da.y);
        lo[1] = __uint_as_float(da.z);
        hi[1] = __uint_as_float(da.w);
        lo[2] = __uint_as_float(db.x);
        hi[2] = __uint_as_float(db.y);
        lo[3] = __uint_as_float(db.z);
        hi[3] = __uint_as_float(db.w);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float2 w = wts[u][hh];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[hh][t] = fmaf(w.y, hi[t], fmaf(w.x, lo[t], acc[hh][t]));
      }
    }
  };
  if (owner)
    sums(std::true_type{});
  else
    sums(std::false_type{});
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
    red[wave][hh][lane] = make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
  __syncthreads();

  // 5. Stores.  Thread (hh, quad) sums the waves' partials for 4 tokens of
  // head hh.
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
    if (gmax != nullptr) {
      // The largest score key of each kGroupTokens-token group: the 4
      // tokens of each lane of the quad (key 0 past n, >= 1 otherwise).
      const float vv[4] = {s.x, s.y, s.z, s.w};
      uint32_t km = 0u;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t kk = score_key(vv[t]);
        km = max(km, (j + t < n) ? (kk ? kk : 1u) : 0u);
      }
      km = max(km, dpp_u32<0xB1>(km));  // quad_perm [1,0,3,2]
      km = max(km, dpp_u32<0x4E>(km));  // quad_perm [2,3,0,1]: the quad's maximum
      // Only groups holding a token of the row: the row's gstride groups
      // end at the capacity, which a last tile may reach past.
      if ((qd & 3) == 0 && j < n)
        gmax[((size_t)b * hq + (size_t)g * G + hh) * gstride + (size_t)(j / kGroupTokens)] = km;
    }
  }
  if (tile == 0) {
#pragma unroll
    for (int r = 0; r < QP; ++r) {
      const int i = tid + r * kTipThreads;
      if (i < G * C) {
        const int hh = i / C, c = i % C;
        float* qr = qrot + ((size_t)b * hq + g * G + hh) * D;
        qr[fc_lo(c, R)] = qy0[r];
        qr[fc_hi(c, R, C)] = qy1[r];
      }
    }
  }
  if (owner && tid < C) {
    const size_t dst = (((size_t)b * hkv + g) * cap + pos) * D;
    store_fc_pair<BF16>(own_bits, vr0, vr1, static_cast<T*>(k_cache) + dst,
                        static_cast<T*>(v_cache) + dst, sidecar, plane0, slot[0],
                        fc_lo(tid, R), fc_hi(tid, R, C), cap, pos);
  }
  if (lead) nb_out[b] = n;
}

// TIP with one wave per query head (G = 4 or 8 heads per KV head, at most
// kHeadPlanes dominant FCs per head).  The workgroup again covers 256 tokens
// of one (sequence, KV head), but wave w streams only the planes of query
// head g G + w's own dominant FCs (a plane dominant for several heads is read
// by each of their waves; the copies meet in the cache) and sums them for its
// 4 tokens per lane: no FMA is spent on a plane whose weight for the head is
// zero (about 2/3 of them for G = 4 in the union layout above), and no sum
// across waves is needed.  Every lane rotates FC lane % C of its head; the
// dominant FCs' rotated pairs are read across the wave.  The order of work,
// the owner tile's append and the stores follow tip_kernel.
constexpr int kHeadPlanes = 16;

template <bool BF16, int G, int D, int PW>
__global__ void __launch_bounds__(G * kWave)
tip_head_kernel(const int32_t* __restrict__ seq_lens, void* sidecar,
                const int2* __restrict__ head_fc, int mode, int max_seq_len, int cap, int P,
                int R, int hkv, const void* __restrict__ q, const double* __restrict__ omega,
                const int32_t* __restrict__ fc_slot, const void* __restrict__ k_new,
                const void* __restrict__ v_new, void* __restrict__ k_cache,
                void* __restrict__ v_cache, int32_t* __restrict__ nb_out, float* __restrict__ qrot,
                float* __restrict__ scores, uint32_t* err, PlaneOffsets po,
                uint32_t* __restrict__ gmax, int gstride) {
  using T = typename CacheT<BF16>::T;
  constexpr int C = D / 2;
  constexpr int kPairBytes = BF16 ? 4 : 8;
  static_assert(PW <= kHeadPlanes && C <= kWave, "planes per head, FCs per lane");
  const int hq = hkv * G;

  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tile0 = tile * kTipTokens;
  const int h = g * G + wave;  // this wave's query head within the KV head's group

  // Scalar loads first, issued together (see tip_kernel): the head's (FC,
  // plane) list, the length and the KV head's plane offset (the first three
  // arguments arrive preloaded).
  int2 hf[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) hf[k] = head_fc[(size_t)h * kHeadPlanes + k];
  int v = seq_lens[b];
  int p0 = po.off[g];
  asm volatile("" : "+s"(v), "+s"(p0), "+s"(fc_slot), "+s"(k_new), "+s"(v_new));
  const global_ptr<const int32_t> fc_slot_g = to_global(fc_slot);
  const global_ptr<const T> k_new_g = to_global(static_cast<const T*>(k_new));
  const global_ptr<const T> v_new_g = to_global(static_cast<const T*>(v_new));
  const size_t plane0 = (size_t)b * P + p0;

  // This lane's FC c = lane % C of head h: query pair and frequency; and the
  // step's key and value pair of FC c (query-only launches read q instead,
  // as in tip_kernel).
  const int c = lane % C;
  const T* qs = static_cast<const T*>(q) + ((size_t)b * hq + h) * D;
  const T qr0 = qs[fc_lo(c, R)];
  const T qr1 = qs[fc_hi(c, R, C)];
  const double om = omega[c];
  const int slot_c = fc_slot_g[g * C + c];
  const bool decode = (mode == kPrologueDecode);
  const size_t kv_src = ((size_t)b * hkv + g) * D;
  const global_ptr<const T> ksrc = decode ? k_new_g : to_global(static_cast<const T*>(q));
  const global_ptr<const T> vsrc = decode ? v_new_g : to_global(static_cast<const T*>(q));
  const T kr0 = ksrc[kv_src + fc_lo(c, R)];
  const T kr1 = ksrc[kv_src + fc_hi(c, R, C)];
  const T vr0 = vsrc[kv_src + fc_lo(c, R)];
  const T vr1 = vsrc[kv_src + fc_hi(c, R, C)];

  __builtin_amdgcn_sched_barrier(0);

  const int n = decode ? v + 1 : v;
  const bool ok = v >= 0 && n >= 1 && n <= max_seq_len && n <= cap;
  const bool lead = (tile == 0 && g == 0 && tid == 0);
  const bool live = ok && tile0 < n;
  const long pos = n - 1;
  const bool owner = live && decode && (pos - tile0 < kTipTokens);

  // The head's planes, all in flight (empty ranges past its list, past n,
  // and for a workgroup with nothing to score).
  const int left = live ? ((n + 3) & ~3) - tile0 : 0;
  const int range = left * kPairBytes;
  const uint32_t voff = (uint32_t)lane * 4 * kPairBytes;
  // The tile's first pair in plane 0 of the KV head; plane sl is sl planes
  // further (a 32-bit offset: the launcher checks that it fits).
  const char* kvb = static_cast<const char*>(sidecar) +
                    (plane0 * (size_t)cap + (size_t)tile0) * kPairBytes;
  const uint32_t plane_bytes = (uint32_t)cap * kPairBytes;
  uint4 xa[PW], xb[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    const int sl = hf[k].y;
    const bool valid = sl >= 0;
    const char* base = kvb + (valid ? (uint32_t)sl * plane_bytes : 0u);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base), (short)0, valid ? range : 0, kBufferRsrcWord3);
    const auto va = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    xa[k] = make_uint4(va[0], va[1], va[2], va[3]);
    if constexpr (!BF16) {
      const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, 0, 0);
      xb[k] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
    }
  }

  __builtin_amdgcn_sched_barrier(0);

  // Rotation of FC c at position n - 1 in fp64 (q~ kept in fp32: each
  // component within half an fp32 ulp of its own value, which a sine and
  // cosine taken in fp32 would not keep for a component that the rotation
  // nearly cancels).
  const bool pass = om == 0.0;
  const double qx0 = to_f64(qr0), qx1 = to_f64(qr1);
  const double ang = (double)pos * om;
  double sn, cs;
  sincos(ang, &sn, &cs);
  const float qy0 = (float)(pass ? qx0 : qx0 * cs - qx1 * sn);
  const float qy1 = (float)(pass ? qx1 : qx1 * cs + qx0 * sn);
  // The tile holding the step's position rotates the step's key too, in
  // every wave: lane c holds FC c's rotated pair, which the sums below read
  // by readlane (no LDS, no barrier).
  uint2 own_bits = make_uint2(0u, 0u);
  if (owner && lane < C) own_bits = rotate_pair<BF16>(to_f64(kr0), to_f64(kr1), sn, cs, pass);
  if (!live) {
    if (lead) {
      nb_out[b] = ok ? n : 0;
      if (!ok && !(mode == kPrologueQueryOnly && v == 0)) raise_flag(err, FASA_DEVFLAG_SEQ_LEN);
    }
    return;
  }

  // The head's weights: the rotated pair of its k-th dominant FC, read from
  // that FC's lane.  For bf16 pairs each weight is split into a high and a
  // low bf16 (w = hi + lo within 2^-18 of w), packed per FC like the pair's
  // (lo, hi) dims, so a token's pair takes two v_dot2_f32_bf16 and no
  // unpacking.
  uint32_t wph = 0u, wpl = 0u;
  if constexpr (BF16) {
    const uint32_t h0 = f32_to_bf16_rne_bits(qy0), h1 = f32_to_bf16_rne_bits(qy1);
    const uint32_t l0 = f32_to_bf16_rne_bits(qy0 - __uint_as_float(h0 << 16));
    const uint32_t l1 = f32_to_bf16_rne_bits(qy1 - __uint_as_float(h1 << 16));
    wph = h0 | (h1 << 16);
    wpl = l0 | (l1 << 16);
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool pos_lane = lane == (int)((pos - tile0) >> 2);
  const int pos_t = (int)(pos & 3);
  auto sums = [&](auto own) {
    constexpr bool OWN = decltype(own)::value;
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int fc = hf[k].x, sl = hf[k].y;
      if (sl < 0) break;
      uint4 da = xa[k], db = xb[k];
      if constexpr (OWN) {
        const uint2 p = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)own_bits.x, fc),
                                   (uint32_t)__builtin_amdgcn_readlane((int)own_bits.y, fc));
        if constexpr (BF16) {
          da.x = (pos_lane && pos_t == 0) ? p.x : da.x;
          da.y = (pos_lane && pos_t == 1) ? p.x : da.y;
          da.z = (pos_lane && pos_t == 2) ? p.x : da.z;
          da.w = (pos_lane && pos_t == 3) ? p.x : da.w;
        } else {
          da.x = (pos_lane && pos_t == 0) ? p.x : da.x;
          da.y = (pos_lane && pos_t == 0) ? p.y : da.y;
          da.z = (pos_lane && pos_t == 1) ? p.x : da.z;
          da.w = (pos_lane && pos_t == 1) ? p.y : da.w;
          db.x = (pos_lane && pos_t == 2) ? p.x : db.x;
          db.y = (pos_lane && pos_t == 2) ? p.y : db.y;
          db.z = (pos_lane && pos_t == 3) ? p.x : db.z;
          db.w = (pos_lane && pos_t == 3) ? p.y : db.w;
        }
      }
      if constexpr (BF16) {
        const uint32_t wh = (uint32_t)__builtin_amdgcn_readlane((int)wph, fc);
        const uint32_t wl = (uint32_t)__builtin_amdgcn_readlane((int)wpl, fc);
        const uint32_t wd[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = tip_dot2(wh, wd[t], tip_dot2(wl, wd[t], acc[t]));
      } else {
        const float wx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qy0), fc));
        const float wy = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qy1), fc));
        const float lo[4] = {__uint_as_float(da.x), __uint_as_float(da.z), __uint_as_float(db.x),
                             __uint_as_float(db.z)};
        const float hi[4] = {__uint_as_float(da.y), __uint_as_float(da.w), __uint_as_float(db.y),
                             __uint_as_float(db.w)};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = fmaf(wy, hi[t], fmaf(wx, lo[t], acc[t]));
      }
    }
  };
  if (owner)
    sums(std::true_type{});
  else
    sums(std::false_type{});

  // Stores: the lane's 4 scores, the group maxima, the rotated query (tile 0),
  // the step's K, V and sidecar pairs (owner tile), the length.
  const int j = tile0 + lane * 4;
  float* dst = scores + ((size_t)b * hq + h) * cap + j;
  const float4 s4 = make_float4(acc[0], acc[1], acc[2], acc[3]);
  if (j + 4 <= n) {
    *reinterpret_cast<float4*>(dst) = s4;
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (j + t < n) dst[t] = acc[t];
  }
  if (gmax != nullptr) {
    uint32_t km = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t kk = score_key(acc[t]);
      km = max(km, (j + t < n) ? (kk ? kk : 1u) : 0u);
    }
    km = max(km, dpp_u32<0xB1>(km));  // quad_perm [1,0,3,2]
    km = max(km, dpp_u32<0x4E>(km));  // quad_perm [2,3,0,1]: the quad's maximum
    if ((lane & 3) == 0 && j < n)
      gmax[((size_t)b * hq + h) * gstride + (size_t)(j / kGroupTokens)] = km;
  }
  if (tile == 0 && lane < C) {
    float* qr = qrot + ((size_t)b * hq + h) * D;
    qr[fc_lo(c, R)] = qy0;
    qr[fc_hi(c, R, C)] = qy1;
  }
  if (owner && wave == 0 && lane < C) {
    const size_t dst_kv = (((size_t)b * hkv + g) * cap + pos) * D;
    store_fc_pair<BF16>(own_bits, vr0, vr1, static_cast<T*>(k_cache) + dst_kv,
                        static_cast<T*>(v_cache) + dst_kv, sidecar, plane0, slot_c,
                        fc_lo(c, R), fc_hi(c, R, C), cap, pos);
  }
  if (lead) nb_out[b] = n;
}

template <bool BF16, int G, int D>
static void launch_tip_t(dim3 grid, hipStream_t s, int mode, const PlaneOffsets& po,
                         const TipArgs& a, const fasa_ctx* c, int32_t* nb, float* qrot,
                         float* scores, uint32_t* err, uint32_t* gmax) {
#define FASA_TIP(PWV)                                                                          \
  hipLaunchKernelGGL((tip_kernel<BF16, G, D, PWV>), grid, dim3(kTipThreads), 0, s, a.seq_lens, \
                     a.sidecar, mode, a.max_seq_len, c->cap, c->P, c->R, c->hkv, a.q,          \
                     c->tab.omega, c->tab.fc_slot, c->tab.dom_mask, a.k_new, a.v_new,          \
                     a.k_cache, a.v_cache, nb, qrot, scores, err, po, gmax, c->ws.gstride)
  if constexpr (G == 4 || G == 8) {
    if (c->F <= kHeadPlanes &&
        (unsigned long long)c->max_union * (unsigned long long)c->cap * (BF16 ? 4u : 8u) <
            (1ull << 32)) {
#define FASA_TIP_HEAD(PWV)                                                                   \
  hipLaunchKernelGGL((tip_head_kernel<BF16, G, D, PWV>), grid, dim3(G * kWave), 0, s,        \
                     a.seq_lens, a.sidecar, c->tab.head_fc, mode, a.max_seq_len, c->cap, c->P, \
                     c->R, c->hkv, a.q, c->tab.omega, c->tab.fc_slot, a.k_new, a.v_new,        \
                     a.k_cache, a.v_cache, nb, qrot, scores, err, po, gmax, c->ws.gstride)
      if (c->F <= 4) FASA_TIP_HEAD(4);
      else if (c->F <= 8) FASA_TIP_HEAD(8);
      else if (c->F <= 12) FASA_TIP_HEAD(12);
      else FASA_TIP_HEAD(16);
#undef FASA_TIP_HEAD
      return;
    }
  }
  // Loads per wave: the largest union over the KV heads, 4 planes per step.
  const int pw = (c->max_union + kTipWaves - 1) / kTipWaves;
  if (pw <= 4) FASA_TIP(4);
  else if (pw <= 8) FASA_TIP(8);
  else if (pw <= 12) FASA_TIP(12);
  else FASA_TIP(16);
#undef FASA_TIP
}

template <int G>
static void launch_tip_g(dim3 grid, hipStream_t s, int mode, const PlaneOffsets& po,
                         const TipArgs& a, const fasa_ctx* c, int32_t* nb, float* qrot,
                         float* scores, uint32_t* err, uint32_t* tc) {
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_tip_t<true, G, 128>(grid, s, mode, po, a, c, nb, qrot, scores, err, tc);
    else launch_tip_t<false, G, 128>(grid, s, mode, po, a, c, nb, qrot, scores, err, tc);
  } else {
    if (bf) launch_tip_t<true, G, 64>(grid, s, mode, po, a, c, nb, qrot, scores, err, tc);
    else launch_tip_t<false, G, 64>(grid, s, mode, po, a, c, nb, qrot, scores, err, tc);
  }
}

hipError_t launch_tip(const fasa_ctx* c, PrologueMode mode, const TipArgs& a, float* scores,
                      uint8_t* ws, hipStream_t s, uint32_t* group_max) {
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
    case 1: launch_tip_g<1>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err, group_max); break;
    case 2: launch_tip_g<2>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err, group_max); break;
    case 4: launch_tip_g<4>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err, group_max); break;
    case 8: launch_tip_g<8>(grid, s, (int)mode, po, a, c, nb, qrot, scores, err, group_max); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fasa
