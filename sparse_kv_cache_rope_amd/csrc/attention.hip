// FAC (sparse attention over the selected rows) and the dense full-KV decode
// comparator, both split-K with an online-softmax merge.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC second and third bullets: full attention is executed only
// over the selected tokens, whose keys keep their original absolute
// positions (the cache already holds them rotated).  The dense kernel is the
// full-KV baseline the pages compare against (same page, section 4).
//
// Rows are gathered 16 bytes per lane (attention_common.hpp).  A head whose
// work spans several workgroups writes
// per-split partials that a separate small kernel merges: no workgroup waits
// on another.  Selection is per query head, so a workgroup's rows form a
// gather, not a dense tile: this stays on VALU and is bound by bytes moved.

#include "attention_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

// ---------------------------------------------------------------- FAC ----

// One workgroup per (b, query head h, split); split s covers idx entries
// [s * kFacSplitRows, ...) of the first min(budget, n_b).
//
// The grid is 1-D.  Workgroups are dealt to the 8 XCDs by linear id mod 8 and
// each XCD has its own L2.  The G query heads of one KV group gather, at the
// same split, rows from the same stretch of positions (each head's indices are
// ascending), and some of the same rows.  So the tuple t = (b, g, split) and
// its G heads take the ids ((t / 8) * G + h % G) * 8 + t % 8: one XCD, back to
// back in dispatch order.  Ids whose t is past the last tuple exit.
template <bool BF16, int D>
__global__ void __launch_bounds__(kFacThreads)
fac_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
           const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
           const int32_t* __restrict__ idx, int budget, int splits, int batch, int hq, int hkv,
           int G, int cap, float* __restrict__ partial, int max_splits, float* __restrict__ out,
           uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = kFacThreads / kWave;
  constexpr int ITERS = kFacSplitRows / (RS * NW);
  static_assert(ITERS >= 1 && ITERS * RS * NW == kFacSplitRows, "split geometry");
  __shared__ float lds[NW * (D + 2 * LPR)];

  const int id = blockIdx.x, round = id >> 3;
  const int t = (round / G) * 8 + (id & 7);
  if (t >= splits * hkv * batch) return;
  const int split = t % splits, g = (t / splits) % hkv, b = t / (splits * hkv);
  const int h = g * G + round % G;
  const size_t row = (size_t)b * hq + h;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;

  // The split's indices and the query are loaded before n_b is known (an idx
  // row is `budget` wide whatever n_b is), so their round trip overlaps the
  // length's instead of following it.
  const int32_t* ids = idx + row * budget + (size_t)split * kFacSplitRows;
  const int in_row = min(kFacSplitRows, budget - split * kFacSplitRows);
  int jr[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * RS * NW + wave * RS + slot;
    jr[it] = (r < in_row) ? ids[r] : -1;
  }
  const float scale = logit_scale<D>();
  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = qrot[row * D + sub * EPL + e] * scale;

  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int take = n < budget ? n : budget;
  const int nsplit = (take + kFacSplitRows - 1) / kFacSplitRows;
  float* o = out + row * D;
  if (nsplit == 0) {
    if (split == 0)
      for (int d = threadIdx.x; d < D; d += kFacThreads) o[d] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int rows_here = min(kFacSplitRows, take - split * kFacSplitRows);

  uint4 kc[ITERS], vc[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = it * RS * NW + wave * RS + slot;
    int j = (r < rows_here) ? jr[it] : -1;
    if (j >= n) {
      if (sub == 0) raise_flag(err, FASA_DEVFLAG_INDEX);
      j = -1;
    }
    jr[it] = j;
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    if (jr[it] >= 0) {
      const size_t off = (kvbase + jr[it]) * LPR + sub;
      kc[it] = K[off];
      vc[it] = V[off];
    } else {
      kc[it] = make_uint4(0, 0, 0, 0);
      vc[it] = make_uint4(0, 0, 0, 0);
    }
  }
  Soft<EPL> st;
  st.init();
  float z[ITERS], vf[ITERS][EPL];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float kf[EPL];
    unpack<BF16, EPL>(kc[it], kf);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s = fmaf(qv[e], kf[e], s);
    s = group_sum<LPR>(s);
    z[it] = jr[it] >= 0 ? s : -INFINITY;
    unpack<BF16, EPL>(vc[it], vf[it]);
  }
  st.template add_batch<ITERS>(z, vf);
  merge_block<D, LPR, EPL, NW>(st, lds);
  write_state<D, LPR, EPL>(st, nsplit == 1, o,
                           partial + (row * max_splits + split) * (D + 2));
}

// -------------------------------------------------------------- dense ----

constexpr int kDenseThreads = 512;
// Query heads a dense workgroup holds softmax states for.
constexpr int kDenseHeads = 2;

// One workgroup per (b, KV head g, split, group of HPW of g's query heads);
// split s covers tokens [s * kDenseSplitTokens, ...).  Fewer heads per
// workgroup than G keep the per-lane softmax states few enough for two
// workgroups per CU; the NG = G / HPW workgroups of one (b, g, split) read
// the same K/V rows, so they take ids on one XCD back to back (the FAC
// kernel's order: ((t / 8) * NG + head group) * 8 + t % 8 for tuple t) and
// all but the first find the rows in that XCD's L2.
template <bool BF16, int D, int HPW>
__global__ void __launch_bounds__(kDenseThreads)
dense_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
             const float* __restrict__ qrot, const int32_t* __restrict__ nb, int max_seq_len,
             int hq, int hkv, int cap, int splits, int batch, int groups,
             float* __restrict__ partial, int max_splits, float* __restrict__ out,
             uint32_t* err) {
  using Geo = RowGeom<BF16, D>;
  constexpr int LPR = Geo::LPR, EPL = Geo::EPL, RS = Geo::RS, NW = kDenseThreads / kWave;
  constexpr int ITERS = kDenseSplitTokens / (RS * NW);
  constexpr int BATCH = 4;
  static_assert(ITERS % BATCH == 0 && ITERS * RS * NW == kDenseSplitTokens, "split geometry");
  __shared__ float lds[NW * (D + 2 * LPR)];

  const int id = blockIdx.x, round = id >> 3;
  const int tt = (round / groups) * 8 + (id & 7);
  if (tt >= splits * hkv * batch) return;
  const int split = tt % splits, g = (tt / splits) % hkv, b = tt / (splits * hkv);
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  const int nsplit = (n + kDenseSplitTokens - 1) / kDenseSplitTokens;
  const size_t row0 = (size_t)b * hq + (size_t)g * (HPW * groups) + (size_t)(round % groups) * HPW;
  if (nsplit == 0) {
    if (split == 0)
      for (int i = threadIdx.x; i < HPW * D; i += kDenseThreads) out[row0 * D + i] = 0.0f;
    return;
  }
  if (split >= nsplit) return;

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int slot = lane / LPR, sub = lane % LPR;
  const float scale = logit_scale<D>();
  float qv[HPW][EPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[hh][e] = qrot[(row0 + hh) * D + sub * EPL + e] * scale;

  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int t0 = split * kDenseSplitTokens;

  Soft<EPL> st[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) st[hh].init();
  // Batches of BATCH rows per row slot, double-buffered: the next batch's
  // loads are issued before the current batch is used, so every workgroup
  // keeps loads in flight while it computes.  Rows past n read row 0 and are
  // masked.
  auto load = [&](int i0, uint4 (&kc)[BATCH], uint4 (&vc)[BATCH]) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int j = t0 + (i0 + i) * RS * NW + wave * RS + slot;
      const size_t off = (kvbase + (j < n ? j : 0)) * LPR + sub;
      kc[i] = K[off];
      vc[i] = V[off];
    }
  };
  uint4 kb[2][BATCH], vb[2][BATCH];
  load(0, kb[0], vb[0]);
#pragma unroll
  for (int i0 = 0; i0 < ITERS; i0 += BATCH) {
    const int cur = (i0 / BATCH) & 1;
    if (i0 + BATCH < ITERS) load(i0 + BATCH, kb[cur ^ 1], vb[cur ^ 1]);
    float z[HPW][BATCH], vf[BATCH][EPL];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const bool ok = t0 + (i0 + i) * RS * NW + wave * RS + slot < n;
      float kf[EPL];
      unpack<BF16, EPL>(kb[cur][i], kf);
      unpack<BF16, EPL>(vb[cur][i], vf[i]);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(qv[hh][e], kf[e], s);
        s = group_sum<LPR>(s);
        z[hh][i] = ok ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) st[hh].template add_batch<BATCH>(z[hh], vf);
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    merge_block<D, LPR, EPL, NW>(st[hh], lds);
    write_state<D, LPR, EPL>(st[hh], nsplit == 1, out + (row0 + hh) * D,
                             partial + ((row0 + hh) * max_splits + split) * (D + 2));
  }
}

// ------------------------------------------------------- dense (MFMA) ----

// bf16 caches at d = 128: the dense comparator's q . K is a real contraction
// (the G <= 4 query heads of a workgroup against every key of its split), so
// it runs on the matrix cores: per 16-token tile, D / 32 steps of
// v_mfma_f32_16x16x32_bf16 with the K tile as the A operand (a lane's 16-byte
// load of a K row is its A fragment) and the queries as B: columns h < HPW
// hold head h's scaled q~ rounded to bf16, columns HPW + h the rest of it
// (q~ - hi, rounded again), so a logit is two columns' sum and keeps about
// 2^-16 relative precision.  The softmax weights and P . V stay on VALU.
//
// A wave takes 32 consecutive tokens (2 tiles) of each 256-token chunk of
// the workgroup's split.  With one chunk per workgroup (MULTI false) all its
// K and V loads go out first (113 VGPRs, so two workgroups share a CU and one
// streams while the other computes).  When the grid would not fit the device
// at once, a workgroup walks several chunks (MULTI) with the next chunk's K
// loads issued as soon as this chunk's logits are done and its V loads as
// soon as the weighted V sum is, an online softmax state carried across
// chunks (about 210 VGPRs, one workgroup per CU, one round of workgroups).
// V rows are read 4 per load, lane l holding row l % 4 and dims
// 8 (l / 4) .. 8 (l / 4) + 7, so the sum over a load's rows is a quad
// reduction.  The 8 waves' states merge once through LDS.
typedef __bf16 fasa_bf16x8 __attribute__((ext_vector_type(8)));
typedef float fasa_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDenseMfmaTiles = 2;  // 16-token tiles per wave

__device__ __forceinline__ uint32_t f32_bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

template <int HPW, bool MULTI>
__global__ void __launch_bounds__(kDenseThreads)
dense_mfma_kernel(const void* __restrict__ k_cache, const void* __restrict__ v_cache,
                  const uint16_t* __restrict__ q, const int32_t* __restrict__ seq_lens,
                  const double* __restrict__ omega, int R, int max_seq_len, int hq, int hkv,
                  int cap, int splits, int cpw, int batch, int groups, float* __restrict__ partial,
                  int max_splits, float* __restrict__ out, int32_t* __restrict__ nb_out,
                  uint32_t* err) {
  constexpr int D = 128;
  constexpr int KK = D / 32;                 // MFMA steps over the head dim
  constexpr int NW = kDenseThreads / kWave;  // 8
  constexpr int T = kDenseMfmaTiles;
  static_assert(NW * T * 16 == kDenseSplitTokens, "a split is 8 waves x T tiles of 16 tokens");
  static_assert(2 * HPW <= 16, "hi and lo columns of the B operand");
  __shared__ float pl[NW][T * 16][4];   // a wave's softmax weights, [token][head]
  __shared__ float red[NW][HPW][D];     // the waves' weighted V sums
  __shared__ float mw[NW][HPW], lw[NW][HPW];
  __shared__ float qs[HPW][D];          // the workgroup's rotated queries

  const int id = blockIdx.x, round = id >> 3;
  const int tt = (round / groups) * 8 + (id & 7);
  if (tt >= splits * hkv * batch) return;
  const int split = tt % splits, g = (tt / splits) % hkv, b = tt / (splits * hkv);
  // The length, validated here (one workgroup per sequence records it for
  // the merge and raises the flag): 1 <= n_b <= min(max_seq_len, cap), and
  // n_b = 0 gives a zero output without a flag.
  const int n_in = seq_lens[b];
  const bool len_ok = n_in >= 1 && n_in <= max_seq_len && n_in <= cap;
  const int n = len_ok ? n_in : 0;
  if (split == 0 && g == 0 && round % groups == 0 && threadIdx.x == 0) {
    nb_out[b] = n;
    if (!len_ok && n_in != 0) raise_flag(err, FASA_DEVFLAG_SEQ_LEN);
  }
  const int span = kDenseSplitTokens * cpw;  // tokens of one split: cpw chunks
  const int nsplit = (n + span - 1) / span;
  const size_t row0 = (size_t)b * hq + (size_t)g * (HPW * groups) + (size_t)(round % groups) * HPW;
  // With several splits in the launch every split writes a partial state
  // (an empty one past the row's tokens) and the merge, which then needs no
  // lengths, writes the output.
  if (split >= nsplit) {
    if (splits > 1) {
      for (int i = threadIdx.x; i < HPW * (D + 2); i += kDenseThreads) {
        const int h = i / (D + 2), e = i % (D + 2);
        partial[((row0 + h) * max_splits + split) * (D + 2) + e] = e == 0 ? -INFINITY : 0.0f;
      }
    } else {
      for (int i = threadIdx.x; i < HPW * D; i += kDenseThreads) out[row0 * D + i] = 0.0f;
    }
    return;
  }

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const size_t kvbase = ((size_t)b * hkv + g) * cap;
  const uint4* K = static_cast<const uint4*>(k_cache);
  const uint4* V = static_cast<const uint4*>(v_cache);
  const int t_split = split * span;
  // Chunks of this split that hold tokens (one without MULTI).
  const int nch = MULTI ? min(cpw, (n - t_split + kDenseSplitTokens - 1) / kDenseSplitTokens) : 1;

  // A chunk's K and V loads for this wave (tokens past n read row 0, masked).
  uint4 kr[T][KK], vr[T][4];
  auto issue_k = [&](int ch) {
    const int tw = t_split + ch * kDenseSplitTokens + wave * (T * 16);
#pragma unroll
    for (int j = 0; j < T; ++j) {
      const int tk = tw + 16 * j + lane % 16;
      const size_t kb = (kvbase + (size_t)(tk < n ? tk : 0)) * (D / 8) + lane / 16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kr[j][kk] = K[kb + 4 * kk];
    }
  };
  auto issue_v = [&](int ch) {
    const int tw = t_split + ch * kDenseSplitTokens + wave * (T * 16);
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int tv = tw + 16 * j + 4 * s4 + lane % 4;
        vr[j][s4] = V[(kvbase + (size_t)(tv < n ? tv : 0)) * (D / 8) + lane / 4];
      }
  };
  issue_k(0);
  issue_v(0);

  // The queries, rotated to position n - 1 while the loads fly: one FC pair
  // per thread (angle reduced in fp64, sine and cosine in fp32; the logits
  // then go through bf16 halves on the matrix cores anyway).
  if (threadIdx.x < HPW * (D / 2)) {
    const int hh = threadIdx.x / (D / 2), cf = threadIdx.x % (D / 2);
    const int lo = fc_lo(cf, R), hi = fc_hi(cf, R, D / 2);
    const uint16_t* qh = q + (row0 + hh) * D;
    const float x0 = bf16_bits_to_f32(qh[lo]), x1 = bf16_bits_to_f32(qh[hi]);
    const double w = omega[cf];
    const double rev = (double)(n - 1) * w * 0.15915494309189533577;  // turns
    float sf, cf2;
    sincosf((float)((rev - rint(rev)) * 6.28318530717958647693), &sf, &cf2);
    const bool pass = w == 0.0;
    qs[hh][lo] = pass ? x0 : (float)((double)x0 * cf2 - (double)x1 * sf);
    qs[hh][hi] = pass ? x1 : (float)((double)x1 * cf2 + (double)x0 * sf);
  }
  __syncthreads();

  // B operands: lane l holds column c = l % 16, dims 32 kk + 8 (l / 16) ..
  const int c = lane % 16;
  fasa_bf16x8 qb[KK];
  {
    const bool hi_col = c < HPW, lo_col = c >= HPW && c < 2 * HPW;
    const int hh = hi_col ? c : (lo_col ? c - HPW : 0);
    const float scale = logit_scale<D>();
    const float4* q4 = reinterpret_cast<const float4*>(qs[hh]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = 32 * kk + 8 * (lane / 16);
      const float4 a = q4[d0 / 4], bq = q4[d0 / 4 + 1];
      const float qv[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = qv[i] * scale;
        const uint32_t h16 = f32_bf16_rne_bits(x);
        const uint32_t l16 = f32_bf16_rne_bits(x - __uint_as_float(h16 << 16));
        const uint16_t bits = hi_col ? (uint16_t)h16 : (lo_col ? (uint16_t)l16 : (uint16_t)0);
        qb[kk][i] = __builtin_bit_cast(__bf16, bits);
      }
    }
  }

  // The wave's running state: max m per head (lanes c < HPW; l, l ^ 16,
  // l ^ 32 hold the same head), sum of weights per lane, and the weighted V
  // sums of every head for the lane's dims.
  float m = -INFINITY, lsum = 0.0f;
  float acc_o[HPW][8];
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc_o[h][e] = 0.0f;
  for (int ch = 0; ch < nch; ++ch) {
    const int tw = t_split + ch * kDenseSplitTokens + wave * (T * 16);  // the wave's first token
    // Logits: tile j's D fragment holds tokens 16 j + 4 (l / 16) + i of
    // column c; head c's logit is column c plus column c + HPW (lane l + HPW).
    float z[T][4];
    float mc = -INFINITY;
#pragma unroll
    for (int j = 0; j < T; ++j) {
      fasa_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(fasa_bf16x8, kr[j][kk]),
                                                      qb[kk], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] + dpp_f<0x100 + HPW>(acc[i]);  // row_shl: lane l + HPW
        const int tk = tw + 16 * j + 4 * (lane / 16) + i;
        z[j][i] = (c < HPW && tk < n) ? v : -INFINITY;
        mc = fmaxf(mc, z[j][i]);
      }
    }
    if (MULTI && ch + 1 < nch) issue_k(ch + 1);  // the K registers are free again
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mn = fmaxf(m, mc);
    // The rescale of the state so far (m = -inf gives 0; nothing yet if the
    // new max is -inf too).
    const float own_sc = mn == -INFINITY ? 1.0f : exp2f(m - mn);
    m = mn;
    lsum *= own_sc;
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = mn == -INFINITY ? 0.0f : exp2f(z[j][i] - mn);  // -inf gives 0
        lsum += p;
        if (c < HPW) pl[wave][16 * j + 4 * (lane / 16) + i][c] = p;
      }
    // The wave reads back what its own lanes wrote (LDS keeps a wave's
    // accesses in order); the barrier only stops the compiler moving them.
    __builtin_amdgcn_wave_barrier();
    if (MULTI) {
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(own_sc), h));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc_o[h][e] *= sc;
      }
    }
    // Weighted V: lane l adds rows 16 j + 4 s + l % 4, dims 8 (l / 4) ...
#pragma unroll
    for (int j = 0; j < T; ++j)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float4 p4 = *reinterpret_cast<const float4*>(pl[wave][16 * j + 4 * s4 + lane % 4]);
        const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
        float vf[8];
        unpack<true, 8>(vr[j][s4], vf);
#pragma unroll
        for (int h = 0; h < HPW; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc_o[h][e] = fmaf(pv[h], vf[e], acc_o[h][e]);
      }
    if (MULTI && ch + 1 < nch) issue_v(ch + 1);  // the V registers are free again
    __builtin_amdgcn_wave_barrier();              // pl is rewritten by the next chunk
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (lane < HPW) {
    mw[wave][lane] = m;
    lw[wave][lane] = lsum;
  }
#pragma unroll
  for (int h = 0; h < HPW; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc_o[h][e];
      v += dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
      v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
      acc_o[h][e] = v;
    }
  if (lane % 4 == 0) {
#pragma unroll
    for (int h = 0; h < HPW; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][h][8 * (lane / 4) + e] = acc_o[h][e];
  }
  __syncthreads();

  // The 8 wave states of each head merged: thread (h, d).
  for (int t = threadIdx.x; t < HPW * D; t += kDenseThreads) {
    const int h = t / D, d = t % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, mw[w][h]);
    float L = 0.0f, S = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = mx == -INFINITY ? 0.0f : exp2f(mw[w][h] - mx);  // -inf gives 0
      L = fmaf(lw[w][h], wt, L);
      S = fmaf(red[w][h][d], wt, S);
    }
    if (splits == 1) {
      out[(row0 + h) * D + d] = L > 0.0f ? S / L : 0.0f;
    } else {
      float* part = partial + ((row0 + h) * max_splits + split) * (D + 2);
      if (d == 0) {
        part[0] = mx;
        part[1] = L;
      }
      part[2 + d] = S;
    }
  }
}

// -------------------------------------------------------------- merge ----

// The merge of per-split partials (m, l, acc) of the rows whose work spanned
// more than one split.  `unit` is the rows (FAC: of min(budget, n)) or tokens
// (dense: of n) per split; with `fixed_splits` > 0 every split of every row
// wrote a state (an empty one past the row) and no length is read.
//
// A 256-thread workgroup covers a 16-dim slice of 16 / SL rows: thread t takes
// dim t % 16 of the slice, split lane (t / 16) % SL and row t / (16 SL), and
// folds splits lane, lane + SL, .. (up to 8 loads in flight) into a state of
// its own; sixteen threads read one split's 64 contiguous bytes.  The SL
// states of a (row, dim) then merge through LDS.  SL is the launch's split
// count rounded up to a power of two, at most 16, so a grid of many rows with
// few splits packs several rows per workgroup and one of few rows with
// hundreds of splits still keeps every load of a lane in flight.
constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 16;

struct MergeState {
  float m, l, a;
};

// The merge of two softmax states; a state with m = -inf is empty.
__device__ __forceinline__ MergeState merge_states(MergeState x, MergeState y) {
  const float mn = fmaxf(x.m, y.m);
  if (mn == -INFINITY) return x;
  const float wx = exp2f(x.m - mn), wy = exp2f(y.m - mn);  // -inf gives 0
  return {mn, fmaf(x.l, wx, y.l * wy), fmaf(x.a, wx, y.a * wy)};
}

template <int D, int SL>
__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ partial, int max_splits, const int32_t* __restrict__ nb,
             int max_seq_len, int cap, int budget, int unit, int hq, int rows, int fixed_splits,
             float* __restrict__ out) {
  constexpr int RPW = kMergeDims / SL;  // rows per workgroup
  constexpr int SLICES = D / kMergeDims;
  constexpr int U = 8;  // splits per lane in flight
  static_assert(RPW * SL * kMergeDims == kMergeThreads, "thread layout");
  __shared__ MergeState ws[kMergeThreads];
  const int t = threadIdx.x;
  const int dd = t % kMergeDims, sl = (t / kMergeDims) % SL;
  const int row = (int)(blockIdx.x / SLICES) * RPW + t / (kMergeDims * SL);
  const int d = (int)(blockIdx.x % SLICES) * kMergeDims + dd;
  int nsplit = 0;
  if (row < rows) {
    nsplit = fixed_splits;
    if (fixed_splits == 0) {
      int n = nb[row / hq];
      if (n < 0 || n > max_seq_len || n > cap) n = 0;
      const int work = (budget > 0 && budget < n) ? budget : n;
      nsplit = (work + unit - 1) / unit;  // <= 1: written directly by the split kernel
    }
  }
  MergeState st = {-INFINITY, 0.0f, 0.0f};
  if (nsplit > 1) {
    const float* p = partial + (size_t)row * max_splits * (D + 2);
    for (int s0 = sl; s0 < nsplit; s0 += U * SL) {
      float mv[U], lv[U], av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sp = s0 + u * SL;
        const float* q = p + (size_t)(sp < nsplit ? sp : s0) * (D + 2);
        mv[u] = sp < nsplit ? q[0] : -INFINITY;
        lv[u] = q[1];
        av[u] = q[2 + d];
      }
      float mx = st.m;
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, mv[u]);
      if (mx != -INFINITY) {
        const float sc = exp2f(st.m - mx);  // -inf gives 0
        st.l *= sc;
        st.a *= sc;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float w = exp2f(mv[u] - mx);  // -inf gives 0
          st.l = fmaf(lv[u], w, st.l);
          st.a = fmaf(av[u], w, st.a);
        }
        st.m = mx;
      }
    }
  }
  ws[t] = st;
  __syncthreads();
  if (sl == 0 && nsplit > 1) {
#pragma unroll
    for (int k = 1; k < SL; ++k) st = merge_states(st, ws[t + k * kMergeDims]);
    out[(size_t)row * D + d] = (st.l > 0.0f) ? st.a / st.l : 0.0f;
  }
}

// ------------------------------------------------------------ launchers --

// max_splits_used: the most splits any row of this launch can have.
static void launch_merge(const fasa_ctx* c, const float* part, int max_splits, const int32_t* nb,
                         int max_seq_len, int budget, int unit, float* out, hipStream_t s,
                         int fixed_splits = 0) {
  const int work_max = (budget > 0 && budget < max_seq_len) ? budget : max_seq_len;
  const int used = fixed_splits > 0 ? fixed_splits : (work_max + unit - 1) / unit;
  const int rows = c->batch * c->hq;
  const int slices = c->d / kMergeDims;
#define FASA_MERGE(DD, SLV)                                                                  \
  hipLaunchKernelGGL((merge_kernel<DD, SLV>),                                                 \
                     dim3((unsigned)(((rows + kMergeDims / SLV - 1) / (kMergeDims / SLV)) *   \
                                     slices)),                                                \
                     dim3(kMergeThreads), 0, s, part, max_splits, nb, max_seq_len, c->cap,    \
                     budget, unit, c->hq, rows, fixed_splits, out)
#define FASA_MERGE_D(DD)             \
  if (used <= 2) FASA_MERGE(DD, 2);  \
  else if (used <= 4) FASA_MERGE(DD, 4); \
  else if (used <= 8) FASA_MERGE(DD, 8); \
  else FASA_MERGE(DD, 16);
  if (c->d == 128) {
    FASA_MERGE_D(128)
  } else {
    FASA_MERGE_D(64)
  }
#undef FASA_MERGE_D
#undef FASA_MERGE
}

hipError_t launch_fac(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                      const int32_t* nb, int max_seq_len, const int32_t* idx, int budget,
                      float* out, uint8_t* ws, hipStream_t s) {
  const int take = budget < max_seq_len ? budget : max_seq_len;
  int splits = (take + kFacSplitRows - 1) / kFacSplitRows;
  if (splits < 1) splits = 1;
  // (b, g, split) tuples rounded up to whole rounds of 8 XCDs, G heads each.
  const long tuples = (long)splits * c->hkv * c->batch;
  const dim3 grid((unsigned)((tuples + 7) / 8 * 8 * c->G));
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.fac);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
#define FASA_FAC(BF, DD)                                                                      \
  hipLaunchKernelGGL((fac_kernel<BF, DD>), grid, dim3(kFacThreads), 0, s, k_cache, v_cache, qrot, \
                     nb, max_seq_len, idx, budget, splits, c->batch, c->hq, c->hkv, c->G,      \
                     c->cap, part, c->ws.fac_splits, out, err)
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) FASA_FAC(true, 128); else FASA_FAC(false, 128);
  } else {
    if (bf) FASA_FAC(true, 64); else FASA_FAC(false, 64);
  }
#undef FASA_FAC
  if (splits > 1)
    launch_merge(c, part, c->ws.fac_splits, nb, max_seq_len, budget, kFacSplitRows, out, s);
  return hipGetLastError();
}

// The dense call on bf16 caches at d = 128: one launch that validates the
// lengths and rotates the queries itself, then the merge of its splits.
hipError_t launch_dense_fused(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                              const void* q, const int32_t* seq_lens, int max_seq_len,
                              float* out, uint8_t* ws, hipStream_t s) {
  if (c->dtype != FASA_BF16 || c->d != 128) return hipErrorInvalidValue;
  // Query heads per workgroup: all of the group's, at most 4.
  const int hpw = c->G < 4 ? c->G : 4;
  const int groups = c->G / hpw;
  // 256-token chunks per workgroup: one while the grid fits two workgroups
  // per CU at once; else enough that it fits one per CU (a workgroup that
  // walks several chunks keeps the next chunk's loads in flight and holds
  // about 210 VGPRs).
  const int chunks = max(1, (max_seq_len + kDenseSplitTokens - 1) / kDenseSplitTokens);
  const long per_split = (long)c->hkv * c->batch * groups;
  const long cus = c->cus > 0 ? c->cus : 256;
  int cpw = 1;
  if ((long)chunks * per_split > 2 * cus)
    cpw = (int)std::min<long>(chunks, ((long)chunks * per_split + cus - 1) / cus);
  const int splits = (chunks + cpw - 1) / cpw;
  float* part = reinterpret_cast<float*>(ws + c->ws.dense);
  int32_t* nb = reinterpret_cast<int32_t*>(ws + c->ws.nb);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const long tuples = (long)splits * c->hkv * c->batch;
  const long ids = (tuples + 7) / 8 * 8 * groups;
  if (ids * kDenseThreads > 0xffffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)ids);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
#define FASA_DENSE_MFMA(GG, MM)                                                             \
  hipLaunchKernelGGL((dense_mfma_kernel<GG, MM>), grid, dim3(kDenseThreads), 0, s, k_cache,    \
                     v_cache, qb, seq_lens, c->tab.omega, c->R, max_seq_len, c->hq, c->hkv,    \
                     c->cap, splits, cpw, c->batch, groups, part, c->ws.dense_splits, out, nb, \
                     err)
  if (cpw == 1) {
    if (hpw == 1) FASA_DENSE_MFMA(1, false);
    else if (hpw == 2) FASA_DENSE_MFMA(2, false);
    else FASA_DENSE_MFMA(4, false);
  } else {
    if (hpw == 1) FASA_DENSE_MFMA(1, true);
    else if (hpw == 2) FASA_DENSE_MFMA(2, true);
    else FASA_DENSE_MFMA(4, true);
  }
#undef FASA_DENSE_MFMA
  if (splits > 1)
    launch_merge(c, part, c->ws.dense_splits, nb, max_seq_len, 0, kDenseSplitTokens * cpw, out,
                 s, splits);
  return hipGetLastError();
}

template <bool BF, int DD>
static bool launch_dense_g(const fasa_ctx* c, int splits, hipStream_t s, const void* k_cache,
                           const void* v_cache, const float* qrot, const int32_t* nb,
                           int max_seq_len, float* part, float* out, uint32_t* err) {
  // Query heads per workgroup: at most kDenseHeads.
  const int hpw = c->G < kDenseHeads ? c->G : kDenseHeads;
  const int groups = c->G / hpw;
  const long tuples = (long)splits * c->hkv * c->batch;
  const long ids = (tuples + 7) / 8 * 8 * groups;
  if (ids * kDenseThreads > 0xffffffffL) {
    (void)hipGetLastError();
    return false;
  }
  const dim3 grid((unsigned)ids);
#define FASA_DENSE(GG)                                                                          \
  hipLaunchKernelGGL((dense_kernel<BF, DD, GG>), grid, dim3(kDenseThreads), 0, s, k_cache,       \
                     v_cache, qrot, nb, max_seq_len, c->hq, c->hkv, c->cap, splits, c->batch,    \
                     groups, part, c->ws.dense_splits, out, err)
  if (hpw == 1) FASA_DENSE(1);
  else if (hpw == 2) FASA_DENSE(2);
  else FASA_DENSE(4);
#undef FASA_DENSE
  return true;
}

hipError_t launch_dense(const fasa_ctx* c, const void* k_cache, const void* v_cache,
                        const int32_t* nb, int max_seq_len, float* out, uint8_t* ws,
                        hipStream_t s) {
  int splits = (max_seq_len + kDenseSplitTokens - 1) / kDenseSplitTokens;
  if (splits < 1) splits = 1;
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  float* part = reinterpret_cast<float*>(ws + c->ws.dense);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const bool bf = (c->dtype == FASA_BF16);
  bool launched;
  if (c->d == 128) {
    launched = bf ? launch_dense_g<true, 128>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err)
                  : launch_dense_g<false, 128>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err);
  } else {
    launched = bf ? launch_dense_g<true, 64>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err)
                  : launch_dense_g<false, 64>(c, splits, s, k_cache, v_cache, qrot, nb, max_seq_len, part, out, err);
  }
  // A grid past one 1-D launch (2^32 work items) is refused before launching.
  if (!launched) return hipErrorInvalidConfiguration;
  if (splits > 1)
    launch_merge(c, part, c->ws.dense_splits, nb, max_seq_len, 0, kDenseSplitTokens, out, s);
  return hipGetLastError();
}

}  // namespace fasa
