// Two-stage top-B selection with FAC fused into the second stage.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC bullets: select the critical token set T_t from the TIP
// scores, then run full attention over T_t only.  Same selection as the
// one-stage kernels (topk.hip): the min(B, n) highest scores, equal scores to
// the lower position, ascending; exact radix select on 64-bit composites
// (select_common.hpp).
//
// A single workgroup cannot stream a 32k-token row of scores quickly enough
// (each dependent pass costs a memory round trip), and workgroups of one
// row must not wait on each other (device-wide hand-offs are expensive on a
// multi-die GPU).  So the row is cut into chunks of 4096 positions:
//   stage 1 (chunk_select_kernel): one 1024-thread workgroup per chunk keeps
//     the chunk's scores in registers (4 per thread, one round trip) and
//     writes the chunk's own top-B composites, ascending.  The row's top B
//     are among these candidates.
//   stage 2 (final_select_kernel): one 1024-thread workgroup per row loads
//     all candidates at once (<= 8192, ascending across chunks), selects the
//     row's top B among them, writes idx, keeps the positions in LDS and runs
//     FAC over them.
// A row of at most one chunk skips stage 1: stage 2 reads its scores directly.

#include "attention_common.hpp"
#include "fasa_internal.hpp"
#include "select_common.hpp"

namespace fasa {

// Many waves with few elements each: a wave's instructions form a dependent
// chain, so the work per wave, not the thread count, sets the latency.
constexpr int kChunkThreads = 1024;
constexpr int kChunkE = kTwoStageChunk / kChunkThreads;  // 4 scores per thread
constexpr int kFinalThreads = 1024;
constexpr int kFinalE = kTwoStageMaxCand / kFinalThreads;  // 8 candidates per thread

using ChunkLds = RegSelectLds<kChunkThreads, 8, 1024>;

struct FinalLds {
  RegSelectLds<kFinalThreads, 8, 4096> s;
  int32_t sel[kFusedMaxBudget];
};

__device__ __forceinline__ int chunks_of(int n) { return (n + kTwoStageChunk - 1) / kTwoStageChunk; }

// Candidates stage 1 leaves for a row of n > budget positions.
__device__ __forceinline__ int candidates_of(int n, int budget) {
  const int nch = chunks_of(n);
  const int last = n - (nch - 1) * kTwoStageChunk;
  return (nch - 1) * budget + (last < budget ? last : budget);
}

__global__ void __launch_bounds__(kChunkThreads)
chunk_select_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                    int max_seq_len, int hq, int cap, int budget, uint64_t* __restrict__ cand,
                    int cand_stride) {
  __shared__ ChunkLds L;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  int n = nb[b];
  if (n < 0 || n > max_seq_len || n > cap) n = 0;
  const int nch = chunks_of(n);
  if (n <= budget || nch <= 1 || chunk >= nch) return;
  const int c0 = chunk * kTwoStageChunk;
  const int cn = min(kTwoStageChunk, n - c0);
  const float* __restrict__ src = scores + row * cap + c0;
  const int t = threadIdx.x;

  // Slab i holds positions c0 + i * 4 * kChunkThreads + 4t .. +3 (coalesced
  // float4 loads).
  uint64_t cv[kChunkE];
  uint32_t vmask = 0;
#pragma unroll
  for (int i = 0; i < kChunkE / 4; ++i) {
    const int o = i * 4 * kChunkThreads + 4 * t;
    float v[4];
    if (o + 4 <= cn) {
      const float4 x = *reinterpret_cast<const float4*>(src + o);
      v[0] = x.x;
      v[1] = x.y;
      v[2] = x.z;
      v[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (o + e < cn) ? src[o + e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cv[4 * i + e] = composite(score_key(v[e]), (uint32_t)(c0 + o + e));
      vmask |= (o + e < cn ? 1u : 0u) << (4 * i + e);
    }
  }
  const uint64_t tau =
      (cn > budget) ? reg_select<kChunkThreads, kChunkE>(cv, vmask, (uint32_t)budget, L) : 0ull;
  uint64_t* out = cand + row * cand_stride + (size_t)chunk * budget;
  uint32_t m4[kChunkE / 4], off[kChunkE / 4];
#pragma unroll
  for (int i = 0; i < kChunkE / 4; ++i) {
    m4[i] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m4[i] |= ((((vmask >> (4 * i + e)) & 1u) && cv[4 * i + e] >= tau) ? 1u : 0u) << e;
  }
  ordered_offsets<kChunkThreads>(m4, off, L);
#pragma unroll
  for (int i = 0; i < kChunkE / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((m4[i] >> e) & 1u) {
        if (off[i] < (uint32_t)budget) out[off[i]] = cv[4 * i + e];
        ++off[i];
      }
}

template <bool ATTEND, bool BF16, int D>
__global__ void __launch_bounds__(kFinalThreads)
final_select_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                    int max_seq_len, int hq, int cap, int budget,
                    const uint64_t* __restrict__ cand, int cand_stride, int32_t* __restrict__ idx,
                    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
                    const float* __restrict__ qrot, int hkv, int G, float* __restrict__ out,
                    int32_t* __restrict__ advance, uint32_t* err) {
  __shared__ FinalLds L;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t row = (size_t)b * hq + h;
  const int n = checked_len(nb, b, max_seq_len, cap, err, h == 0 && threadIdx.x == 0);
  if (advance != nullptr && h == 0 && threadIdx.x == 0 && n > 0) advance[b] = n;
  const int t = threadIdx.x;
  int32_t* o = idx ? idx + row * budget : nullptr;
  const int take = n < budget ? n : budget;

  if (n <= budget) {
    for (int j = t; j < budget; j += kFinalThreads) {
      if (o) o[j] = (j < n) ? j : -1;
      if (ATTEND && j < kFusedMaxBudget) L.sel[j] = j;
    }
  } else {
    // Candidate k = 4 (g * kFinalThreads + t) + e: group g holds 4 consecutive
    // candidates per thread; k ascends with position.
    const bool direct = chunks_of(n) <= 1;
    const int M = direct ? n : candidates_of(n, budget);
    uint64_t cv[kFinalE];
    uint32_t vmask = 0;
#pragma unroll
    for (int g = 0; g < kFinalE / 4; ++g) {
      const int k0 = 4 * (g * kFinalThreads + t);
      if (direct) {
        const float* __restrict__ src = scores + row * cap;
        if (k0 + 4 <= M) {
          const float4 x = *reinterpret_cast<const float4*>(src + k0);
          const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[4 * g + e] = composite(score_key(v[e]), (uint32_t)(k0 + e));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cv[4 * g + e] = (k0 + e < M) ? composite(score_key(src[k0 + e]), (uint32_t)(k0 + e)) : 0ull;
        }
      } else {
        const uint64_t* __restrict__ src = cand + row * cand_stride;
        if (k0 + 4 <= M) {
          const ulonglong2 a = *reinterpret_cast<const ulonglong2*>(src + k0);
          const ulonglong2 c2 = *reinterpret_cast<const ulonglong2*>(src + k0 + 2);
          cv[4 * g] = a.x;
          cv[4 * g + 1] = a.y;
          cv[4 * g + 2] = c2.x;
          cv[4 * g + 3] = c2.y;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) cv[4 * g + e] = (k0 + e < M) ? src[k0 + e] : 0ull;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) vmask |= (k0 + e < M ? 1u : 0u) << (4 * g + e);
    }
    const uint64_t tau = reg_select<kFinalThreads, kFinalE>(cv, vmask, (uint32_t)budget, L.s);
    uint32_t m4[kFinalE / 4], off[kFinalE / 4];
#pragma unroll
    for (int g = 0; g < kFinalE / 4; ++g) {
      m4[g] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m4[g] |= ((((vmask >> (4 * g + e)) & 1u) && cv[4 * g + e] >= tau) ? 1u : 0u) << e;
    }
    ordered_offsets<kFinalThreads>(m4, off, L.s);
#pragma unroll
    for (int g = 0; g < kFinalE / 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((m4[g] >> e) & 1u) {
          if (off[g] < (uint32_t)budget) {
            const int pos = (int)composite_pos(cv[4 * g + e]);
            if (o) o[off[g]] = pos;
            if (ATTEND) L.sel[off[g]] = pos;
          }
          ++off[g];
        }
  }
  if constexpr (ATTEND) {
    __syncthreads();
    float* out_row = out + row * D;
    if (take == 0) {
      for (int d = t; d < D; d += kFinalThreads) out_row[d] = 0.0f;
      return;
    }
    const size_t kvbase = ((size_t)b * hkv + h / G) * cap;
    attend_rows<BF16, D, kFinalThreads / kWave>(L.sel, take, k_cache, v_cache, qrot, row, kvbase,
                                                out_row, reinterpret_cast<float*>(&L.s.hist[0][0]));
  }
}

bool two_stage_applies(int max_seq_len, int budget) {
  const int nch = (max_seq_len + kTwoStageChunk - 1) / kTwoStageChunk;
  return budget <= kFusedMaxBudget && 2 * budget <= kTwoStageChunk &&
         (long long)nch * budget <= kTwoStageMaxCand && max_seq_len > 0;
}

template <bool ATT, bool BF, int DD>
static void launch_final(const fasa_ctx* c, hipStream_t s, const float* scores, const int32_t* nb,
                         int max_seq_len, int budget, const uint64_t* cand, int stride,
                         int32_t* idx, const void* k, const void* v, const float* qrot, float* out,
                         int32_t* advance, uint32_t* err) {
  hipLaunchKernelGGL((final_select_kernel<ATT, BF, DD>), dim3((unsigned)c->hq, (unsigned)c->batch),
                     dim3(kFinalThreads), 0, s, scores, nb, max_seq_len, c->hq, c->cap, budget,
                     cand, stride, idx, k, v, qrot, c->hkv, c->G, out, advance, err);
}

hipError_t launch_two_stage(const fasa_ctx* c, const float* scores, const int32_t* nb,
                            int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                            const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                            hipStream_t s) {
  if (!two_stage_applies(max_seq_len, budget)) return hipErrorInvalidValue;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + c->ws.cand);
  const int stride = c->ws.cand_stride;
  const int nch = (max_seq_len + kTwoStageChunk - 1) / kTwoStageChunk;
  if (nch > 1)
    hipLaunchKernelGGL(chunk_select_kernel, dim3((unsigned)nch, (unsigned)c->hq, (unsigned)c->batch),
                       dim3(kChunkThreads), 0, s, scores, nb, max_seq_len, c->hq, c->cap, budget,
                       cand, stride);
  if (out == nullptr) {
    launch_final<false, true, 128>(c, s, scores, nb, max_seq_len, budget, cand, stride, idx,
                                   nullptr, nullptr, nullptr, nullptr, advance, err);
    return hipGetLastError();
  }
  const bool bf = (c->dtype == FASA_BF16);
  if (c->d == 128) {
    if (bf) launch_final<true, true, 128>(c, s, scores, nb, max_seq_len, budget, cand, stride, idx, k_cache, v_cache, qrot, out, advance, err);
    else launch_final<true, false, 128>(c, s, scores, nb, max_seq_len, budget, cand, stride, idx, k_cache, v_cache, qrot, out, advance, err);
  } else {
    if (bf) launch_final<true, true, 64>(c, s, scores, nb, max_seq_len, budget, cand, stride, idx, k_cache, v_cache, qrot, out, advance, err);
    else launch_final<true, false, 64>(c, s, scores, nb, max_seq_len, budget, cand, stride, idx, k_cache, v_cache, qrot, out, advance, err);
  }
  return hipGetLastError();
}

}  // namespace fasa
