// Top-B selection of the critical token set, fused with FAC when B is small.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC bullets: select the critical token set T_t from the TIP
// scores, then run full attention over T_t only.  Selection: the min(B, n)
// highest scores of each (sequence, query head) row, equal scores to the
// lower position, listed ascending; exact, by range refinement over 64-bit
// composites (select_common.hpp).
//
// A row of up to 8192 positions is held whole in the registers of one
// 512-thread workgroup (up to 16384, in 1024 threads, when chunking cannot
// reduce it; up to 40960, 32 or 40 per thread in 1024 threads, when B is
// past the fused limit and chunks would not cut the row much), loaded in one round of coalesced loads, selected there, and,
// for B <= 1024, attended in the same workgroup: one launch after TIP.  No workgroup ever waits on another
// (device-wide hand-offs are expensive on a multi-die GPU).
//
// Longer rows are cut into chunks: chunk_select_kernel writes each chunk's
// own top-B composites (the row's top B are among them), and
// row_select_kernel then selects among those candidates (at most 16384).

#include "attention_common.hpp"
#include "budget.hpp"
#include "fasa_internal.hpp"
#include "select_common.hpp"
#include "select_src.hpp"

namespace fasa {

// 8 waves (2 per SIMD) with up to 32 elements each: every wave repeats the
// fixed work of a pass (scans, picks), so fewer waves with more elements
// finish a pass sooner than 16 waves with fewer, and 2 waves per SIMD leave
// 256 VGPRs each, enough to hold 32 keys or composites without spilling.
constexpr int kRowThreads = 512;
// Workgroup size of the selects that hold 16384 scores (the longest chunk,
// the most candidates): 16 per thread rather than 32, in 1024 threads.
constexpr int kWideThreads = 1024;
constexpr int kMaxE = 32;  // scores per thread, at most (chunk and candidate selects)
// Scores per thread, at most, of a whole row in kWideThreads when B is past
// the fused limit (no FAC in the workgroup, so the registers go to scores).
constexpr int kWideMaxE = 40;
static_assert(kWideMaxE / 4 <= kMaxSlabs, "slab table");
static_assert(kSelectChunk == kRowThreads * kMaxE, "the longest chunk is one workgroup's registers");
static_assert(kTwoStageMaxCand <= kRowThreads * kMaxE, "candidates fit one workgroup");
constexpr int kHistCopiesSel = 4;
constexpr int kCandCapSel = 4096;

template <int NT>
using SelLds = RegSelectLds<NT, kHistCopiesSel, kCandCapSel>;

// LDS the fused FAC needs for its state merge (attend_rows), worst case over
// the head sizes and dtypes built (bf16, d = 64: 128 states of 64 dims).
constexpr int kAttendScratch = 9728;

template <int NT>
struct RowLds {
  union {
    SelLds<NT> s;
    float att[kAttendScratch];
  };
  int32_t sel[kFusedMaxBudget];
};

// Candidates the chunk stage leaves for a row of n positions in chunks of
// `chunk`: min(B, chunk) per full chunk, min(B, rest) for the last.
__device__ __forceinline__ int candidates_of(int n, int budget, int chunk) {
  const int nch = (n + chunk - 1) / chunk;
  const int last = n - (nch - 1) * chunk;
  return (nch - 1) * (budget < chunk ? budget : chunk) + (last < budget ? last : budget);
}

// Stage 1 for rows of several chunks (E * 1024 positions each): the chunk's
// own top-B composites, ascending, at cand[row][chunk * min(B, chunk) ...],
// B the row's budget (see row_budget).  The row's top B are among them.
template <int E, int NT>
__global__ void __launch_bounds__(NT)
chunk_select_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                    int max_seq_len, int hq, int cap, int budget,
                    const int32_t* __restrict__ head_budget, uint64_t* __restrict__ cand,
                    int cand_stride) {
  constexpr int kChunk = E * NT;
  __shared__ RegSelectLds<NT, kHistCopiesSel, kCandCapSel> L;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  const int c0 = chunk * kChunk;
  // The chunk's loads go out before n_b arrives (bounded by the launch's
  // longest row; the grid holds no chunk past it).
  RawScores<E> raw;
  issue_scores<E, NT>(raw, scores + row * cap, c0, min(kChunk, min(max_seq_len, cap) - c0));
  int n = nb[b];
  if (n < 0 || n > max_seq_len || n > cap) n = 0;
  const int nch = (n + kChunk - 1) / kChunk;
  budget = row_budget(head_budget, h, budget, nullptr, false);
  // Rows the second stage takes whole (n <= B, or B = 0) need no candidates;
  // a one-chunk row is a chunk too.
  if (budget == 0 || n <= budget || chunk >= nch) return;
  const int cn = min(kChunk, n - c0);
  ScoreSrc<E, NT> src;
  scores_to_keys<E, NT>(src, raw, c0, cn);
  // A short last chunk keeps all its positions (need = cn selects them all).
  const uint32_t need = (uint32_t)(cn > budget ? budget : cn);
  const uint64_t tau = adaptive_select<NT, E>(src, need, L);
  const int per = budget < kChunk ? budget : kChunk;
  uint64_t* out = cand + row * cand_stride + (size_t)chunk * per;
  emit_ordered<E, NT>(src, tau, (uint32_t)per, L, [&](uint32_t r, int e) {
    out[r] = ((uint64_t)src.key(e) << 32) | src.low(e);
  });
}

// Selects a row's top B from its raw scores (FROM_CAND = false, n <= E * NT)
// or from the chunk stage's candidates (FROM_CAND = true, chunks of `chunk`
// positions, at most E * NT candidates), writes idx
// (if given) and, with ATTEND, runs FAC over the selection in LDS.  B is the
// row's budget (row_budget); idx rows are `budget` wide, -1 past the set.
// Also stores n_b into advance[b] (if given): seq_lens may be advanced here
// since no kernel of this launch reads it.
//
// With S > 1 (ATTEND only) every row runs on S workgroups (grid x = S * hq;
// part x / hq, head x % hq, so with hq a multiple of 8 a head's parts share an
// XCD and its K rows come from that XCD's L2).  Each part makes the same
// selection and attends over it for D / S output columns (attend_rows_split);
// part 0 alone writes idx, advance and flags.
template <bool ATTEND, bool BF16, int D, int E, bool FROM_CAND, int NT, int S = 1>
__global__ void __launch_bounds__(NT)
row_select_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                  int max_seq_len, int hq, int cap, int budget,
                  const int32_t* __restrict__ head_budget,
                  const uint64_t* __restrict__ cand, int cand_stride, int chunk,
                  int32_t* __restrict__ idx, const void* __restrict__ k_cache,
                  const void* __restrict__ v_cache, const float* __restrict__ qrot, int hkv,
                  int G, float* __restrict__ out, int32_t* __restrict__ advance, uint32_t* err) {
  static_assert(NT / kWave * RowGeom<BF16, D>::RS * (D + 3) + 1 + NT <=
                    kAttendScratch,
                "attend_rows scratch");
  static_assert(S == 1 || ATTEND, "column split is for the fused FAC");
  __shared__ RowLds<NT> L;
  const int part = S > 1 ? (int)blockIdx.x / hq : 0;
  const int h = S > 1 ? (int)blockIdx.x % hq : (int)blockIdx.x, b = blockIdx.y;
  const bool lead = part == 0;
  const size_t row = (size_t)b * hq + h;
  // The row's scores (or candidates) go out before n_b arrives; what lies
  // past the row's own length is masked once it is known.
  RawScores<FROM_CAND ? 4 : E> raw_s;
  RawCands<FROM_CAND ? E : 4> raw_c;
  if constexpr (FROM_CAND)
    issue_cands<E, NT>(raw_c, cand + row * cand_stride, cand_stride);
  else
    issue_scores<E, NT>(raw_s, scores + row * cap, 0, min(E * NT, min(max_seq_len, cap)));
  const int n = checked_len(nb, b, max_seq_len, cap, err, lead && h == 0 && threadIdx.x == 0);
  if (advance != nullptr && lead && h == 0 && threadIdx.x == 0 && n > 0) advance[b] = n;
  const int t = threadIdx.x;
  int32_t* o = (idx && lead) ? idx + row * budget : nullptr;
  const int bh = row_budget(head_budget, h, budget, err, lead && b == 0 && t == 0);
  const int take = n < bh ? n : bh;
  const bool whole = n <= bh || bh == 0;  // every position, or none

  if (whole) {
    for (int j = t; j < budget; j += NT) {
      if (o) o[j] = (j < take) ? j : -1;
      if (ATTEND && j < kFusedMaxBudget) L.sel[j] = j;
    }
  } else if constexpr (!FROM_CAND) {
    ScoreSrc<E, NT> src;
    scores_to_keys<E, NT>(src, raw_s, 0, n);
    const uint64_t tau = adaptive_select<NT, E>(src, (uint32_t)bh, L.s);
    emit_ordered<E, NT>(src, tau, (uint32_t)bh, L.s, [&](uint32_t r, int e) {
      const int pos = src.pos(e);
      if (o) o[r] = pos;
      if (ATTEND) L.sel[r] = pos;
    });
  } else {
    CandSrc<E, NT> src;
    cands_to_src<E, NT>(src, raw_c, candidates_of(n, bh, chunk));
    const uint64_t tau = adaptive_select<NT, E>(src, (uint32_t)bh, L.s);
    emit_ordered<E, NT>(src, tau, (uint32_t)bh, L.s, [&](uint32_t r, int e) {
      const int pos = (int)(0xffffffffu - src.lo[e]);
      if (o) o[r] = pos;
      if (ATTEND) L.sel[r] = pos;
    });
  }
  if (!whole && o != nullptr)
    for (int j = bh + t; j < budget; j += NT) o[j] = -1;
  if constexpr (ATTEND) {
    __syncthreads();
    float* out_row = out + row * D;
    if (take == 0) {
      if (lead)
        for (int d = t; d < D; d += NT) out_row[d] = 0.0f;
      return;
    }
    const size_t kvbase = ((size_t)b * hkv + h / G) * cap;
    if constexpr (S > 1)
      attend_rows_split<BF16, D, NT / kWave, S>(L.sel, take, k_cache, v_cache, qrot, row,
                                                kvbase, part, out_row, L.att);
    else
      attend_rows<BF16, D, NT / kWave>(L.sel, take, k_cache, v_cache, qrot, row, kvbase,
                                       out_row, L.att);
  }
}

// How a (max_seq_len, budget) pair is selected: a row held whole by one
// workgroup (direct_e scores per thread), or chunks of chunk_e * 1024
// positions and then their candidates (cand_e per thread).
struct SelectPlan {
  int direct_e = 0, chunk_e = 0, cand_e = 0;
  int wide_e = 0;  // whole row, wide_e per thread in kWideThreads (no FAC)
  bool ok() const { return direct_e || chunk_e || wide_e; }
};

static int round_e(int per_thread) {
  return per_thread <= 4 ? 4 : per_thread <= 8 ? 8 : per_thread <= 16 ? 16 : 32;
}

// Short rows go whole to one workgroup (one launch).  Longer rows are cut
// into the shortest chunks (4096 positions and up) whose chunk is longer than
// B and that leave at most 8192 candidates, else at most 16384: more
// workgroups with fewer scores each finish sooner than one workgroup per row,
// but the second stage is one workgroup per row, so halving its candidates
// is worth longer chunks.  When B is past the fused limit and chunking would
// leave the second stage more than a quarter of the row (or cannot be
// planned), the row goes whole to one 1024-thread workgroup instead: 16 per
// thread up to 16384 positions, 32 or 40 per thread up to 40960.  That stage
// would redo most of the first one's work, one workgroup per row anyway.
// Other rows where no chunk reduces anything but that fit one workgroup are
// held whole.
static SelectPlan select_plan(int max_seq_len, int budget) {
  SelectPlan p;
  if (max_seq_len <= 0 || budget < 1) return p;
  if (max_seq_len <= 16 * kRowThreads) {
    p.direct_e = round_e((max_seq_len + kRowThreads - 1) / kRowThreads);
    return p;
  }
  long long cands = 0;
  for (const long long cap : {(long long)kTwoStageMaxCand / 2, (long long)kTwoStageMaxCand}) {
    for (int e = 8; e <= kMaxE && !p.chunk_e; e *= 2) {
      const long long chunk = (long long)e * kRowThreads;
      const long long nch = (max_seq_len + chunk - 1) / chunk;
      const long long last = max_seq_len - (nch - 1) * chunk;
      // Candidates of the longest row (no row of the launch has more).
      const long long c = (nch - 1) * budget + (last < budget ? last : budget);
      if (nch > 1 && budget < chunk && c <= cap) {
        p.chunk_e = e;
        p.cand_e = round_e((int)((c + kRowThreads - 1) / kRowThreads));
        cands = c;
      }
    }
    if (p.chunk_e) break;
  }
  if (budget > kFusedMaxBudget && max_seq_len <= kWideMaxE * kWideThreads &&
      (!p.chunk_e || 4 * cands > max_seq_len)) {
    SelectPlan w;
    if (max_seq_len <= kMaxE * kRowThreads)
      w.direct_e = round_e((max_seq_len + kRowThreads - 1) / kRowThreads);  // 1024 x 16
    else
      w.wide_e = max_seq_len <= 32 * kWideThreads ? 32 : kWideMaxE;
    return w;
  }
  if (!p.chunk_e && max_seq_len <= kMaxE * kRowThreads)
    p.direct_e = round_e((max_seq_len + kRowThreads - 1) / kRowThreads);
  return p;
}

bool select_path_applies(int max_seq_len, int budget) {
  return select_plan(max_seq_len, budget).ok();
}

SelectLayout select_layout(int max_seq_len, int budget) {
  const SelectPlan p = select_plan(max_seq_len, budget);
  SelectLayout l;
  if (p.wide_e) {
    l.kind = 3;
    l.threads = kWideThreads;
    l.per_thread = p.wide_e;
  } else if (p.direct_e) {
    // Elements past 16 per thread go to the 1024-thread build (16 each).
    l.kind = 1;
    l.threads = p.direct_e > 16 ? kWideThreads : kRowThreads;
    l.per_thread = p.direct_e > 16 ? 16 : p.direct_e;
  } else if (p.chunk_e) {
    l.kind = 2;
    l.chunk = p.chunk_e * kRowThreads;
    l.threads = p.cand_e > 16 ? kWideThreads : kRowThreads;  // the candidate stage
    l.per_thread = p.cand_e > 16 ? 16 : p.cand_e;
  } else {
    l.kind = 4;
  }
  return l;
}

template <bool ATT, bool BF, int DD, int E, bool FC, int NT, int S = 1>
static void launch_row(const fasa_ctx* c, hipStream_t s, const float* scores, const int32_t* nb,
                       int max_seq_len, int budget, const int32_t* hb, const uint64_t* cand,
                       int stride, int chunk, int32_t* idx, const void* k, const void* v,
                       const float* qrot, float* out, int32_t* advance, uint32_t* err) {
  hipLaunchKernelGGL((row_select_kernel<ATT, BF, DD, E, FC, NT, S>),
                     dim3((unsigned)(c->hq * S), (unsigned)c->batch), dim3(NT), 0, s, scores,
                     nb, max_seq_len, c->hq, c->cap, budget, hb, cand, stride, chunk, idx, k, v,
                     qrot, c->hkv, c->G, out, advance, err);
}

// Column parts of the fused FAC when the rows are few: with S workgroups per
// row the selection is made S times over, in parallel on otherwise idle CUs,
// and each part attends for D / S output columns.
constexpr int kFacColumnParts = 4;

template <int E, bool FC, int NT = kRowThreads>
static void launch_row_e(const fasa_ctx* c, hipStream_t s, const float* scores,
                         const int32_t* nb, int max_seq_len, int budget, const int32_t* hb,
                         const uint64_t* cand, int stride, int chunk, int32_t* idx,
                         const void* k, const void* v, const float* qrot, float* out,
                         int32_t* advance, uint32_t* err) {
  if (out == nullptr) {
    launch_row<false, true, 128, E, FC, NT>(c, s, scores, nb, max_seq_len, budget, hb, cand, stride,
                                        chunk, idx, nullptr, nullptr, nullptr, nullptr, advance,
                                        err);
    return;
  }
  const bool bf = (c->dtype == FASA_BF16);
  // Split when every part of every row still has a CU of its own.
  const bool split = (long long)c->batch * c->hq * kFacColumnParts <= c->cus;
#define FASA_ROW(BFV, DV)                                                                       \
  do {                                                                                          \
    if (split)                                                                                  \
      launch_row<true, BFV, DV, E, FC, NT, kFacColumnParts>(c, s, scores, nb, max_seq_len,       \
                                                            budget, hb, cand, stride, chunk,    \
                                                            idx, k, v, qrot, out, advance, err); \
    else                                                                                        \
      launch_row<true, BFV, DV, E, FC, NT>(c, s, scores, nb, max_seq_len, budget, hb, cand,     \
                                           stride, chunk, idx, k, v, qrot, out, advance, err);  \
  } while (0)
  if (c->d == 128) {
    if (bf) FASA_ROW(true, 128); else FASA_ROW(false, 128);
  } else {
    if (bf) FASA_ROW(true, 64); else FASA_ROW(false, 64);
  }
#undef FASA_ROW
}

hipError_t launch_select(const fasa_ctx* c, const float* scores, const int32_t* nb,
                         int max_seq_len, int budget, int32_t* idx, const void* k_cache,
                         const void* v_cache, float* out, int32_t* advance, uint8_t* ws,
                         hipStream_t s, const int32_t* head_budget) {
  const SelectPlan p = select_plan(max_seq_len, budget);
  if (!p.ok() || (out != nullptr && budget > kFusedMaxBudget)) return hipErrorInvalidValue;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  const float* qrot = reinterpret_cast<const float*>(ws + c->ws.qrot);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + c->ws.cand);
  const int stride = c->ws.cand_stride;
#define FASA_ROWE(EV, FC, CH)                                                                  \
  launch_row_e<EV, FC>(c, s, scores, nb, max_seq_len, budget, head_budget, cand, stride, CH,  \
                       idx, k_cache, v_cache, qrot, out, advance, err)
#define FASA_ROWW(FC, CH)                                                                      \
  launch_row_e<16, FC, kWideThreads>(c, s, scores, nb, max_seq_len, budget, head_budget, cand, \
                                     stride, CH, idx, k_cache, v_cache, qrot, out, advance, err)
  if (p.wide_e) {
#define FASA_WIDE(EV)                                                                          \
  launch_row<false, true, 128, EV, false, kWideThreads>(c, s, scores, nb, max_seq_len, budget, \
                                                        head_budget, cand, stride, 0, idx,     \
                                                        nullptr, nullptr, nullptr, nullptr,    \
                                                        advance, err)
    if (p.wide_e == 32) FASA_WIDE(32); else FASA_WIDE(kWideMaxE);
#undef FASA_WIDE
    return hipGetLastError();
  }
  if (p.direct_e) {
    switch (p.direct_e) {
      case 4: FASA_ROWE(4, false, 0); break;
      case 8: FASA_ROWE(8, false, 0); break;
      case 16: FASA_ROWE(16, false, 0); break;
      default: FASA_ROWW(false, 0); break;
    }
    return hipGetLastError();
  }
  const int chunk = p.chunk_e * kRowThreads;
  const dim3 grid((unsigned)((max_seq_len + chunk - 1) / chunk), (unsigned)c->hq,
                  (unsigned)c->batch);
#define FASA_CHUNK(EV)                                                                        \
  hipLaunchKernelGGL((chunk_select_kernel<EV, kRowThreads>), grid, dim3(kRowThreads), 0, s,    \
                     scores, nb,                                                              \
                     max_seq_len, c->hq, c->cap, budget, head_budget, cand, stride)
  switch (p.chunk_e) {
    case 8: FASA_CHUNK(8); break;
    case 16: FASA_CHUNK(16); break;
    default:
      hipLaunchKernelGGL((chunk_select_kernel<16, kWideThreads>), grid, dim3(kWideThreads), 0, s,
                         scores, nb, max_seq_len, c->hq, c->cap, budget, head_budget, cand,
                         stride);
      break;
  }
  if (p.cand_e <= 4) FASA_ROWE(4, true, chunk);
  else if (p.cand_e <= 8) FASA_ROWE(8, true, chunk);
  else if (p.cand_e <= 16) FASA_ROWE(16, true, chunk);
  else FASA_ROWW(true, chunk);
#undef FASA_CHUNK
#undef FASA_ROWE
#undef FASA_ROWW
  return hipGetLastError();
}

}  // namespace fasa
