// Per-head top-B selection of the critical token set T_t.
//
// "FASA: Frequency-aware Sparse Attention", gist.science/pt, "Resumo Tecnico"
// section 2, FAC first bullet: from the TIP scores a critical subset of tokens
// is selected.  Here: the min(B, n) highest scores of each (sequence, query
// head) row, equal scores going to the lower position, listed ascending.
//
// Exact radix select on 64-bit composites (order-preserving 32-bit key of the
// fp32 score, then the inverted position), which are all distinct, so the
// B-th largest composite tau splits the row: selected <=> composite >= tau.
// Three kernels, each over chunks of 4096 scores (enough workgroups to fill
// the chip even for a single long row):
//   1. hist:  LDS histogram of the top 11 key bits per chunk, summed into a
//             row histogram with device atomics; the last chunk to finish
//             finds the digit holding the B-th largest and how many of that
//             bin are still needed.
//   2. cand:  counts each chunk's tokens above that digit and gathers the
//             bin's tokens as composites; the last chunk resolves tau with
//             further radix passes over the (small) candidate list, then
//             turns per-chunk counts into output offsets.
//   3. emit:  each chunk compacts its selected positions, in order, to its
//             offset: the output is ascending without a sort.
// Rows with n <= B take every position and are padded with -1.

#include "device_common.hpp"
#include "fasa_internal.hpp"

namespace fasa {

// Loads the kPerThread consecutive scores of this thread (positions j0 ..)
// as keys; positions >= n get key 0 and valid = false.
__device__ __forceinline__ void load_keys(const float* __restrict__ src, int j0, int n,
                                          uint32_t (&key)[kPerThread]) {
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    const int j = j0 + 4 * k;
    if (j + 3 < n) {
      const float4 v = *reinterpret_cast<const float4*>(src + j);
      key[4 * k + 0] = score_key(v.x);
      key[4 * k + 1] = score_key(v.y);
      key[4 * k + 2] = score_key(v.z);
      key[4 * k + 3] = score_key(v.w);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * k + e] = (j + e < n) ? score_key(src[j + e]) : 0u;
    }
  }
}

// Scans a histogram of `bins` counts (LDS) from the top bin down and finds the
// bin where the running count reaches `need`.  256 threads.  Returns, in every
// thread, the bin, the count above it and the bin's own count.
struct BinPick {
  uint32_t bin, above, count;
};
__device__ __forceinline__ BinPick pick_bin_from_top(const uint32_t* hist, int bins,
                                                     uint32_t need, uint32_t* scan_lds,
                                                     uint32_t* pick_lds) {
  const int per = (bins + 255) / 256;  // bins per thread (1..8)
  uint32_t cnt[8];
  uint32_t local = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int rank = threadIdx.x * per + e;  // rank 0 = top bin
    cnt[e] = (e < per && rank < bins) ? hist[bins - 1 - rank] : 0u;
    local += cnt[e];
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan<256>(local, scan_lds, &total);
  if (before < need && need <= before + local) {
    uint32_t acc = before;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < per && acc < need && need <= acc + cnt[e]) {
        pick_lds[0] = (uint32_t)(bins - 1 - (threadIdx.x * per + e));
        pick_lds[1] = acc;
        pick_lds[2] = cnt[e];
      }
      acc += cnt[e];
    }
  }
  __syncthreads();
  BinPick p{pick_lds[0], pick_lds[1], pick_lds[2]};
  __syncthreads();
  return p;
}

__global__ void __launch_bounds__(256)
topk_hist_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                 int max_seq_len, int hq, int cap, int budget, uint32_t* __restrict__ ghist,
                 uint32_t* __restrict__ tickets, RowState* __restrict__ rowst, uint32_t* err) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan_lds[4];
  __shared__ uint32_t pick_lds[4];
  __shared__ uint32_t flag;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  const int n = checked_len(nb, b, max_seq_len, cap, err, chunk == 0 && h == 0 && threadIdx.x == 0);
  if (n <= budget) return;
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (chunk >= nchunks) return;

  for (int i = threadIdx.x; i < kHistBins; i += 256) hist[i] = 0u;
  __syncthreads();
  uint32_t key[kPerThread];
  const int j0 = chunk * kChunk + threadIdx.x * kPerThread;
  load_keys(scores + row * cap, j0, n, key);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (j0 + e < n) atomicAdd(&hist[key[e] >> (32 - kHistBits)], 1u);
  __syncthreads();
  uint32_t* gh = ghist + row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t c = hist[i];
    if (c) atomic_add_agent(&gh[i], c);
  }
  if (!last_block_arrives(&tickets[row * kTicketsPerRow + 0], (uint32_t)nchunks, &flag)) return;

  // Last chunk of the row: take the row histogram (and clear it for the next call).
  for (int i = threadIdx.x; i < kHistBins; i += 256) hist[i] = atomic_xchg_agent(&gh[i], 0u);
  __syncthreads();
  const BinPick p = pick_bin_from_top(hist, kHistBins, (uint32_t)budget, scan_lds, pick_lds);
  if (threadIdx.x == 0) {
    rowst[row].digit1 = p.bin;
    rowst[row].need = (uint32_t)budget - p.above;
  }
}

__global__ void __launch_bounds__(256)
topk_cand_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                 int max_seq_len, int hq, int cap, int budget, int max_chunks,
                 uint32_t* __restrict__ tickets, RowState* __restrict__ rowst,
                 uint64_t* __restrict__ cand, uint32_t* __restrict__ chunk_gt,
                 uint32_t* __restrict__ chunk_off, uint32_t* err) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t chunk_cnt[kMaxChunks];
  __shared__ uint32_t scan_lds[4];
  __shared__ uint32_t pick_lds[4];
  __shared__ uint32_t flag;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  if (n <= budget) return;
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (chunk >= nchunks) return;
  const int lane = threadIdx.x & (kWave - 1);

  const uint32_t d1 = rowst[row].digit1;
  uint32_t key[kPerThread];
  const int j0 = chunk * kChunk + threadIdx.x * kPerThread;
  load_keys(scores + row * cap, j0, n, key);
  uint64_t* cr = cand + row * cap;
  uint32_t gt = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t dg = key[e] >> (32 - kHistBits);
    const bool valid = (j0 + e < n);
    gt += (valid && dg > d1) ? 1u : 0u;
    const bool is_c = valid && dg == d1;
    const uint64_t m = __ballot(is_c);
    if (m) {
      const int first = __builtin_ctzll(m);
      uint32_t base = 0;
      if (lane == first) base = atomic_add_agent(&rowst[row].cand_count, (uint32_t)__popcll(m));
      base = __shfl(base, first);
      const uint32_t rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
      if (is_c && base + rank < (uint32_t)n) cr[base + rank] = composite(key[e], (uint32_t)(j0 + e));
    }
  }
  uint32_t total;
  block_exclusive_scan<256>(gt, scan_lds, &total);
  if (threadIdx.x == 0) chunk_gt[row * max_chunks + chunk] = total;
  if (!last_block_arrives(&tickets[row * kTicketsPerRow + 1], (uint32_t)nchunks, &flag)) return;

  // Last chunk of the row: resolve tau among the M candidates of digit d1.
  uint32_t M = atomic_load_agent(&rowst[row].cand_count);
  if (M > (uint32_t)n) M = (uint32_t)n;  // never read past the row's candidates
  uint32_t need = rowst[row].need;
  uint64_t prefix = d1;
  int known = kHistBits;
  while (known < 64) {
    const int width = (64 - known < kHistBits) ? (64 - known) : kHistBits;
    const int shift = 64 - known - width;
    const int bins = 1 << width;
    for (int i = threadIdx.x; i < bins; i += 256) hist[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < M; i += 256) {
      const uint64_t cv = cr[i];
      if ((cv >> (64 - known)) == prefix)
        atomicAdd(&hist[(uint32_t)(cv >> shift) & (uint32_t)(bins - 1)], 1u);
    }
    __syncthreads();
    const BinPick p = pick_bin_from_top(hist, bins, need, scan_lds, pick_lds);
    prefix = (prefix << width) | p.bin;
    known += width;
    need -= p.above;
    if (p.count == need) break;  // the whole bin is taken
  }
  const uint64_t tau = (known >= 64) ? prefix : (prefix << (64 - known));

  for (int i = threadIdx.x; i < nchunks; i += 256) chunk_cnt[i] = 0u;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < M; i += 256) {
    const uint64_t cv = cr[i];
    const uint32_t pos = composite_pos(cv);
    if (cv >= tau && pos < (uint32_t)n) atomicAdd(&chunk_cnt[pos / kChunk], 1u);
  }
  __syncthreads();
  // Exclusive scan over chunks of (above-digit count + selected candidates).
  constexpr int kPer = kMaxChunks / 256;
  uint32_t v[kPer];
  uint32_t local = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int ck = threadIdx.x * kPer + e;
    v[e] = (ck < nchunks) ? chunk_gt[row * max_chunks + ck] + chunk_cnt[ck] : 0u;
    local += v[e];
  }
  uint32_t all;
  uint32_t off = block_exclusive_scan<256>(local, scan_lds, &all);
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int ck = threadIdx.x * kPer + e;
    if (ck < nchunks) chunk_off[row * max_chunks + ck] = off;
    off += v[e];
  }
  if (threadIdx.x == 0) {
    rowst[row].tau = tau;
    atomic_store_agent(&rowst[row].cand_count, 0u);
  }
}

__global__ void __launch_bounds__(256)
topk_emit_kernel(const float* __restrict__ scores, const int32_t* __restrict__ nb,
                 int max_seq_len, int hq, int cap, int budget, int max_chunks,
                 const RowState* __restrict__ rowst, const uint32_t* __restrict__ chunk_off,
                 int32_t* __restrict__ idx, uint32_t* err) {
  __shared__ uint32_t scan_lds[4];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * hq + h;
  const int n = checked_len(nb, b, max_seq_len, cap, err, false);
  int32_t* out = idx + row * budget;
  const int j0 = chunk * kChunk + threadIdx.x * kPerThread;
  if (n <= budget) {
    if (chunk == 0)
      for (int j = n + threadIdx.x; j < budget; j += 256) out[j] = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (j0 + e < n) out[j0 + e] = j0 + e;
    return;
  }
  const int nchunks = (n + kChunk - 1) / kChunk;
  if (chunk >= nchunks) return;
  const uint64_t tau = rowst[row].tau;
  uint32_t key[kPerThread];
  load_keys(scores + row * cap, j0, n, key);
  uint32_t sel = 0, cnt = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool s = (j0 + e < n) && composite(key[e], (uint32_t)(j0 + e)) >= tau;
    sel |= (s ? 1u : 0u) << e;
    cnt += s ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = chunk_off[row * max_chunks + chunk] + block_exclusive_scan<256>(cnt, scan_lds, &total);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if ((sel & (1u << e)) && pos < (uint32_t)budget) out[pos++] = j0 + e;
}

hipError_t launch_topk(const fasa_ctx* c, const float* scores, const int32_t* nb,
                       int max_seq_len, int budget, int32_t* idx, uint8_t* ws, hipStream_t s) {
  dim3 grid((unsigned)((max_seq_len + kChunk - 1) / kChunk), (unsigned)c->hq, (unsigned)c->batch);
  if (grid.x == 0) grid.x = 1;
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + c->ws.err);
  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + c->ws.hist);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws + c->ws.ticket);
  RowState* rowst = reinterpret_cast<RowState*>(ws + c->ws.rowst);
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + c->ws.cand);
  uint32_t* cgt = reinterpret_cast<uint32_t*>(ws + c->ws.chunk_gt);
  uint32_t* coff = reinterpret_cast<uint32_t*>(ws + c->ws.chunk_off);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(256), 0, s, scores, nb, max_seq_len, c->hq,
                     c->cap, budget, ghist, tickets, rowst, err);
  hipLaunchKernelGGL(topk_cand_kernel, grid, dim3(256), 0, s, scores, nb, max_seq_len, c->hq,
                     c->cap, budget, c->ws.max_chunks, tickets, rowst, cand, cgt, coff, err);
  hipLaunchKernelGGL(topk_emit_kernel, grid, dim3(256), 0, s, scores, nb, max_seq_len, c->hq,
                     c->cap, budget, c->ws.max_chunks, rowst, coff, idx, err);
  return hipGetLastError();
}

}  // namespace fasa
